/*
 * libpagedattn -- host KV-cache block manager: the allocator behind the
 * block tables and slot mappings that the decode entry points take.
 *
 * Rules (vLLM project manual, doramagic.ai/projects/vllm/manual):
 *   "KVCacheManager -- cache block management": the free blocks form a deque
 *   holding 0 .. num_blocks-1 at creation; a request of n tokens takes
 *   ceil(n / block_size) blocks from the front; freeing a request returns
 *   its blocks to the back, in the request's block order.
 *   "sharing mechanism": a block several requests map carries a reference
 *   count and goes back to the free deque only when that count reaches 0.
 *   "cache allocation strategy": a request that grows at run time past its
 *   last block gets one more block from the front.
 * Slot of token t of a request: table[t / block_size] * block_size +
 * t % block_size ("vLLM 2026 推理引擎全解" (chenxutan.com) §2.2).
 *
 * All state lives in host memory owned by the manager object; nothing here
 * touches a GPU.  A manager is not thread-safe: one thread at a time.
 * Status codes are those of pagedattn.h.
 */
#ifndef PAGEDATTN_BLOCKS_H
#define PAGEDATTN_BLOCKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

/* A manager over num_blocks blocks (1 .. INT32_MAX) of block_size tokens;
 * NULL for invalid sizes or when host memory runs out.  Destroy with
 * pa_bm_destroy (NULL is a no-op). */
pa_block_manager* pa_bm_create(int64_t num_blocks, int32_t block_size);
void pa_bm_destroy(pa_block_manager* m);

/* Give request `request_id` (a new id) ceil(num_tokens / block_size) blocks
 * from the front of the free deque; its length becomes num_tokens.
 * PA_ERR_EXHAUSTED (nothing taken) when fewer blocks are free; PA_ERR_RANGE
 * for an id that already holds blocks or num_tokens < 0. */
int pa_bm_allocate(pa_block_manager* m, int64_t request_id, int64_t num_tokens);

/* New request dst_id maps the first num_blocks blocks of src_id (one more
 * reference each); its length becomes num_blocks * block_size.  Only whole
 * blocks of the source may be shared (num_blocks * block_size <= its
 * length), so appends never write into a shared block.  PA_ERR_RANGE for an
 * unknown source, an existing destination or too many blocks. */
int pa_bm_share(pa_block_manager* m, int64_t src_id, int64_t dst_id, int64_t num_blocks);

/* New request dst_id maps every block of src_id (one more reference each)
 * and has its length: two continuations of one prompt (parallel sampling,
 * beam search).  PA_ERR_RANGE for an unknown source or existing
 * destination. */
int pa_bm_fork(pa_block_manager* m, int64_t src_id, int64_t dst_id);

/* Add one token to a request.  When its length is a multiple of block_size a
 * block is taken from the front first; when the token would land in a last
 * block that other requests still map, the request gets a fresh block from
 * the front in its place (copy-on-write): copy_pair receives (shared block,
 * fresh block), which the caller copies with pa_copy_blocks before writing
 * the token, else (-1, -1).  *slot receives the new token's slot (for
 * pa_reshape_and_cache).  PA_ERR_EXHAUSTED (nothing changed) when no block is
 * free; PA_ERR_RANGE for an unknown id. */
int pa_bm_append(pa_block_manager* m, int64_t request_id, int64_t* slot, int32_t* copy_pair);

/* pa_bm_append for each of n distinct requests in order, slots[i] for
 * request_ids[i] (host arrays); the copies it needs go to copy_pairs
 * ([n, 2] capacity, the first *num_copies filled), ready for
 * pa_copy_blocks.  All or nothing: PA_ERR_RANGE for an unknown or repeated
 * id, PA_ERR_EXHAUSTED when the batch needs more blocks than are free -- in
 * both cases no request changes. */
int pa_bm_append_batch(pa_block_manager* m, const int64_t* request_ids, int32_t n,
                       int64_t* slots, int32_t* copy_pairs, int32_t* num_copies);

/* Drop a request: one reference less on each of its blocks, blocks whose
 * count reaches 0 go to the back of the free deque in the request's block
 * order.  Unknown ids are ignored (PA_OK). */
int pa_bm_free(pa_block_manager* m, int64_t request_id);

/* Free blocks (-1 for NULL), a request's length (-1 when unknown). */
int64_t pa_bm_num_free(const pa_block_manager* m);
int64_t pa_bm_seq_len(const pa_block_manager* m, int64_t request_id);

/* Block tables and context lengths of num_seqs requests, in the layout the
 * decode entry points take: block_tables [num_seqs, max_blocks_per_seq]
 * int32 (entries past a request's blocks = pad), context_lens [num_seqs]
 * int32 (host pointers).  PA_ERR_RANGE (nothing written) for an unknown id,
 * a request with more blocks than max_blocks_per_seq or a length beyond
 * INT32_MAX. */
int pa_bm_block_tables(const pa_block_manager* m, const int64_t* request_ids, int32_t num_seqs,
                       int32_t max_blocks_per_seq, int32_t pad, int32_t* block_tables,
                       int32_t* context_lens);

/* The free deque, front first, into out[0 .. pa_bm_num_free - 1];
 * PA_ERR_SHAPE when capacity is smaller. */
int pa_bm_free_blocks(const pa_block_manager* m, int32_t* out, int64_t capacity);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_BLOCKS_H */
