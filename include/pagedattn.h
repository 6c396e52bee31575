/*
 * libpagedattn -- paged KV-cache decode attention for AMD Instinct MI355X
 * (gfx950).  Plain C ABI: pointers and sizes only.
 *
 * Pages defining the operations:
 *   [CX] "vLLM 2026 推理引擎全解：从 PagedAttention 到分离式 Prefill"
 *        (chenxutan.com/d/4119.html): §1.1 decode attention
 *        o_t = Attention(q_t, K_{1:t}, V_{1:t}) over cached K/V; §2.1 the
 *        cache cut into fixed 16-token pages found through a per-request page
 *        table, pages anywhere in memory and shareable between requests;
 *        §2.2 cache layout [num_pages, num_heads, page_size, head_dim] and
 *        the in-pool token address page_id * BLOCK_SIZE + page_offset;
 *        §2.3 requests sharing a prompt prefix map the same pages.
 *   [MJ] vLLM tutorial (mjmagnets.cn/news/49643), §2.2: the attention op
 *        gathers K and V blocks named by the block table, then computes.
 *   [DM] vLLM project manual (doramagic.ai/projects/vllm/manual), PagedAttention
 *        V1/V2 kernels: paged KV reads, wavefront-level reductions, fused
 *        kernel, wide vector loads; KV cache manager: reference-counted
 *        blocks shared between requests ("sharing mechanism").
 *
 * Common conventions
 *   - Element types (dtype): PA_F32, PA_F16 (IEEE binary16), PA_BF16.  q,
 *     key, value, the caches and out share one type; all arithmetic inside
 *     is float32.
 *   - Layouts (row-major, contiguous):
 *       q, out             [num_seqs, num_q_heads, head_dim]
 *       key, value         [num_tokens, num_kv_heads, head_dim]
 *       k_cache, v_cache   [num_blocks, num_kv_heads, block_size, head_dim]
 *       block_tables       [num_seqs, max_blocks_per_seq] int32
 *       context_lens       [num_seqs] int32
 *       slot_mapping       [num_tokens] int64
 *     Logical token t of sequence s lives in block block_tables[s][t / bs]
 *     at offset t % bs (bs = block_size: 16 by default, 8 or 32 also taken;
 *     [DM] block-size notes: 16 default, 8 and 32 as tuning choices).
 *     context_lens[s] counts every cached token, the one
 *     being decoded included.  Query head h reads KV head
 *     h / (num_q_heads / num_kv_heads).
 *   - Pointers are device pointers on the current HIP device, owned by the
 *     caller; the library allocates, frees and synchronises nothing.  Every
 *     call is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and returns before the work completes.  Calls keep no state.
 *   - Every argument a host can check is checked before anything is
 *     launched; a failed check returns its status and launches nothing.
 *     Device-side contents are not checked for validity, but the kernels
 *     never read or write outside the buffers the arguments describe:
 *     block ids outside [0, num_blocks) are skipped, context lengths are
 *     clamped to [0, min(max_context_len, 16 * max_blocks_per_seq)], and
 *     slots outside [0, 16 * num_blocks) are not written.
 *   - No C++ exception crosses this interface.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum pa_dtype { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2 };

enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = 2,       /* a size is out of range (num_seqs, num_q_heads and the
                             partition count are limited to 65535), or
                             num_q_heads % num_kv_heads != 0 */
  PA_ERR_UNSUPPORTED = 3, /* head_dim not 64/128, block_size not 8/16/32, unknown dtype,
                             partition_size not a positive multiple of 16 (or 0) */
  PA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than pa_decode_workspace_bytes
                             (pa_cascade_workspace_bytes for the cascade entry point) */
  PA_ERR_RANGE = 5,       /* host table check: an entry, length or slot out of range */
  PA_ERR_LAUNCH = 6,      /* the HIP runtime refused a launch */
  PA_ERR_EXHAUSTED = 7,   /* block manager (pagedattn_blocks.h): no free block left */
  PA_ERR_SCRATCH = 8      /* pa_reshape_and_decode_static: the partials need more than
                             PA_STATIC_SCRATCH_BYTES */
};

/*
 * KV write ([CX] §1.1: the new tokens' K and V are stored in the cache;
 * [CX] §2.2: token address = block * 16 + offset).  For each token i with
 * 0 <= slot = slot_mapping[i] < 16 * num_blocks:
 *     k_cache[slot / bs, h, slot % bs, :] = key[i, h, :]   for every h
 *     v_cache[slot / bs, h, slot % bs, :] = value[i, h, :]
 * A bit copy.  Negative slots mean "no write" (padding).  Two tokens with
 * the same slot leave either one's row in it (a caller error).
 * block_size (bs) 8, 16 or 32; head_dim 64 or 128.  num_tokens = 0 is a no-op.
 */
int pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                         const int64_t* slot_mapping, int32_t num_tokens,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int64_t num_blocks, int32_t dtype, void* stream);

/*
 * Decode attention over the paged cache ([CX] §1.1, §2.1-§2.2; [MJ] §2.2):
 * for every sequence s and query head h, with L = context_lens[s],
 * g = h / (num_q_heads / num_kv_heads), b_t = block_tables[s][t / bs]:
 *     z_t = scale * sum_d q[s,h,d] * k_cache[b_t, g, t % bs, d]
 *     out[s,h,:] = sum_{t<L} exp(z_t - max z) v_cache[b_t, g, t % bs, :]
 *                  / sum_{t<L} exp(z_t - max z)
 * rounded to nearest-even into out's type.  L = 0 gives a zero row.
 *
 * partition_size = 0 processes each sequence in one pass.  Otherwise it must
 * be a multiple of 16: each sequence is cut into ceil(L / partition_size)
 * partitions, processed in parallel, and sequences with more than one are
 * merged by the log-sum-exp reduce (pa_paged_attention_reduce), all on
 * `stream`.
 *
 * The partials live in `workspace` (device memory, caller-owned), which must
 * hold at least pa_decode_workspace_bytes(num_seqs, num_q_heads, head_dim,
 * max_context_len, partition_size) bytes (may be NULL when that is 0).  Calls
 * that share a workspace must not run concurrently.
 * max_context_len is a host-side bound on context_lens (sizes the grid);
 * longer contexts are clamped to it.  Tail slots of a sequence's last block
 * and blocks past ceil(L / bs) are never used, whatever they hold.
 * block_size 8 or 32 runs the workgroup-per-item kernels for every
 * partition count (the one-wave and streaming forms are 16-token only);
 * partition_size stays a multiple of 16 tokens.
 */
int pa_paged_attention_decode(void* out, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_tables,
                              const int32_t* context_lens, int32_t num_seqs,
                              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int32_t max_blocks_per_seq,
                              int64_t num_blocks, float scale, int32_t dtype,
                              int32_t partition_size, int32_t max_context_len,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode step in one call: the KV write of each sequence's new token
 * followed by decode attention ([CX] §1.1: the new token's K and V join the
 * cache, then o_t attends over K_{1:t}, V_{1:t} with token t included).
 * The result equals
 *     pa_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping,
 *                          num_seqs, ...);
 *     pa_paged_attention_decode(out, q, k_cache, v_cache, ...);
 * with one new token per sequence: key, value [num_seqs, num_kv_heads,
 * head_dim] (row s = sequence s's token), slot_mapping [num_seqs] int64
 * (negative or >= block_size * num_blocks: not written).  Every other
 * argument, the workspace rule and the errors are those of
 * pa_paged_attention_decode; key, value and slot_mapping must not be NULL
 * when num_seqs > 0.
 *
 * Precondition (the normal decode step, where slot_mapping[s] is the slot of
 * position context_lens[s] - 1 of sequence s's table): no context reads, in
 * this call, a slot written in this call other than its own last position.
 * The decode kernels then store each new row once and use it from registers
 * where a context ends with it, so no kernel waits for the write; when the
 * precondition does not hold the result is undefined (pa_validate_step_host
 * checks it on host copies of the step).  Every decode kernel does this,
 * the streaming one (16-token blocks, >= 8 partitions, <= 64 sequences,
 * grouped heads) included.
 */
int pa_reshape_and_decode(void* out, const void* q, const void* key, const void* value,
                          void* k_cache, void* v_cache, const int64_t* slot_mapping,
                          const int32_t* block_tables, const int32_t* context_lens,
                          int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                          int64_t num_blocks, float scale, int32_t dtype, int32_t partition_size,
                          int32_t max_context_len, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the step
 * of pa_reshape_and_decode with no workspace argument.  Its split-K partials
 * live in a device array the library owns, PA_STATIC_SCRATCH_BYTES
 * (64 MiB) per GPU, held from the library's load until the process ends.
 * Same arguments (minus workspace), result, precondition and errors as
 * pa_reshape_and_decode, plus PA_ERR_SCRATCH when the launch's partials
 * (pa_decode_workspace_bytes of its sizes) exceed the array, and
 * PA_ERR_LAUNCH when the array's address cannot be found on the current
 * device.  It calls no allocating routine; the array's device address is
 * looked up once per device, on the first call made with that device
 * current.
 *
 * Unlike every other call this one keeps state: all calls on one GPU share
 * its array, which holds the last call's partials afterwards (no call reads
 * what an earlier one left: every slot the merge reads is written first in
 * the same call).  Calls that overlap on one GPU -- enqueued on different
 * streams without ordering between them -- race on the array and give
 * undefined results; calls on one stream, or ordered by events, are safe.
 */
#define PA_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int pa_reshape_and_decode_static(void* out, const void* q, const void* key, const void* value,
                                 void* k_cache, void* v_cache, const int64_t* slot_mapping,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                 int64_t num_blocks, float scale, int32_t dtype,
                                 int32_t partition_size, int32_t max_context_len, void* stream);

/*
 * Split-K merge.  Sequence s has P = ceil(L / partition_size) partitions,
 * L = context_lens[s] clamped to [0, partition_size * max_partitions].  For
 * query head h the partials are
 *     max_logits[s,h,p] = max of scale * q.k_t over partition p's tokens
 *     exp_sums[s,h,p]   = sum of exp(z_t - max_logits[s,h,p]) over them
 *     tmp_out[s,h,p,:]  = sum exp(z_t - max_logits) v_t / exp_sums   (normalised)
 * and the result is
 *     M = max_p max_logits,  w_p = exp_sums * exp(max_logits - M),
 *     out[s,h,:] = sum_p w_p tmp_out[s,h,p,:] / sum_p w_p
 * rounded into out's type (P = 1 copies the single partial, P = 0 writes
 * zeros).  Layouts: max_logits, exp_sums [num_seqs, num_q_heads,
 * max_partitions] float32; tmp_out [num_seqs, num_q_heads, max_partitions,
 * head_dim] float32.  Entries p >= P are not read.
 */
int pa_paged_attention_reduce(void* out, const float* max_logits, const float* exp_sums,
                              const float* tmp_out, const int32_t* context_lens,
                              int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                              int32_t partition_size, int32_t max_partitions, int32_t dtype,
                              void* stream);

/*
 * Workspace bytes pa_paged_attention_decode needs for these sizes: 0 for
 * partition_size = 0 or when every sequence fits one partition, else room
 * for tmp_out, max_logits and exp_sums with
 * max_partitions = ceil(max_context_len / partition_size).  Returns 0 for
 * invalid arguments (which the decode call then rejects).
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_size);

/*
 * Cascade decode, for batches whose sequences share prompt pages ([CX] §2.1
 * and §2.3: several sequences' tables point at the same physical blocks;
 * [DM] "sharing mechanism").  Same result as pa_paged_attention_decode with
 * partition_size = 0, computed in two parts.  Runs of 16 / G consecutive
 * sequences (G = num_q_heads / num_kv_heads; runs start at sequence 0) whose
 * tables begin with the same physical blocks -- whole blocks inside every
 * member's context, at least 4 of them -- get the attention over those
 * blocks once for the whole run, the query rows of all members in one
 * matrix-core tile; each sequence's remaining blocks are then processed as in
 * pa_paged_attention_decode and the two parts merged by the log-sum-exp rule
 * of pa_paged_attention_reduce.  Runs that share fewer blocks are decoded as
 * usual; float32, G > 8, num_seqs < 2 or a block size other than 16 skip the
 * shared part altogether.
 *
 * `workspace` (device memory, caller-owned) must hold at least
 * pa_cascade_workspace_bytes(num_seqs, num_q_heads, head_dim) bytes: it
 * carries the shared part's per-row state from the first kernel to the
 * second.  Calls that share a workspace must not run concurrently.  Other
 * arguments, layouts and errors as for pa_paged_attention_decode.
 */
int pa_paged_attention_decode_cascade(void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size,
                                      int32_t max_blocks_per_seq, int64_t num_blocks,
                                      float scale, int32_t dtype, int32_t max_context_len,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * The one-call step of the cascade entry point: each sequence's new token
 * (key, value [num_seqs, num_kv_heads, head_dim], slot_mapping [num_seqs])
 * written into the caches, then pa_paged_attention_decode_cascade.  The
 * shared-prefix kernel stores the new rows (each of its workgroups those of
 * its run of sequences, while it measures the shared part), so the decode
 * kernel after it reads them from the caches; where that kernel does not run
 * (fp32, more than 8 query heads per KV head, fewer than two sequences,
 * block sizes other than 16) the decode kernels store them, as in
 * pa_reshape_and_decode.  Precondition as
 * for pa_reshape_and_decode: no context reads, in this call, a slot written
 * in this call other than its own last position (the shared-prefix kernel
 * reads shared blocks while the rows are stored).  Under it the result is
 * the two calls'; otherwise it is undefined (pa_validate_step_host checks
 * it).  Other arguments, workspace and errors as for
 * pa_paged_attention_decode_cascade; key, value and slot_mapping must not be
 * NULL when num_seqs > 0.
 */
int pa_reshape_and_decode_cascade(void* out, const void* q, const void* key, const void* value,
                                  void* k_cache, void* v_cache, const int64_t* slot_mapping,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                  int64_t num_blocks, float scale, int32_t dtype,
                                  int32_t max_context_len, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * Workspace bytes of pa_paged_attention_decode_cascade: one int32 per
 * sequence, and per (sequence, query head) row two floats plus head_dim
 * floats, each array 256-byte aligned.  Returns 0 for invalid arguments.
 */
size_t pa_cascade_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim);

/*
 * Multi-token queries over the paged cache: several new tokens per sequence
 * in one call (chunked prefill; checking drafted tokens in one forward pass,
 * [CX] §4.1; variable-length attention with per-sequence query offsets,
 * [DM] FlashAttention backend).  Sequence s owns query tokens
 * query_start[s] <= t < query_start[s + 1] (n_s of them, the last n_s
 * tokens of its context, their K/V already written by
 * pa_reshape_and_cache).  Token i of the span sits at position
 * p = L - n_s + i (L = context_lens[s], clamped as in decode) and attends to
 * tokens 0 .. p:
 *     out[t,h,:] = sum_{u<=p} softmax_u(scale * q[t,h,:] . k_u) v_u,
 * which is [CX] §1.1's o_t = Attention(q_t, K_{1:t}, V_{1:t}) for every new
 * token at once.  A token with p < 0 gets a zero row; n_s = 1 is decode.
 *
 * Layouts: q, out [num_query_tokens, num_q_heads, head_dim];
 * query_start [num_seqs + 1] int32 device array, query_start[0] = 0,
 * non-decreasing, query_start[num_seqs] = num_query_tokens (rows of tokens
 * that no sequence's span covers are left undefined);
 * caches, block_tables, context_lens as for decode.  max_query_len bounds
 * every n_s (the kernels take at most that many tokens of a span; the rest
 * of it is left undefined).  pa_validate_query_start_host checks a host copy.
 *
 * dtype PA_F16 or PA_BF16 (PA_F32: PA_ERR_UNSUPPORTED).  partition_size as
 * for decode (0: one partition); with more than one partition `workspace`
 * must hold pa_multi_query_workspace_bytes(...) bytes (partials as in
 * decode with one row per (query token, head), and each token's causal
 * length).  num_seqs, num_query_tokens <= 65535.  Errors as for decode;
 * num_seqs, num_query_tokens or max_query_len = 0 is a no-op.
 */
int pa_paged_attention_multi_query(void* out, const void* q, const void* k_cache,
                                   const void* v_cache, const int32_t* block_tables,
                                   const int32_t* context_lens, const int32_t* query_start,
                                   int32_t num_seqs, int32_t num_query_tokens,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t max_blocks_per_seq,
                                   int64_t num_blocks, float scale, int32_t dtype,
                                   int32_t max_query_len, int32_t partition_size,
                                   int32_t max_context_len, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * Workspace bytes of pa_paged_attention_multi_query: 0 when every token
 * fits one partition (partition_size = 0 or max_context_len <=
 * partition_size), else the decode partials for num_query_tokens rows plus
 * one int32 per query token.  Returns 0 for invalid arguments.
 */
size_t pa_multi_query_workspace_bytes(int32_t num_query_tokens, int32_t num_q_heads,
                                      int32_t head_dim, int32_t max_context_len,
                                      int32_t partition_size);

/*
 * A partition size for pa_paged_attention_multi_query (host only, no
 * device work): 0 (one pass) when the one-pass items -- (sequence, KV head,
 * unit of up to 128 query rows) -- already number at least four per compute
 * unit of the current device; else the longest power-of-two partition that
 * still makes that many items at max_context_len, and no shorter than 16
 * tokens per query row of an item (512 at least), so that the float partials
 * stay under 1/16 of the K/V bytes each item reads; 0 when that covers
 * max_context_len.  The result is a suggestion: any valid partition_size
 * gives the same attention up to rounding.  Returns 0 for invalid arguments.
 */
int32_t pa_multi_query_partition_size(int32_t num_seqs, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t max_query_len,
                                      int32_t max_context_len);

/*
 * Host-side check of query offsets (host pointers): query_start[0] = 0,
 * query_start[num_seqs] = num_query_tokens, every span length n_s in
 * [0, max_query_len] and, when context_lens is not NULL, n_s <=
 * context_lens[s].  Returns PA_OK, PA_ERR_RANGE, PA_ERR_NULL or PA_ERR_SHAPE.
 * Touches no GPU.
 */
int pa_validate_query_start_host(const int32_t* query_start, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t num_query_tokens,
                                 int32_t max_query_len);

/*
 * Copy-on-write of shared blocks ([CX] §2.1: requests of one prompt --
 * parallel sampling, beam search -- share its pages; [DM] sharing
 * mechanism): for every pair i, block block_pairs[2i] of both caches (all
 * KV heads) is copied onto block block_pairs[2i+1].  block_pairs is a
 * device array [num_pairs, 2] int32.  Destinations must be distinct and no
 * destination may be a source in the same call (a caller error otherwise;
 * pa_validate_copy_host checks a host copy); pairs naming a block outside
 * [0, num_blocks) are skipped.  num_pairs <= 65535; 0 is a no-op.
 */
int pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_pairs, int32_t num_pairs,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                   int64_t num_blocks, int32_t dtype, void* stream);

/*
 * Swap blocks between two caches of the same layout, one of them usually in
 * pinned host memory ([DM] block manager: blocks swapped out to CPU memory
 * and back in): for every pair i, block_bytes bytes at block
 * block_pairs[2i] of src_cache go to block block_pairs[2i+1] of dst_cache
 * (one call per cache: K and V are separate arrays).  block_pairs is a host
 * array [num_pairs, 2] int64; runs of consecutive pairs move as one copy.
 * Enqueued on `stream` as asynchronous copies (host memory must be pinned
 * for them to be asynchronous).  Negative ids give PA_ERR_RANGE (nothing
 * enqueued); the caller keeps ids inside both caches.
 */
int pa_swap_blocks(const void* src_cache, void* dst_cache, const int64_t* block_pairs,
                   int32_t num_pairs, int64_t block_bytes, void* stream);

/*
 * The same block moves as pa_swap_blocks, done by one kernel instead of a
 * copy per block: for every pair i, block_bytes bytes at block
 * block_pairs[2i] of src_cache go to block block_pairs[2i+1] of dst_cache.
 * Either cache may be pinned host memory (the kernel reaches it through its
 * device mapping) or device memory; block_pairs [num_pairs, 2] int64 must
 * be device memory or pinned host memory too.  Pointers the device cannot
 * reach (pageable host memory) give PA_ERR_UNSUPPORTED before anything is
 * launched, as do caches not 16-byte aligned.  Pairs naming a block outside
 * [0, src_blocks) or [0, dst_blocks) are skipped.  block_bytes a positive
 * multiple of 16; num_pairs <= 65535; 0 is a no-op.  Destinations must be
 * distinct (a caller error otherwise).
 */
int pa_swap_blocks_mapped(const void* src_cache, void* dst_cache, const int64_t* block_pairs,
                          int32_t num_pairs, int64_t block_bytes, int64_t src_blocks,
                          int64_t dst_blocks, void* stream);

/*
 * Host check of copy pairs (host pointer): ids in [0, num_blocks), distinct
 * destinations, no destination used as a source.  PA_OK or PA_ERR_RANGE.
 */
int pa_validate_copy_host(const int32_t* block_pairs, int32_t num_pairs, int64_t num_blocks);

/*
 * Host-side check of block tables (host pointers): every entry a sequence
 * uses, logical blocks 0 .. ceil(L/block_size)-1, must lie in
 * [0, num_blocks), ceil(L/block_size) must not exceed max_blocks_per_seq and
 * L must be >= 0.  Returns PA_OK, PA_ERR_RANGE, PA_ERR_NULL or PA_ERR_SHAPE.
 * Touches no GPU.
 */
int pa_validate_tables_host(const int32_t* block_tables, const int32_t* context_lens,
                            int32_t num_seqs, int32_t max_blocks_per_seq,
                            int64_t num_blocks, int32_t block_size);

/*
 * Host-side check of a slot mapping (host pointer): every slot is negative
 * or below 16 * num_blocks, and no two non-negative slots are equal.
 * Returns PA_OK, PA_ERR_RANGE, PA_ERR_NULL or PA_ERR_SHAPE.
 */
int pa_validate_slots_host(const int64_t* slot_mapping, int32_t num_tokens,
                           int64_t num_blocks, int32_t block_size);

/*
 * Host-side check of one decode step for pa_reshape_and_decode and
 * pa_reshape_and_decode_cascade (host pointers; one new token per sequence,
 * slot_mapping [num_seqs]): the tables
 * and the slots pass pa_validate_tables_host and pa_validate_slots_host, and
 * no context reads a slot written in this step other than the writer's own
 * last position context_lens[s] - 1 -- the condition under which the one-call
 * step equals the KV write followed by the decode.  Returns PA_OK,
 * PA_ERR_RANGE (first violation), PA_ERR_NULL or PA_ERR_SHAPE.
 */
int pa_validate_step_host(const int64_t* slot_mapping, const int32_t* block_tables,
                          const int32_t* context_lens, int32_t num_seqs,
                          int32_t max_blocks_per_seq, int64_t num_blocks, int32_t block_size);

/* Static description of a status code. */
const char* pa_status_string(int status);

/* Library version string. */
const char* pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
