// KV write: scatter each new token's K and V rows into its cache slot.
//
// "vLLM 2026 推理引擎全解" (chenxutan.com), §1.1: the K and V of every token
// are stored in HBM once and re-read by later decode steps.  §2.2 of the same
// page: a token's address in the pool is page_id * BLOCK_SIZE + page_offset,
// which is the slot this kernel receives.
//
// One work-item moves one 16-byte chunk of one (token, kv head) row of K and
// the matching chunk of V; a row of head_dim elements is D*e/16 chunks, so
// consecutive work-items read consecutive 16 bytes of `key` and write
// consecutive 16 bytes of one cache row (coalesced on both sides).
#include "common.h"
#include "launch.h"

namespace pa {

__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const u32x4* __restrict__ key, const u32x4* __restrict__ value, u32x4* __restrict__ k_cache,
    u32x4* __restrict__ v_cache, const int64_t* __restrict__ slot_mapping, int64_t total_chunks,
    int chunks_per_row, int num_kv_heads, int block_size, int64_t num_slots) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total_chunks) return;
  const int chunk = (int)(i % chunks_per_row);
  const int64_t row = i / chunks_per_row;           // token * num_kv_heads + head
  const int head = (int)(row % num_kv_heads);
  const int64_t token = row / num_kv_heads;
  const int64_t slot = slot_mapping[token];
  if (slot < 0 || slot >= num_slots) return;        // padding / out of the pool
  const int64_t block = slot / block_size;
  const int offset = (int)(slot % block_size);
  const int64_t dst = ((block * num_kv_heads + head) * block_size + offset) * chunks_per_row + chunk;
  k_cache[dst] = key[i];
  v_cache[dst] = value[i];
}

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_cache,
                                    void* v_cache, const int64_t* slot_mapping, int num_tokens,
                                    int num_kv_heads, int head_dim, int elem_bytes, int block_size,
                                    int64_t num_blocks, hipStream_t stream) {
  clear_stale_error();
  const int chunks_per_row = head_dim * elem_bytes / 16;
  const int64_t total = (int64_t)num_tokens * num_kv_heads * chunks_per_row;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     (const u32x4*)key, (const u32x4*)value, (u32x4*)k_cache, (u32x4*)v_cache,
                     slot_mapping, total, chunks_per_row, num_kv_heads, block_size,
                     num_blocks * block_size);
  return hipGetLastError();
}

}  // namespace pa
