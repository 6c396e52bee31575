// Block copies inside the KV pool (copy-on-write of a shared block).
//
// The pages' sharing mechanism (vLLM manual (doramagic.ai), "sharing
// mechanism"; "vLLM 2026 推理引擎全解" (chenxutan.com) §2.1: parallel sampling
// and beam search share a prefix's pages) keeps one physical copy of a
// block for several requests; a request about to write into a block it still
// shares first gets a private copy.  For every (src, dst) pair this kernel
// copies block src of both caches, all KV heads, onto block dst.
// swap_blocks_kernel moves blocks between two caches instead (swap out to /
// in from pinned host memory through its device mapping).
//
// Work split: one workgroup per (pair, 16 KiB chunk of the block); each lane
// moves 16-byte chunks of K and V (coalesced reads and writes, non-temporal:
// the data is not read again by this kernel).  Pairs naming a block outside
// the pool are skipped.
#include "common.h"
#include "launch.h"

namespace pa {

namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyChunksPerLane = 4;
constexpr int kCopyChunkBytes = kCopyThreads * kCopyChunksPerLane * 16;  // 16 KiB per workgroup

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    u32x4* __restrict__ k_cache, u32x4* __restrict__ v_cache, const int32_t* __restrict__ pairs,
    int64_t block_chunks, int64_t num_blocks) {
  const int p = blockIdx.y;
  const int64_t src = pairs[2 * p], dst = pairs[2 * p + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const int64_t base = (int64_t)blockIdx.x * (kCopyChunkBytes / 16);
  u32x4 k[kCopyChunksPerLane], v[kCopyChunksPerLane];
#pragma unroll
  for (int i = 0; i < kCopyChunksPerLane; ++i) {
    const int64_t c = base + i * kCopyThreads + threadIdx.x;
    if (c < block_chunks) {
      k[i] = __builtin_nontemporal_load(&k_cache[src * block_chunks + c]);
      v[i] = __builtin_nontemporal_load(&v_cache[src * block_chunks + c]);
    }
  }
#pragma unroll
  for (int i = 0; i < kCopyChunksPerLane; ++i) {
    const int64_t c = base + i * kCopyThreads + threadIdx.x;
    if (c < block_chunks) {
      __builtin_nontemporal_store(k[i], &k_cache[dst * block_chunks + c]);
      __builtin_nontemporal_store(v[i], &v_cache[dst * block_chunks + c]);
    }
  }
}

// Blocks from one cache to another (either may be pinned host memory seen
// through its device mapping): block pairs[2p] of src onto block
// pairs[2p + 1] of dst, block_chunks 16-byte chunks each; pairs naming a
// block outside either cache are skipped.
__global__ __launch_bounds__(kCopyThreads) void swap_blocks_kernel(
    const u32x4* __restrict__ src, u32x4* __restrict__ dst, const int64_t* __restrict__ pairs,
    int64_t block_chunks, int64_t src_blocks, int64_t dst_blocks) {
  const int p = blockIdx.y;
  const int64_t sb = pairs[2 * p], db = pairs[2 * p + 1];
  if (sb < 0 || sb >= src_blocks || db < 0 || db >= dst_blocks) return;
  const int64_t base = (int64_t)blockIdx.x * (kCopyChunkBytes / 16);
  u32x4 x[kCopyChunksPerLane];
#pragma unroll
  for (int i = 0; i < kCopyChunksPerLane; ++i) {
    const int64_t c = base + i * kCopyThreads + threadIdx.x;
    if (c < block_chunks) x[i] = __builtin_nontemporal_load(&src[sb * block_chunks + c]);
  }
#pragma unroll
  for (int i = 0; i < kCopyChunksPerLane; ++i) {
    const int64_t c = base + i * kCopyThreads + threadIdx.x;
    if (c < block_chunks) __builtin_nontemporal_store(x[i], &dst[db * block_chunks + c]);
  }
}

}  // namespace

hipError_t launch_swap_blocks(const void* src, void* dst, const int64_t* pairs, int num_pairs,
                              int64_t block_bytes, int64_t src_blocks, int64_t dst_blocks,
                              hipStream_t stream) {
  clear_stale_error();
  const int64_t chunks = block_bytes / 16;
  const int64_t per_block = (block_bytes + kCopyChunkBytes - 1) / kCopyChunkBytes;
  hipLaunchKernelGGL(swap_blocks_kernel, dim3((unsigned)per_block, (unsigned)num_pairs),
                     dim3(kCopyThreads), 0, stream, (const u32x4*)src, (u32x4*)dst, pairs, chunks,
                     src_blocks, dst_blocks);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int num_pairs,
                              int64_t block_bytes, int64_t num_blocks, hipStream_t stream) {
  clear_stale_error();
  const int64_t chunks = block_bytes / 16;
  const int64_t per_block = (block_bytes + kCopyChunkBytes - 1) / kCopyChunkBytes;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)per_block, (unsigned)num_pairs),
                     dim3(kCopyThreads), 0, stream, (u32x4*)k_cache, (u32x4*)v_cache, pairs,
                     chunks, num_blocks);
  return hipGetLastError();
}

}  // namespace pa
