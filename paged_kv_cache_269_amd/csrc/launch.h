// Internal launch interface between the C-ABI host layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Everything a decode kernel needs, passed by value as one kernel argument.
struct DecodeArgs {
  void* out;                    // [B, Hq, D] element type
  const void* q;                // [B, Hq, D]
  const void* k_cache;          // [N, Hkv, 16, D]
  const void* v_cache;          // [N, Hkv, 16, D]
  const int32_t* block_tables;  // [B, M]
  const int32_t* context_lens;  // [B]
  float* tmp_out;               // [B, Hq, P, D] partial outputs (normalised)
  float* max_logits;            // [B, Hq, P]  (natural-log units)
  float* exp_sums;              // [B, Hq, P]
  int num_seqs;                 // B
  int num_blocks_i32;           // N, clamped to INT32_MAX (block ids are int32)
  int num_q_heads;              // Hq
  int num_kv_heads;             // Hkv
  int max_blocks_per_seq;       // M
  int max_len;                  // contexts are clamped to [0, max_len]
  int part_blocks;              // blocks per partition
  int max_partitions;           // P (partials stride)
  float scale_log2;             // scale * log2(e)
  int block_size;               // tokens per pool block: 8, 16 or 32 (kernels work on
                                // 16-token tiles; lengths and partitions count those)
  // Shared-prefix launches: per sequence, the leading blocks whose attention
  // the prefix kernel has already computed (nullptr: none), and that part's
  // state per (sequence, query head) row.
  const int32_t* prefix_blocks;  // [B]
  const float* prefix_m;         // [B, Hq] max score, base 2
  const float* prefix_l;         // [B, Hq] sum of exp2(score - max)
  const float* prefix_o;         // [B, Hq, D] normalised output of the prefix part
  // Fused KV write (new_slots != nullptr): each sequence's new token, rows
  // new_k / new_v [B, Hkv, D], goes to slot new_slots[s] of the caches (skipped
  // when the slot is negative or past the pool).  One item per (sequence, KV
  // head) stores it; every item whose context ends with that slot takes the
  // row from new_k / new_v instead of reading the cache.
  const void* new_k;
  const void* new_v;
  const int64_t* new_slots;     // [B]
  int64_t num_blocks;           // N (slot bound of the write)
  int grid_order;               // 1: grid slots take the sequences in grid order (a launch
                                // whose items all start at once; see longest_first)
};

// Outputs of the shared-prefix kernel (the same arrays DecodeArgs reads).
struct PrefixOut {
  int32_t* prefix_blocks;
  float* m;
  float* l;
  float* o;
};

// The step's KV write when the shared-prefix kernel carries it: sequence s's
// new K/V rows ([B, Hkv, D]) go to slot slots[s] of the pools (skipped when
// the slot is negative or at or past num_slots).  slots == nullptr: no write.
struct KvWrite {
  const void* key;
  const void* value;
  void* k_cache;
  void* v_cache;
  const int64_t* slots;
  int64_t num_slots;
};

// Multi-token queries (query tokens t of sequence s: query_start[s] <=
// t < query_start[s + 1]).  `d.q` and `d.out` are [T, Hq, D]; the partials
// are laid out as in decode with one row per (query token, query head).
struct MultiQueryArgs {
  DecodeArgs d;
  const int32_t* query_start;  // [B + 1]
  int32_t* token_lens;         // [T] causal length of each query token, written for the
                               // reduce (nullptr: a single partition)
  int num_query_tokens;        // T
  int max_query_len;           // query tokens per sequence are clamped to this
  int wide;                    // 1: the waves of an item own disjoint row tiles and share
                               //    every K/V tile through LDS; 0: they split the tiles
  int row_tiles;               // 16-row tiles per item, or per wave of a wide item: 1 or 2
  int units;                   // items per KV head
  int reread;                  // 1: K/V tiles are read by several items (cache them)
};

struct ReduceArgs {
  void* out;
  const float* max_logits;
  const float* exp_sums;
  const float* tmp_out;
  const int32_t* context_lens;
  int num_q_heads;
  int partition_size;
  int max_partitions;
  int max_len;
  int skip_single;              // 1: sequences with <= 1 partition are left alone
};

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_cache,
                                    void* v_cache, const int64_t* slot_mapping, int num_tokens,
                                    int num_kv_heads, int head_dim, int elem_bytes, int block_size,
                                    int64_t num_blocks, hipStream_t stream);

// Block copies inside both caches: pairs [num_pairs, 2] int32 (src, dst) on
// the device; block_bytes = one block of one cache (all KV heads).
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int num_pairs,
                              int64_t block_bytes, int64_t num_blocks, hipStream_t stream);

// Blocks between two caches: pairs [num_pairs, 2] int64 (src block, dst
// block), device-accessible; src/dst device-accessible (device memory or the
// device mapping of pinned host memory).
hipError_t launch_swap_blocks(const void* src, void* dst, const int64_t* pairs, int num_pairs,
                              int64_t block_bytes, int64_t src_blocks, int64_t dst_blocks,
                              hipStream_t stream);

// Vector-ALU decode: one workgroup per (query head, sequence, partition) item.
hipError_t launch_decode_valu(const DecodeArgs& a, int dtype, int head_dim, hipStream_t stream);

// Matrix-core decode for grouped heads: one workgroup per (kv head x 16-head
// tile, sequence, partition) item.
hipError_t launch_decode_mfma(const DecodeArgs& a, int dtype, int head_dim, hipStream_t stream);

// Whether launch_decode_mfma takes the streaming kernel for these arguments
// (it does no fused KV write: the caller writes first).
bool decode_mfma_streams(const DecodeArgs& a);

// Shared-prefix pass: for runs of consecutive sequences whose block tables
// start with the same full blocks, the attention over those blocks, once per
// run (f16/bf16, at most 8 query heads per KV head); with w.slots set it also
// does the step's KV write (block size 16).
hipError_t launch_prefix(const DecodeArgs& a, const PrefixOut& o, const KvWrite& w, int dtype,
                         int head_dim, hipStream_t stream);

// Matrix-core multi-query attention: one workgroup per (kv head x 16-row
// unit, sequence, partition) item (f16/bf16).
hipError_t launch_multi_query(const MultiQueryArgs& a, int dtype, int head_dim,
                              hipStream_t stream);

hipError_t launch_reduce(const ReduceArgs& a, int dtype, int head_dim, int num_seqs,
                         hipStream_t stream);

// hipGetLastError() reports the last error of any runtime call made on this
// thread, not only of the launch it follows.  Every launch function below
// clears one left behind by an earlier call (another library's, or a failed
// device query) before it launches, so the status it returns is that of its
// own launches.
inline void clear_stale_error() { (void)hipGetLastError(); }

// Host: compute units of the current device (cached per device; <= 0 on a
// runtime error).
inline int compute_units() {
  static int per_device[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  const bool cacheable = dev >= 0 && dev < 64;
  int cus = cacheable ? __atomic_load_n(&per_device[dev], __ATOMIC_RELAXED) : 0;
  if (cus <= 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return -1;
    if (cacheable && cus > 0) __atomic_store_n(&per_device[dev], cus, __ATOMIC_RELAXED);
  }
  return cus;
}

// Host: workgroups of `kernel` (block of `threads`) resident on the current
// device at once, cached per device.  Returns <= 0 on a runtime error.
struct ResidentCache {
  int per_device[64] = {};
};

inline int resident_workgroups(const void* kernel, int threads, ResidentCache& c) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  const bool cacheable = dev >= 0 && dev < 64;
  int resident = cacheable ? __atomic_load_n(&c.per_device[dev], __ATOMIC_RELAXED) : 0;
  if (resident <= 0) {
    int per_cu = 0;
    const int cus = compute_units();
    if (cus <= 0 ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess)
      return -1;
    resident = per_cu * cus;
    if (cacheable && resident > 0) __atomic_store_n(&c.per_device[dev], resident, __ATOMIC_RELAXED);
  }
  return resident;
}

}  // namespace pa
