// C-ABI host layer of libpagedattn: argument checks, kernel choice, launches.
// Declarations and the meaning of every argument: include/pagedattn.h.
#include "pagedattn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdint>
#include <utility>
#include <vector>

#include "launch.h"

namespace {

#ifndef PA_MQ_WIDE_ROWS
#define PA_MQ_WIDE_ROWS 32  // multi-query rows per KV head above which items are wide
#endif

#ifndef PA_MFMA_MIN_GROUP
#define PA_MFMA_MIN_GROUP 2  // smallest head group sent to the matrix-core kernel
#endif

constexpr int kBlock = 16;  // tokens per kernel tile; partitions are multiples of it

// Pool block sizes the kernels take (tokens per block).
bool block_size_ok(int32_t bs) { return bs == 8 || bs == 16 || bs == 32; }
constexpr int kMaxGridYZ = 65535;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int elem_bytes(int32_t dtype) {
  switch (dtype) {
    case PA_F32: return 4;
    case PA_F16: return 2;
    case PA_BF16: return 2;
    default: return 0;
  }
}

bool head_dim_ok(int32_t d) { return d == 64 || d == 128; }

struct WsLayout {
  size_t tmp_out = 0, max_logits = 0, exp_sums = 0, total = 0;
};

// Partials layout for P > 1 partitions: [tmp_out | max_logits | exp_sums].
WsLayout ws_layout(int64_t num_seqs, int64_t heads, int64_t head_dim, int64_t parts) {
  WsLayout w;
  if (parts <= 1) return w;
  const size_t rows = (size_t)num_seqs * heads * parts;
  w.tmp_out = 0;
  w.max_logits = w.tmp_out + align256(rows * head_dim * sizeof(float));
  w.exp_sums = w.max_logits + align256(rows * sizeof(float));
  w.total = w.exp_sums + align256(rows * sizeof(float));
  return w;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Shared-prefix state layout: [prefix_blocks (B) int32 | m (B Hq) | l (B Hq) |
// o (B Hq D)], each 256-byte aligned.
struct CascadeLayout {
  size_t prefix_blocks = 0, m = 0, l = 0, o = 0, total = 0;
};

CascadeLayout cascade_layout(int64_t num_seqs, int64_t heads, int64_t head_dim) {
  CascadeLayout c;
  const size_t rows = (size_t)num_seqs * heads;
  c.m = align256((size_t)num_seqs * sizeof(int32_t));
  c.l = c.m + align256(rows * sizeof(float));
  c.o = c.l + align256(rows * sizeof(float));
  c.total = c.o + align256(rows * head_dim * sizeof(float));
  return c;
}

// The largest query-head group the shared-prefix kernel handles (16 / G
// sequences per matrix-core tile).
constexpr int kCascadeMaxGroup = 8;

int decode_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                int32_t max_blocks_per_seq, int64_t num_blocks, float scale, int32_t dtype,
                int32_t partition_size, int32_t max_context_len, void* workspace,
                size_t workspace_bytes, void* stream, bool cascade,
                const void* new_k = nullptr, const void* new_v = nullptr,
                const int64_t* new_slots = nullptr);

}  // namespace

namespace {

int decode_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                int32_t max_blocks_per_seq, int64_t num_blocks, float scale, int32_t dtype,
                int32_t partition_size, int32_t max_context_len, void* workspace,
                size_t workspace_bytes, void* stream, bool cascade,
                const void* new_k, const void* new_v, const int64_t* new_slots) {
  if (!elem_bytes(dtype) || !block_size_ok(block_size) || !head_dim_ok(head_dim))
    return PA_ERR_UNSUPPORTED;
  if (partition_size < 0 || partition_size % kBlock) return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || num_seqs > kMaxGridYZ || num_q_heads <= 0 || num_q_heads > kMaxGridYZ ||
      num_kv_heads <= 0 || num_q_heads % num_kv_heads || max_blocks_per_seq <= 0 ||
      num_blocks <= 0 || max_context_len < 0)
    return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_NULL;

  // Longest context any kernel will look at.
  const int64_t max_len =
      std::min<int64_t>(max_context_len, (int64_t)max_blocks_per_seq * block_size);
  const int64_t table_blocks = ceil_div(std::max<int64_t>(max_len, 1), kBlock);
  int64_t part_blocks, parts;
  if (partition_size == 0) {
    part_blocks = table_blocks;
    parts = 1;
  } else {
    part_blocks = partition_size / kBlock;
    parts = std::max<int64_t>(1, ceil_div(max_len, partition_size));
  }
  if (parts > kMaxGridYZ) return PA_ERR_SHAPE;  // partitions are a grid dimension

  const WsLayout ws = ws_layout(num_seqs, num_q_heads, head_dim, parts);
  if (ws.total && (!workspace || workspace_bytes < ws.total)) return PA_ERR_WORKSPACE;
  const CascadeLayout cl = cascade_layout(num_seqs, num_q_heads, head_dim);
  if (cascade && (!workspace || workspace_bytes < cl.total)) return PA_ERR_WORKSPACE;

  pa::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  char* wsb = static_cast<char*>(workspace);
  a.tmp_out = parts > 1 ? reinterpret_cast<float*>(wsb + ws.tmp_out) : nullptr;
  a.max_logits = parts > 1 ? reinterpret_cast<float*>(wsb + ws.max_logits) : nullptr;
  a.exp_sums = parts > 1 ? reinterpret_cast<float*>(wsb + ws.exp_sums) : nullptr;
  a.num_seqs = num_seqs;
  a.num_blocks_i32 = (int)std::min<int64_t>(num_blocks, INT32_MAX);
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_len = (int)max_len;
  a.part_blocks = (int)part_blocks;
  a.max_partitions = (int)parts;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  {
    // every item starts at once when there are no more than compute units
    const int cus = pa::compute_units();
    const int64_t items = (int64_t)num_seqs * num_q_heads * parts;
    a.grid_order = (cus > 0 && items <= cus) ? 1 : 0;
  }

  const hipStream_t st = (hipStream_t)stream;
  const int group = num_q_heads / num_kv_heads;
  // Grouped heads share every K/V tile: a matrix-core product pays off from
  // two heads up.  Single heads and fp32 stay on the vector ALU.
  const bool use_mfma = dtype != PA_F32 && group >= PA_MFMA_MIN_GROUP;
  const bool prefix_pass = cascade && dtype != PA_F32 && group <= kCascadeMaxGroup &&
                           num_seqs >= 2 && block_size == kBlock;
  pa::KvWrite kw{};
  if (new_slots != nullptr) {
    // New tokens' K/V: written by the decode kernel itself; where the
    // shared-prefix pass runs, by the shared-prefix kernel (the decode's
    // short items after it measured 1.3% slower doing the write themselves).
    if (prefix_pass) {
      kw = pa::KvWrite{new_k, new_v, const_cast<void*>(k_cache), const_cast<void*>(v_cache),
                       new_slots, num_blocks * block_size};
    } else {
      a.new_k = new_k;
      a.new_v = new_v;
      a.new_slots = new_slots;
    }
  }
  if (prefix_pass) {
    // Shared-prefix pass first; the decode kernel then covers each
    // sequence's remaining blocks and merges the two parts.
    char* c = static_cast<char*>(workspace);
    pa::PrefixOut po{reinterpret_cast<int32_t*>(c + cl.prefix_blocks),
                     reinterpret_cast<float*>(c + cl.m), reinterpret_cast<float*>(c + cl.l),
                     reinterpret_cast<float*>(c + cl.o)};
    a.prefix_blocks = po.prefix_blocks;
    a.prefix_m = po.m;
    a.prefix_l = po.l;
    a.prefix_o = po.o;
    if (pa::launch_prefix(a, po, kw, dtype, head_dim, st) != hipSuccess) return PA_ERR_LAUNCH;
  }
  hipError_t e = use_mfma ? pa::launch_decode_mfma(a, dtype, head_dim, st)
                          : pa::launch_decode_valu(a, dtype, head_dim, st);
  if (e != hipSuccess) return PA_ERR_LAUNCH;
  if (parts > 1) {
    pa::ReduceArgs r{};
    r.out = out;
    r.max_logits = a.max_logits;
    r.exp_sums = a.exp_sums;
    r.tmp_out = a.tmp_out;
    r.context_lens = context_lens;
    r.num_q_heads = num_q_heads;
    r.partition_size = partition_size;
    r.max_partitions = (int)parts;
    r.max_len = (int)max_len;
    r.skip_single = 1;
    e = pa::launch_reduce(r, dtype, head_dim, num_seqs, st);
    if (e != hipSuccess) return PA_ERR_LAUNCH;
  }
  return PA_OK;
}

}  // namespace

extern "C" {

const char* pa_version(void) { return "libpagedattn 0.1.0 (gfx950)"; }

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "a size is out of range or num_q_heads is not a multiple of num_kv_heads";
    case PA_ERR_UNSUPPORTED:
      return "unsupported head_dim (64, 128), block_size (8, 16, 32), dtype or partition_size";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_RANGE: return "table entry, context length or slot out of range";
    case PA_ERR_LAUNCH: return "the HIP runtime refused a kernel launch";
    case PA_ERR_EXHAUSTED: return "KV cache exhausted: no free block left";
    case PA_ERR_SCRATCH:
      return "the partials need more than the library's static scratch array holds";
    default: return "unknown status";
  }
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_size) {
  if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0 ||
      partition_size < 0)
    return 0;
  const int64_t parts = partition_size ? ceil_div(max_context_len, partition_size) : 1;
  return ws_layout(num_seqs, num_q_heads, head_dim, parts).total;
}

int pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                         const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int64_t num_blocks, int32_t dtype,
                         void* stream) {
  const int eb = elem_bytes(dtype);
  if (!eb || !block_size_ok(block_size) || !head_dim_ok(head_dim)) return PA_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PA_ERR_NULL;
  hipError_t e = pa::launch_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping,
                                              num_tokens, num_kv_heads, head_dim, eb, block_size,
                                              num_blocks, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int pa_paged_attention_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                              int64_t num_blocks, float scale, int32_t dtype,
                              int32_t partition_size, int32_t max_context_len, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale,
                     dtype, partition_size, max_context_len, workspace, workspace_bytes, stream,
                     false);
}

int pa_reshape_and_decode(void* out, const void* q, const void* key, const void* value,
                          void* k_cache, void* v_cache, const int64_t* slot_mapping,
                          const int32_t* block_tables, const int32_t* context_lens,
                          int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                          int64_t num_blocks, float scale, int32_t dtype, int32_t partition_size,
                          int32_t max_context_len, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (num_seqs > 0 && (!key || !value || !slot_mapping)) return PA_ERR_NULL;
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale,
                     dtype, partition_size, max_context_len, workspace, workspace_bytes, stream,
                     false, key, value, slot_mapping);
}

int pa_reshape_and_decode_cascade(void* out, const void* q, const void* key, const void* value,
                                  void* k_cache, void* v_cache, const int64_t* slot_mapping,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                  int64_t num_blocks, float scale, int32_t dtype,
                                  int32_t max_context_len, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  if (num_seqs > 0 && (!key || !value || !slot_mapping)) return PA_ERR_NULL;
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale,
                     dtype, 0, max_context_len, workspace, workspace_bytes, stream, true, key,
                     value, slot_mapping);
}

size_t pa_cascade_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim) {
  if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0) return 0;
  return cascade_layout(num_seqs, num_q_heads, head_dim).total;
}

int pa_paged_attention_decode_cascade(void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t max_blocks_per_seq,
                                      int64_t num_blocks, float scale, int32_t dtype,
                                      int32_t max_context_len, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale,
                     dtype, 0, max_context_len, workspace, workspace_bytes, stream, true);
}

size_t pa_multi_query_workspace_bytes(int32_t num_query_tokens, int32_t num_q_heads,
                                      int32_t head_dim, int32_t max_context_len,
                                      int32_t partition_size) {
  if (num_query_tokens < 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0 ||
      partition_size < 0)
    return 0;
  const int64_t parts = partition_size ? ceil_div(max_context_len, partition_size) : 1;
  const WsLayout w = ws_layout(num_query_tokens, num_q_heads, head_dim, parts);
  return w.total ? w.total + align256((size_t)num_query_tokens * sizeof(int32_t)) : 0;
}

int32_t pa_multi_query_partition_size(int32_t num_seqs, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t max_query_len,
                                      int32_t max_context_len) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads ||
      max_query_len <= 0 || max_context_len <= 0)
    return 0;
  // items of one pass: (sequence, KV head, unit of up to 128 rows)
  const int64_t rows = (int64_t)max_query_len * (num_q_heads / num_kv_heads);
  const int64_t item_rows = std::min<int64_t>(rows, 128);
  const int64_t one_pass = (int64_t)num_seqs * num_kv_heads * ceil_div(rows, 128);
  const int cus = pa::compute_units();
  const int64_t target = 4LL * (cus > 0 ? cus : 256);
  if (one_pass >= target) return 0;
  // a partition of at least 16 tokens per row of its item keeps the float
  // partials under 1/16 of the K/V bytes it reads; the longest such partition
  // that still yields `target` items (counted at max_context_len)
  int64_t part = 512;
  while (part < 16 * item_rows) part *= 2;
  while (one_pass * ceil_div(max_context_len, 2 * part) >= target) part *= 2;
  return part >= max_context_len ? 0 : (int32_t)part;
}

int pa_paged_attention_multi_query(void* out, const void* q, const void* k_cache,
                                   const void* v_cache, const int32_t* block_tables,
                                   const int32_t* context_lens, const int32_t* query_start,
                                   int32_t num_seqs, int32_t num_query_tokens,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t max_blocks_per_seq,
                                   int64_t num_blocks, float scale, int32_t dtype,
                                   int32_t max_query_len, int32_t partition_size,
                                   int32_t max_context_len, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if ((dtype != PA_F16 && dtype != PA_BF16) || !block_size_ok(block_size) ||
      !head_dim_ok(head_dim))
    return PA_ERR_UNSUPPORTED;
  if (partition_size < 0 || partition_size % kBlock) return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || num_seqs > kMaxGridYZ || num_query_tokens < 0 ||
      num_query_tokens > kMaxGridYZ || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads || max_blocks_per_seq <= 0 || num_blocks <= 0 ||
      max_context_len < 0 || max_query_len < 0)
    return PA_ERR_SHAPE;
  if (num_seqs == 0 || num_query_tokens == 0 || max_query_len == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
    return PA_ERR_NULL;
  // Query rows per KV head.  Up to 16 (32): items of one (two) 16-row
  // tiles whose 4 waves split the K/V tiles; more: wide items whose 4 waves
  // own one (up to 64 rows) or two 16-row tiles each and share every K/V
  // tile through LDS.
  const int64_t rows = std::min<int64_t>(max_query_len, num_query_tokens) *
                       (num_q_heads / num_kv_heads);
  const int wide = rows > PA_MQ_WIDE_ROWS ? 1 : 0;
  const int row_tiles = wide ? (rows > 64 ? 2 : 1) : (rows > 16 ? 2 : 1);
  const int64_t item_rows = (wide ? 4 : 1) * 16 * row_tiles;
  const int64_t units = ceil_div(rows, item_rows);
  if (units * num_kv_heads > INT_MAX) return PA_ERR_SHAPE;

  const int64_t max_len =
      std::min<int64_t>(max_context_len, (int64_t)max_blocks_per_seq * block_size);
  int64_t part_blocks, parts;
  if (partition_size == 0) {
    part_blocks = ceil_div(std::max<int64_t>(max_len, 1), kBlock);
    parts = 1;
  } else {
    part_blocks = partition_size / kBlock;
    parts = std::max<int64_t>(1, ceil_div(max_len, partition_size));
  }
  if (parts > kMaxGridYZ) return PA_ERR_SHAPE;
  const WsLayout ws = ws_layout(num_query_tokens, num_q_heads, head_dim, parts);
  const size_t need =
      ws.total ? ws.total + align256((size_t)num_query_tokens * sizeof(int32_t)) : 0;
  if (need && (!workspace || workspace_bytes < need)) return PA_ERR_WORKSPACE;

  pa::MultiQueryArgs m{};
  pa::DecodeArgs& a = m.d;
  char* wsb = static_cast<char*>(workspace);
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.tmp_out = parts > 1 ? reinterpret_cast<float*>(wsb + ws.tmp_out) : nullptr;
  a.max_logits = parts > 1 ? reinterpret_cast<float*>(wsb + ws.max_logits) : nullptr;
  a.exp_sums = parts > 1 ? reinterpret_cast<float*>(wsb + ws.exp_sums) : nullptr;
  a.num_seqs = num_seqs;
  a.num_blocks_i32 = (int)std::min<int64_t>(num_blocks, INT32_MAX);
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_len = (int)max_len;
  a.part_blocks = (int)part_blocks;
  a.max_partitions = (int)parts;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.block_size = block_size;
  m.query_start = query_start;
  m.token_lens = parts > 1 ? reinterpret_cast<int32_t*>(wsb + ws.total) : nullptr;
  m.num_query_tokens = num_query_tokens;
  m.max_query_len = max_query_len;
  m.wide = wide;
  m.row_tiles = row_tiles;
  m.units = (int)units;
  m.reread = units > 1 ? 1 : 0;

  const hipStream_t st = (hipStream_t)stream;
  if (pa::launch_multi_query(m, dtype, head_dim, st) != hipSuccess) return PA_ERR_LAUNCH;
  if (parts > 1) {
    // rows (query token, head) with the causal length of each token
    pa::ReduceArgs r{};
    r.out = out;
    r.max_logits = a.max_logits;
    r.exp_sums = a.exp_sums;
    r.tmp_out = a.tmp_out;
    r.context_lens = m.token_lens;
    r.num_q_heads = num_q_heads;
    r.partition_size = partition_size;
    r.max_partitions = (int)parts;
    r.max_len = (int)max_len;
    r.skip_single = 1;
    if (pa::launch_reduce(r, dtype, head_dim, num_query_tokens, st) != hipSuccess)
      return PA_ERR_LAUNCH;
  }
  return PA_OK;
}

int pa_validate_query_start_host(const int32_t* query_start, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t num_query_tokens,
                                 int32_t max_query_len) {
  if (num_seqs < 0 || num_query_tokens < 0 || max_query_len < 0) return PA_ERR_SHAPE;
  if (!query_start) return PA_ERR_NULL;
  if (query_start[0] != 0 || query_start[num_seqs] != num_query_tokens) return PA_ERR_RANGE;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t n = (int64_t)query_start[s + 1] - query_start[s];
    if (n < 0 || n > max_query_len) return PA_ERR_RANGE;
    if (context_lens && n > context_lens[s]) return PA_ERR_RANGE;
  }
  return PA_OK;
}

int pa_paged_attention_reduce(void* out, const float* max_logits, const float* exp_sums,
                              const float* tmp_out, const int32_t* context_lens, int32_t num_seqs,
                              int32_t num_q_heads, int32_t head_dim, int32_t partition_size,
                              int32_t max_partitions, int32_t dtype, void* stream) {
  if (!elem_bytes(dtype) || !head_dim_ok(head_dim)) return PA_ERR_UNSUPPORTED;
  if (partition_size <= 0) return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || num_seqs > kMaxGridYZ || num_q_heads <= 0 || max_partitions <= 0)
    return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!out || !max_logits || !exp_sums || !tmp_out || !context_lens) return PA_ERR_NULL;
  pa::ReduceArgs r{};
  r.out = out;
  r.max_logits = max_logits;
  r.exp_sums = exp_sums;
  r.tmp_out = tmp_out;
  r.context_lens = context_lens;
  r.num_q_heads = num_q_heads;
  r.partition_size = partition_size;
  r.max_partitions = max_partitions;
  r.max_len = (int)std::min<int64_t>((int64_t)partition_size * max_partitions, INT_MAX);
  r.skip_single = 0;
  hipError_t e = pa::launch_reduce(r, dtype, head_dim, num_seqs, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int pa_validate_tables_host(const int32_t* block_tables, const int32_t* context_lens,
                            int32_t num_seqs, int32_t max_blocks_per_seq, int64_t num_blocks,
                            int32_t block_size) {
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || num_blocks < 0 || block_size <= 0)
    return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!block_tables || !context_lens) return PA_ERR_NULL;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t L = context_lens[s];
    if (L < 0) return PA_ERR_RANGE;
    const int64_t used = ceil_div(L, block_size);
    if (used > max_blocks_per_seq) return PA_ERR_RANGE;
    const int32_t* row = block_tables + (int64_t)s * max_blocks_per_seq;
    for (int64_t j = 0; j < used; ++j)
      if (row[j] < 0 || row[j] >= num_blocks) return PA_ERR_RANGE;
  }
  return PA_OK;
}

int pa_validate_slots_host(const int64_t* slot_mapping, int32_t num_tokens, int64_t num_blocks,
                           int32_t block_size) {
  if (num_tokens < 0 || num_blocks < 0 || block_size <= 0) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!slot_mapping) return PA_ERR_NULL;
  const int64_t limit = num_blocks * block_size;
  std::vector<int64_t> used;
  used.reserve(num_tokens);
  for (int32_t i = 0; i < num_tokens; ++i) {
    const int64_t slot = slot_mapping[i];
    if (slot >= limit) return PA_ERR_RANGE;
    if (slot >= 0) used.push_back(slot);
  }
  std::sort(used.begin(), used.end());
  if (std::adjacent_find(used.begin(), used.end()) != used.end()) return PA_ERR_RANGE;
  return PA_OK;
}

int pa_validate_step_host(const int64_t* slot_mapping, const int32_t* block_tables,
                          const int32_t* context_lens, int32_t num_seqs,
                          int32_t max_blocks_per_seq, int64_t num_blocks, int32_t block_size) {
  int rc = pa_validate_tables_host(block_tables, context_lens, num_seqs, max_blocks_per_seq,
                                   num_blocks, block_size);
  if (rc != PA_OK) return rc;
  rc = pa_validate_slots_host(slot_mapping, num_seqs, num_blocks, block_size);
  if (rc != PA_OK || num_seqs == 0) return rc;
  // Every (sequence, logical block) of every context, grouped by pool block.
  std::vector<std::pair<int32_t, int64_t>> reads;  // (pool block, s * M + j)
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t nb = ceil_div(context_lens[s], block_size);
    for (int64_t j = 0; j < nb; ++j)
      reads.emplace_back(block_tables[(int64_t)s * max_blocks_per_seq + j],
                         (int64_t)s * max_blocks_per_seq + j);
  }
  std::sort(reads.begin(), reads.end());
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t slot = slot_mapping[s];
    if (slot < 0) continue;
    const int32_t b = (int32_t)(slot / block_size), off = (int32_t)(slot % block_size);
    const int32_t L = context_lens[s];
    auto it = std::lower_bound(reads.begin(), reads.end(), std::make_pair(b, INT64_MIN));
    for (; it != reads.end() && it->first == b; ++it) {
      const int32_t r = (int32_t)(it->second / max_blocks_per_seq);
      const int64_t j = it->second % max_blocks_per_seq;
      const int64_t pos = j * block_size + off;  // position of the slot in r's context
      if (pos >= context_lens[r]) continue;                // not read by r
      if (r == s && pos == (int64_t)L - 1) continue;       // the writer's own last position
      return PA_ERR_RANGE;
    }
  }
  return PA_OK;
}

}  // extern "C"
