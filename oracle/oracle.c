/*
 * Plain float64 CPU oracle for paged KV-cache decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code, header or constant with the HIP library.
 *
 * Sources (the pages this follows):
 *   [CX] "vLLM 2026 推理引擎全解：从 PagedAttention 到分离式 Prefill"
 *        (chenxutan.com/d/4119.html)
 *          §1.1  decode attention o_t = Attention(q_t, K_{1:t}, V_{1:t});
 *                K and V of past tokens are cached in HBM and re-read.
 *          §2.1  KV split into fixed pages of 16 tokens, pages anywhere in
 *                memory, reached through a logical->physical page table;
 *                several requests may point at one physical page.
 *          §2.2  K-cache layout [num_pages, num_heads, page_size, head_dim];
 *                page lookup page_id = table[logical page] and the in-pool
 *                token address page_id * BLOCK_SIZE + page_offset.
 *   [MJ] vLLM tutorial (mjmagnets.cn/news/49643), §2.2: the attention op
 *        gathers the K and V blocks named by the block table, then computes.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - V uses the same layout as K.
 *   - Grouped heads: query head h reads KV head h / (Hq / Hkv).
 *   - context_lens[s] counts every cached token, the newest included, and
 *     logical token t lives in page table[s][t / 16] at offset t % 16.
 *   - A negative slot in slot_mapping means "no write".
 *   - A zero-length context produces a zero output row.
 *
 * Arithmetic: every stored element is decoded exactly to double (fp32,
 * IEEE binary16 and bfloat16 are all exactly representable), scores and the
 * softmax are formed in double in logical token order.  No blocking, no
 * online rescaling: scores first, then the max, then the weighted sum.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* element type codes understood by the oracle */
enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };

/* status codes */
enum {
  ORC_OK = 0,
  ORC_ERR_ARG = 1,   /* null pointer, bad size or unknown type */
  ORC_ERR_RANGE = 2, /* table entry / length / slot outside its range */
  ORC_ERR_DUP = 3,   /* two tokens written to one slot */
  ORC_ERR_NOMEM = 4
};

static size_t elem_bytes(int dtype) {
  switch (dtype) {
    case ORC_F32: return 4;
    case ORC_F16: return 2;
    case ORC_BF16: return 2;
    default: return 0;
  }
}

/* IEEE 754 binary16 -> double, from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double half_bits_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24); /* subnormal: f * 2^-14 * 2^-10 */
  } else if (e == 31) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(f | 0x400), e - 25); /* (1.f) * 2^(e-15) */
  }
  return sign ? -v : v;
}

/* bfloat16 -> double: bfloat16 is the upper half of an IEEE binary32. */
static double bf16_bits_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double load_elem(const void* base, size_t idx, int dtype) {
  if (dtype == ORC_F32) {
    float f;
    memcpy(&f, (const char*)base + idx * 4, 4);
    return (double)f;
  }
  uint16_t u;
  memcpy(&u, (const char*)base + idx * 2, 2);
  return dtype == ORC_F16 ? half_bits_to_double(u) : bf16_bits_to_double(u);
}

/*
 * The KV-write step ([CX] §1.1: the new token's K and V are stored in HBM;
 * [CX] §2.2: token address = page_id * BLOCK_SIZE + page_offset).
 * For each token i with slot_mapping[i] >= 0:
 *   k_cache[slot / block_size, h, slot % block_size, :] = key[i, h, :]
 * and the same for V.  A byte copy: the cache keeps the key's own type.
 * key/value: [num_tokens, num_kv_heads, head_dim];
 * caches:    [num_blocks, num_kv_heads, block_size, head_dim].
 * Rejects slots beyond the pool and duplicate slots (the pages define no
 * result for two writes to one slot).
 */
int oracle_reshape_and_cache(const void* key, const void* value, void* k_cache,
                             void* v_cache, const int64_t* slot_mapping,
                             int64_t num_tokens, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size,
                             int64_t num_blocks, int32_t dtype) {
  size_t eb = elem_bytes(dtype);
  if (!eb || num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || num_blocks < 0)
    return ORC_ERR_ARG;
  if (num_tokens == 0) return ORC_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return ORC_ERR_ARG;

  const int64_t num_slots = num_blocks * block_size;
  for (int64_t i = 0; i < num_tokens; ++i) {
    int64_t slot = slot_mapping[i];
    if (slot >= num_slots) return ORC_ERR_RANGE;
    if (slot < 0) continue;
    for (int64_t j = 0; j < i; ++j)
      if (slot_mapping[j] == slot) return ORC_ERR_DUP;
  }

  const size_t row = (size_t)head_dim * eb;
  for (int64_t i = 0; i < num_tokens; ++i) {
    int64_t slot = slot_mapping[i];
    if (slot < 0) continue;
    int64_t block = slot / block_size;
    int64_t offset = slot % block_size;
    for (int32_t h = 0; h < num_kv_heads; ++h) {
      size_t src = ((size_t)i * num_kv_heads + h) * row;
      size_t dst = (((size_t)block * num_kv_heads + h) * block_size + offset) * row;
      memcpy((char*)k_cache + dst, (const char*)key + src, row);
      memcpy((char*)v_cache + dst, (const char*)value + src, row);
    }
  }
  return ORC_OK;
}

/*
 * Host check of block tables against the pool: every entry a sequence
 * actually uses (logical pages 0 .. ceil(L/block_size)-1) must name a pool
 * block, and ceil(L/block_size) must fit the table's row.
 */
int oracle_check_tables(const int32_t* block_tables, const int32_t* context_lens,
                        int32_t num_seqs, int32_t max_blocks_per_seq,
                        int64_t num_blocks, int32_t block_size) {
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || block_size <= 0) return ORC_ERR_ARG;
  if (num_seqs > 0 && (!block_tables || !context_lens)) return ORC_ERR_ARG;
  for (int32_t s = 0; s < num_seqs; ++s) {
    int32_t L = context_lens[s];
    if (L < 0) return ORC_ERR_RANGE;
    int64_t pages = ((int64_t)L + block_size - 1) / block_size;
    if (pages > max_blocks_per_seq) return ORC_ERR_RANGE;
    for (int64_t j = 0; j < pages; ++j) {
      int32_t b = block_tables[(size_t)s * max_blocks_per_seq + j];
      if (b < 0 || (int64_t)b >= num_blocks) return ORC_ERR_RANGE;
    }
  }
  return ORC_OK;
}

/*
 * Decode attention ([CX] §1.1) over the paged cache ([CX] §2.1-§2.2,
 * [MJ] §2.2), one output row per requested (sequence, query head) and
 * logical token range [t_begin, t_end):
 *
 *   g   = h / (Hq / Hkv)
 *   b_t = block_tables[s, t / block_size],   r_t = t % block_size
 *   z_t = scale * sum_d q[s, h, d] * k_cache[b_t, g, r_t, d]
 *   m   = max_t z_t
 *   w_t = exp(z_t - m),   l = sum_t w_t
 *   out = sum_t w_t * v_cache[b_t, g, r_t, :] / l
 *
 * rows_t_end[r] < 0 stands for the sequence's context length.  The full
 * decode of a sequence is the range [0, context_lens[s]).  m and l are
 * returned (when the pointers are non-null) so that a split of the range
 * can be checked against the unsplit result; an empty range gives m = -inf,
 * l = 0 and a zero row.
 */
int oracle_decode_rows(double* out, double* out_m, double* out_l, const void* q,
                       const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens,
                       int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size,
                       int32_t max_blocks_per_seq, int64_t num_blocks, double scale,
                       int32_t dtype, const int32_t* rows_seq,
                       const int32_t* rows_head, const int32_t* rows_t_begin,
                       const int32_t* rows_t_end, int64_t num_rows,
                       int32_t num_threads) {
  if (!elem_bytes(dtype) || num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || block_size <= 0 || max_blocks_per_seq <= 0 || num_rows < 0)
    return ORC_ERR_ARG;
  if (num_q_heads % num_kv_heads) return ORC_ERR_ARG;
  if (num_rows == 0) return ORC_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens ||
      !rows_seq || !rows_head || !rows_t_begin || !rows_t_end)
    return ORC_ERR_ARG;

  /* validate every request before computing anything */
  int rc = oracle_check_tables(block_tables, context_lens, num_seqs,
                               max_blocks_per_seq, num_blocks, block_size);
  if (rc) return rc;
  for (int64_t r = 0; r < num_rows; ++r) {
    int32_t s = rows_seq[r], h = rows_head[r];
    if (s < 0 || s >= num_seqs || h < 0 || h >= num_q_heads) return ORC_ERR_RANGE;
    int32_t L = context_lens[s];
    int32_t t0 = rows_t_begin[r];
    int32_t t1 = rows_t_end[r] < 0 ? L : rows_t_end[r];
    if (t0 < 0 || t1 > L || t0 > t1) return ORC_ERR_RANGE;
  }

  const int32_t group = num_q_heads / num_kv_heads;
  const int32_t D = head_dim;
  int status = ORC_OK;

  /* the thread count applies to this call only (a clause, not the
     process-wide default) */
#ifdef _OPENMP
  const int nthr = num_threads > 0 ? num_threads : omp_get_max_threads();
#else
  (void)num_threads;
#endif

#pragma omp parallel num_threads(nthr)
  {
    double* qv = (double*)malloc(sizeof(double) * D);
    double* z = NULL;
    size_t zcap = 0;
    if (!qv) {
#pragma omp atomic write
      status = ORC_ERR_NOMEM;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < num_rows; ++r) {
      if (!qv) continue;
      const int32_t s = rows_seq[r], h = rows_head[r];
      const int32_t L = context_lens[s];
      const int32_t t0 = rows_t_begin[r];
      const int32_t t1 = rows_t_end[r] < 0 ? L : rows_t_end[r];
      const int32_t g = h / group;
      double* o = out + (size_t)r * D;
      for (int32_t d = 0; d < D; ++d) {
        qv[d] = load_elem(q, ((size_t)s * num_q_heads + h) * D + d, dtype);
        o[d] = 0.0;
      }
      const size_t n = (size_t)(t1 - t0);
      if (n == 0) {
        if (out_m) out_m[r] = -INFINITY;
        if (out_l) out_l[r] = 0.0;
        continue;
      }
      if (n > zcap) {
        free(z);
        z = (double*)malloc(sizeof(double) * n);
        zcap = z ? n : 0;
        if (!z) {
#pragma omp atomic write
          status = ORC_ERR_NOMEM;
          continue;
        }
      }
      /* scores, in logical token order */
      for (int32_t t = t0; t < t1; ++t) {
        int64_t b = block_tables[(size_t)s * max_blocks_per_seq + t / block_size];
        size_t base = (((size_t)b * num_kv_heads + g) * block_size + t % block_size) * D;
        double acc = 0.0;
        for (int32_t d = 0; d < D; ++d) acc += qv[d] * load_elem(k_cache, base + d, dtype);
        z[t - t0] = scale * acc;
      }
      double m = -INFINITY;
      for (size_t i = 0; i < n; ++i)
        if (z[i] > m) m = z[i];
      /* softmax weights and the weighted sum of V */
      double l = 0.0;
      for (int32_t t = t0; t < t1; ++t) {
        double w = exp(z[t - t0] - m);
        l += w;
        int64_t b = block_tables[(size_t)s * max_blocks_per_seq + t / block_size];
        size_t base = (((size_t)b * num_kv_heads + g) * block_size + t % block_size) * D;
        for (int32_t d = 0; d < D; ++d) o[d] += w * load_elem(v_cache, base + d, dtype);
      }
      for (int32_t d = 0; d < D; ++d) o[d] /= l;
      if (out_m) out_m[r] = m;
      if (out_l) out_l[r] = l;
    }
    free(qv);
    free(z);
  }
  return status;
}

/*
 * Merge of partial results over disjoint token ranges (the split-K step).
 * Each part p of row r carries m_p = max of its scores, l_p = sum of
 * exp(z - m_p) over it and its normalised output o_p.  Softmax over the
 * union of the ranges is then
 *   M = max_p m_p,  w_p = l_p * exp(m_p - M),  out = sum_p w_p o_p / sum_p w_p,
 * which follows from exp(z - M) = exp(z - m_p) * exp(m_p - M).
 * Parts with l_p = 0 (empty ranges) carry no weight; a row whose parts are
 * all empty gives zeros.
 * Layout: m, l [num_rows, max_parts]; o [num_rows, max_parts, head_dim];
 * num_parts[r] <= max_parts.
 */
int oracle_lse_merge(double* out, const double* m, const double* l, const double* o,
                     const int32_t* num_parts, int64_t num_rows, int32_t max_parts,
                     int32_t head_dim) {
  if (num_rows < 0 || max_parts <= 0 || head_dim <= 0) return ORC_ERR_ARG;
  if (num_rows == 0) return ORC_OK;
  if (!out || !m || !l || !o || !num_parts) return ORC_ERR_ARG;
  for (int64_t r = 0; r < num_rows; ++r)
    if (num_parts[r] < 0 || num_parts[r] > max_parts) return ORC_ERR_RANGE;

  for (int64_t r = 0; r < num_rows; ++r) {
    const int32_t P = num_parts[r];
    const double* mr = m + (size_t)r * max_parts;
    const double* lr = l + (size_t)r * max_parts;
    double* orow = out + (size_t)r * head_dim;
    double M = -INFINITY;
    for (int32_t p = 0; p < P; ++p)
      if (lr[p] > 0.0 && mr[p] > M) M = mr[p];
    for (int32_t d = 0; d < head_dim; ++d) orow[d] = 0.0;
    if (M == -INFINITY) continue;
    double wsum = 0.0;
    for (int32_t p = 0; p < P; ++p) {
      if (!(lr[p] > 0.0)) continue;
      double w = lr[p] * exp(mr[p] - M);
      wsum += w;
      const double* op = o + ((size_t)r * max_parts + p) * head_dim;
      for (int32_t d = 0; d < head_dim; ++d) orow[d] += w * op[d];
    }
    for (int32_t d = 0; d < head_dim; ++d) orow[d] /= wsum;
  }
  return ORC_OK;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
