// Paged attention for several new query tokens per sequence (chunked
// prefill, verification of drafted tokens) on the gfx950 matrix cores.
//
// Query token i of a sequence with n new tokens and a context of L tokens
// (the new ones included, their K/V already in the cache) sits at position
// p = L - n + i and attends to tokens 0 .. p: the decode definition
// o_t = Attention(q_t, K_{1:t}, V_{1:t}) of "vLLM 2026 推理引擎全解"
// (chenxutan.com) §1.1, for several t in one pass (same page, §4.1: the
// target model checks all drafted tokens in one forward pass; vLLM manual
// (doramagic.ai), FlashAttention backend: variable-length attention with
// per-sequence query and key offsets).
//
// Rows of the matrix-core tile (mfma_tile.h) are (query token, query head)
// pairs of one KV head, token-major: row R of (sequence, KV head) is token
// R / G, head kvh * G + R % G.  An item holds some 16-row tiles of one KV
// head and streams the K/V tiles up to the position of its last row once;
// rows whose position ends inside a tile mask the rest of it, and tiles that
// every row sees whole go down the unmasked path.  Two shapes:
//   * multi_query_kernel (up to 32 rows per item): the 4 waves take every
//     4th tile, fold it into all rows, and merge through LDS at the end;
//   * multi_query_wide_kernel (64 or 128 rows): each wave owns 16 or 32 of
//     the rows; the K/V tiles are loaded once per item and shared through
//     LDS, and each wave folds them in runs of several tiles.
// Rows with several partitions leave partials for the log-sum-exp reduce,
// with each query token's causal length beside them.
#include <type_traits>

#include "common.h"
#include "items.h"
#include "launch.h"
#include "mfma_tile.h"

namespace pa {

namespace {

// Workgroup shape: waves and tiles in flight per wave.
constexpr int kMqWaves = 4;
constexpr int kMqDepth = 2;
// Staged tiles a wave of a wide item folds together (fold_group): four with
// one row tile per wave (64-row items: 306 against 314 us on GQA with 8 new
// tokens), two with two row tiles (four spill registers there: 412 against
// 374-380 us with 16 new tokens).
template <int RT>
constexpr int kFoldTiles = RT == 1 ? 4 : 2;

// Fold staged tile jt (`limit` tokens) into a wave's RT row tiles, one row
// tile at a time (folding them side by side needs more registers than two
// waves per SIMD leave).  Row tile r holds rows_t[r] rows whose query
// positions run from pos_first[r] to pos_last[r] (pos_n[r]: this lane's
// row); a row sees the tile's tokens up to its own position.  A row tile
// none of whose rows sees the tile is skipped, one all of whose rows see
// all of it goes unmasked.  All tests are wave-uniform.
template <int DT, int D, int RT>
__device__ __forceinline__ void fold_row_tiles(
    MfmaState<D> (&st)[RT], const u32x4 (&qb)[RT][D / 32], const int (&rows_t)[RT],
    const int (&pos_first)[RT], const int (&pos_last)[RT], const int (&pos_n)[RT],
    const u32x4 (&kt)[D / 32], typename MfmaShape<DT, D>::VT (&vt)[4], int limit, int jt,
    float scale_log2, const MfmaLane& ln) {
  const int t_first = jt * kBlockSize, t_end = t_first + kBlockSize;
  u32x2 vb[D / 16];
  if (limit == kBlockSize)
    v_operands<DT, D, false>(vt, limit, ln, vb);
  else
    v_operands<DT, D, true>(vt, limit, ln, vb);
  static_for<0, RT>([&](auto rc) __attribute__((always_inline)) {
    constexpr int r = decltype(rc)::value;
    if (rows_t[r] == 0 || pos_last[r] < t_first) return;
    if (limit == kBlockSize && pos_first[r] + 1 >= t_end) {
      fold_tile<DT, D, false>(st[r], qb[r], kt, vb, limit, scale_log2, ln);
    } else {
      const int rl = min(limit, max(0, pos_n[r] + 1 - t_first));
      fold_tile<DT, D, true>(st[r], qb[r], kt, vb, rl, scale_log2, ln);
    }
  });
}

// Grid: x = KV head + Hkv * unit (the units of one KV head of a sequence read
// the same tiles; with Hkv a multiple of the 8 XCDs they land on one XCD and
// share its L2), y = sequence slot (longest context first), z = partition.
// An item holds RT 16-row tiles: every staged K/V tile is folded into each.
template <int DT, int D, int NW, int DEPTH, int BS, int RT>
__global__ __launch_bounds__(NW * 64, 2) void multi_query_kernel(MultiQueryArgs ma) {
  using S = MfmaShape<DT, D>;
  using VT = typename S::VT;
  constexpr int EPL = S::EPL;
  __shared__ MfmaLds<D, NW> sm;
  __shared__ u32x4 kst_all[NW][kKStageSlots<D>];
  const DecodeArgs& a = ma.d;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int kvh = blockIdx.x % a.num_kv_heads, unit = blockIdx.x / a.num_kv_heads;
  const int s = longest_first(a, blockIdx.y), part = blockIdx.z;
  const int L = clamp_len(a, s);

  // Query tokens of s, kept inside [0, T) and to max_query_len.
  const int T = ma.num_query_tokens;
  const int t0 = ma.query_start[s];
  int nq = ma.query_start[s + 1] - t0;
  nq = (t0 < 0 || t0 > T) ? 0 : max(0, min(nq, min(ma.max_query_len, T - t0)));
  const int base_pos = L - nq;  // position of query token 0
  if (ma.token_lens != nullptr && kvh == 0 && unit == 0 && part == 0)
    for (int i = threadIdx.x; i < nq; i += NW * 64) ma.token_lens[t0 + i] = max(base_pos + i + 1, 0);

  const int r0 = unit * 16 * RT;
  if (r0 >= nq * G) return;  // past this sequence's rows
  const int rows = min(16 * RT, nq * G - r0);
  const int span = max(base_pos + (r0 + rows - 1) / G + 1, 0);  // tokens the item reads
  const int nblocks = (span + kBlockSize - 1) / kBlockSize;
  if (part >= parts_of(span, a.part_blocks)) return;

  const MfmaLane ln;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  u32x4* kst = kst_all[w];
  // Row tile r: rows r0 + 16 r + n.  Per lane (row n of each tile) the
  // position of its query token (idle rows take the tile's last row's, so
  // they never narrow the unmasked test) and its q slices.
  int rows_t[RT], pos_first[RT], pos_last[RT], pos_n[RT];
  u32x4 qb[RT][S::NJ];
  const u32x4* q = reinterpret_cast<const u32x4*>(a.q);
  static_for<0, RT>([&](auto rc) __attribute__((always_inline)) {
    constexpr int r = decltype(rc)::value;
    const int rb = r0 + 16 * r;
    rows_t[r] = max(0, min(16, rows - 16 * r));
    pos_first[r] = base_pos + rb / G;
    pos_last[r] = base_pos + (rb + max(rows_t[r] - 1, 0)) / G;
    const bool active = ln.n < rows_t[r];
    const int rn = rb + (active ? ln.n : max(rows_t[r] - 1, 0));
    pos_n[r] = base_pos + rn / G;
    const int64_t qrow = (int64_t)(t0 + rn / G) * a.num_q_heads + kvh * G + rn % G;
#pragma unroll
    for (int jj = 0; jj < S::NJ; ++jj)
      qb[r][jj] = active ? q[qrow * S::CPR + 4 * jj + ln.g] : u32x4{0u, 0u, 0u, 0u};
  });

  const int32_t* __restrict__ bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  const int jb = part * a.part_blocks;
  const int je = min(jb + a.part_blocks, nblocks);
  const int j0 = jb + w;                                   // tiles j0, j0 + NW, ...
  const int nk = je > j0 ? (je - j0 + NW - 1) / NW : 0;   // how many

  MfmaState<D> st[RT];
  static_for<0, RT>([&](auto rc) __attribute__((always_inline)) { st[decltype(rc)::value].reset(); });

  const TableRow btc = table_row(bt);
  auto id_at = [&](int kk) __attribute__((always_inline)) {
    return tile_ids<BS>(btc, j0 + min(kk, nk - 1) * NW, a.max_blocks_per_seq);
  };
  // Descriptors of the wave's kk-th tile, its index and its token count
  // (tokens up to the item's last position, inside the pool).
  auto tile = [&](int kk, const TileIds<BS>& ids, int& limit, int& jt) __attribute__((always_inline)) {
    jt = j0 + min(kk, nk - 1) * NW;
    const bool ok = kk < nk;
    limit = ok ? tile_limit<BS>(a, ids, span - jt * kBlockSize) : 0;
    return tile_desc<BS, S::TILE_BYTES>(a, ids, jt, kvh, ok);
  };
  // (The lambdas here are forced inline: a call would leave everything they
  // capture in scratch memory.)
  // Stage tile jt's K once, then fold it into the row tiles.
  auto consume = [&](u32x4 (&kr)[S::NJ], VT (&vr)[4], int limit,
                     int jt) __attribute__((always_inline)) {
    stage_k<D>(kst, kr, ln);
    fold_row_tiles<DT, D, RT>(st, qb, rows_t, pos_first, pos_last, pos_n, kr, vr, limit, jt,
                              a.scale_log2, ln);
  };

  // Software pipeline as in decode: DEPTH register sets, loads issued on
  // every step (empty past the end) so the wait counts never branch.
  u32x4 kr[DEPTH][S::NJ];
  VT vr[DEPTH][4];
  int lim[DEPTH], jts[DEPTH];
  auto pipeline = [&](auto shared) __attribute__((always_inline)) {
    constexpr bool SH = decltype(shared)::value;
    static_for<0, DEPTH - 1>([&](auto dc) __attribute__((always_inline)) {
      constexpr int d = decltype(dc)::value;
      load_tile<DT, D, SH>(tile(d, id_at(d), lim[d], jts[d]), ln, kr[d], vr[d]);
    });
    TileIds<BS> next_id = id_at(DEPTH - 1);
    for (int k = 0; k < nk; k += DEPTH) {
      static_for<0, DEPTH>([&](auto dc) __attribute__((always_inline)) {
        constexpr int d = decltype(dc)::value;
        constexpr int dn = (d + DEPTH - 1) % DEPTH;
        const int kn = k + d + DEPTH - 1;
        const TileIds<BS> id = next_id;
        next_id = id_at(kn + 1);
        load_tile<DT, D, SH>(tile(kn, id, lim[dn], jts[dn]), ln, kr[dn], vr[dn]);
        consume(kr[d], vr[d], lim[d], jts[d]);
      });
    }
  };
  if (nk > 0) {
    // Tiles read again soon -- by the other units of this KV head, or by the
    // neighbouring sequence when it maps the same first block -- load with
    // the cache-allocating policy; the rest stream past the caches.
    const int32_t* nb = a.num_seqs > 1 ? a.block_tables +
                            (int64_t)(s > 0 ? s - 1 : s + 1) * a.max_blocks_per_seq : nullptr;
    const bool reread = nq * G > 16 * RT ||
                        (nb != nullptr && tile_ids<BS>(nb, j0, a.max_blocks_per_seq).id[0] ==
                                              tile_ids<BS>(bt, j0, a.max_blocks_per_seq).id[0]);
    if (reread)
      pipeline(std::true_type{});
    else
      pipeline(std::false_type{});
  }

  // Per row tile: this wave's per-row totals, then the cross-wave merge
  // through LDS (one tile at a time, reusing the same LDS).
  const int n = ln.n, g = ln.g;
  static_for<0, RT>([&](auto rc) __attribute__((always_inline)) {
    constexpr int r = decltype(rc)::value;
    if (rows_t[r] == 0) return;  // uniform over the workgroup
    if (r > 0) __syncthreads();  // the previous tile's readers are done
    float lsum = xor16_combine(st[r].lsum, AddOp{});
    lsum = xor32_combine(lsum, AddOp{});
    if (g == 0) {
      sm.m[w][n] = st[r].m;
      sm.l[w][n] = lsum;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int jj = 0; jj < EPL; ++jj) sm.o[w][4 * g + e][EPL * n + jj] = st[r].o[jj][e];
    __syncthreads();
    if (threadIdx.x < 16) {
      const int hh = threadIdx.x;
      float M = -INFINITY;
#pragma unroll
      for (int i = 0; i < NW; ++i) M = __builtin_fmaxf(M, sm.m[i][hh]);
      float tot = 0.f;
      float f[NW];
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        f[i] = (sm.m[i][hh] == -INFINITY) ? 0.f : fast_exp2(sm.m[i][hh] - M);
        tot += sm.l[i][hh] * f[i];
      }
      const float inv = tot > 0.f ? 1.f / tot : 0.f;
#pragma unroll
      for (int i = 0; i < NW; ++i) sm.f[i][hh] = f[i] * inv;
      sm.tot[hh] = tot;
      sm.mx[hh] = M;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < rows_t[r] * D; i += NW * 64) {
      const int hh = i / D, d = i % D;
      const int R = r0 + 16 * r + hh, tok = R / G;
      // partitions of this row's own causal span; later ones are not its
      const int row_parts = parts_of(max(base_pos + tok + 1, 0), a.part_blocks);
      if (part >= row_parts) continue;
      float v = 0.f;
#pragma unroll
      for (int k = 0; k < NW; ++k) v += sm.o[k][hh][d] * sm.f[k][hh];
      const int64_t orow = (int64_t)(t0 + tok) * a.num_q_heads + kvh * G + R % G;
      if (row_parts <= 1) {
        store_elem<DT>(a.out, orow * D + d, v);
      } else {
        const int64_t prow = orow * a.max_partitions + part;
        a.tmp_out[prow * D + d] = v;
        if (d == 0) {
          a.max_logits[prow] = sm.mx[hh] * kLn2;
          a.exp_sums[prow] = sm.tot[hh];
        }
      }
    }
  });
}

// One staged tile of the wide kernel in LDS.  K and V rows keep their
// 16-byte chunks permuted within the row (kswz), so the column-wise operand
// reads of 16 rows spread over the banks.  The kernel keeps its two buffers
// of NW tiles in two separate LDS variables and names the one it touches at
// compile time: the compiler can then tell the loads into one buffer from
// the reads of the other, instead of waiting for every load in flight before
// a read.
template <int D>
struct WideTile {
  u32x4 k[kBlockSize * D / 8];  // 16-byte chunk c of row r at r * D/8 + (c ^ r % (D/8))
  u32x4 v[kBlockSize * D / 8];  // the same layout for V
};

// Position of K chunk c of token row r in a wide tile: chunks are permuted
// within each row so that the S operand reads (16 rows, one chunk each, for
// one contraction slice) fall on distinct banks.
template <int D>
__device__ __forceinline__ int kswz(int r, int c) {
  constexpr int CPR = D / 8;
  return r * CPR + (c ^ (r % CPR));
}

// 16-byte buffer load of each lane straight into LDS: lane l writes the
// 16 bytes at dst + 16 l (dst wave-uniform).  The builtin exists only for
// the device pass; the host pass (which instantiates the kernel templates
// for their launch stubs) sees an empty body.
template <int AUX>
__device__ __forceinline__ void load16_to_lds(Rsrc r, u32x4* dst, int voffset) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16,
                                           voffset, 0, 0, AUX);
#endif
}

// Transposing LDS read (gfx950): within each 16-lane group, lane i receives
// [x_0[i % 4], x_1[i % 4], x_2[i % 4], x_3[i % 4]] where x_k is the 8 bytes
// (four 16-bit elements) that lane 4k + i / 4 of the group addresses -- the
// lane layout was checked on the device.  It turns four token rows into
// one column of four tokens per lane, the B operand of the P.V products.
__device__ __forceinline__ u32x2 lds_read_tr16(const void* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(const_cast<void*>(p)));
  return __builtin_bit_cast(u32x2, v);
#else
  (void)p;
  return u32x2{0u, 0u};
#endif
}

// Wait for this wave's loads into LDS to land.
__device__ __forceinline__ void wait_lds_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Fold NT staged tiles (tile t of `tiles`: tokens g_first + 16 t + 0..15,
// lims[t] of them valid) into a wave's RT row tiles at once: the scores of
// all NT * 16 tokens first, then one max reduction and one rescale test per
// row tile, the exponentials, and the P.V products -- over pairs of tiles
// as 16x16x32 products.  No branch separates the row
// tiles, so their matrix-core chains interleave.  MASKED: a token counts for
// row n when it is one of its tile's valid tokens and not past the row's
// position pos_n; rows that see none of the group add nothing.  Scores stay
// raw until the exponent (one fma per score: scale * s - max); scale_log2
// must be >= 0 (the caller turns a negative scale into a negated query).
template <int DT, int D, int NT, int RT, bool MASKED, typename Tile>
__device__ __forceinline__ void fold_group(MfmaState<D> (&st)[RT],
                                           const u32x4 (&qb)[RT][D / 32],
                                           const int (&pos_n)[RT], const Tile* tiles,
                                           const int (&lims)[NT], int g_first,
                                           float scale_log2, const MfmaLane& ln) {
  using S = MfmaShape<DT, D>;
  const int lane = ln.n + 16 * ln.g;
  float sc[RT][NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    u32x4 kt[S::NJ];
#pragma unroll
    for (int jj = 0; jj < S::NJ; ++jj) kt[jj] = tiles[t].k[kswz<D>(ln.tok_k, 4 * jj + ln.g)];
    f32x4 sacc[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) sacc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < S::NJ; ++jj)
#pragma unroll
      for (int r = 0; r < RT; ++r) sacc[r] = mfma_qk<DT>(kt[jj], qb[r][jj], sacc[r]);
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sc[r][t][e] = sacc[r][e];  // raw; the scale goes into the exponent's fma
        if constexpr (MASKED) {
          const int k = ln.g + 4 * e;
          const bool ok = k < lims[t] && g_first + kBlockSize * t + k <= pos_n[r];
          sc[r][t][e] = ok ? sc[r][t][e] : -INFINITY;
        }
      }
  }
  float mb[RT];
  bool grow = false;
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    float x = sc[r][0][0];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) x = max_nn(x, sc[r][t][e]);
    mb[r] = xor16_combine(x, MaxNnOp{});
  }
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    // the largest raw score, scaled (scale_log2 >= 0 keeps it the largest)
    const float mr = xor32_combine(mb[r], MaxNnOp{});
    mb[r] = mr == -INFINITY ? -INFINITY : mr * scale_log2;
    grow = grow || mb[r] > st[r].m + (kRescaleSlack + kMaxOffset<DT>);
  }
  // The running max moves once a score passes it by more than
  // kRescaleSlack (weights stay below 2^kRescaleSlack; for f16 the reference
  // sits kF16MaxOffset below the largest score).  Wave-uniform: a rescale to
  // a larger max never changes the result, so all row tiles take it.
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const float mn = max_nn(st[r].m, mb[r] - kMaxOffset<DT>);
      const float alpha = mn == -INFINITY ? 1.f : fast_exp2(st[r].m - mn);
      st[r].lsum *= alpha;
      st[r].m = mn;
      float arow[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        arow[e] =
            u2f((uint32_t)__builtin_amdgcn_ds_bpermute((4 * ln.g + e) << 2, (int)f2u(alpha)));
#pragma unroll
      for (int jj = 0; jj < S::EPL; ++jj)
#pragma unroll
        for (int e = 0; e < 4; ++e) st[r].o[jj][e] *= arow[e];
    }
  }
  // bf16 weights also carry their residuals (a second P.V product): one
  // weight's 8-bit rounding moves the output by up to 2^-9 of the spread of
  // V, past the 1e-2 bound in the tail of N(0,1) data (see fold_tile).
  constexpr bool SPLIT = DT == kBF16;
  u32x2 pa[RT][NT], pl[RT][NT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const bool none = MASKED && st[r].m == -INFINITY;  // no valid token of this row so far
    float sum = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[e] = fast_exp2(__builtin_fmaf(sc[r][t][e], scale_log2, -st[r].m));
        // dropped tokens (and rows with none so far) weigh nothing, also when
        // the scale is 0 (-inf * 0 is not -inf)
        if constexpr (MASKED) p[e] = (none || sc[r][t][e] == -INFINITY) ? 0.f : p[e];
      }
      pa[r][t] = u32x2{pack2<DT>(p[0], p[1]), pack2<DT>(p[2], p[3])};
      sum = packed_sum<DT>(pa[r][t], sum);  // the weights as rounded for P.V
      if constexpr (SPLIT) {
        pl[r][t] = residual_pack<DT>(p, pa[r][t]);
        sum = packed_sum<DT>(pl[r][t], sum);
      }
    }
    st[r].lsum += sum;
  }
  // P.V over pairs of tiles: the two tiles' 4 + 4 tokens of a lane are one
  // 8-wide contraction slice of a 16x16x32 product (P and V take the tokens
  // in the same order), half the instructions of two 16x16x16 products.
  // Product jj gives output dims 16 jj + n.  Its V operand -- tokens
  // g + 4k (k = 0..3) of dim 16 jj + n, per tile -- comes straight out of
  // LDS through the transposing read: lane 4k + q of a 16-lane group
  // addresses row g + 4k, dims 16 jj + 4q .. + 3.
  static_assert(NT % 2 == 0, "tiles are folded in pairs");
  constexpr int CPR = D / 8;
  const int tr_row = ln.g + 4 * ((lane & 15) >> 2), tr_q = lane & 3;
  // byte offset in a tile of this lane's 8 bytes for product jj (kswz layout)
  auto tr_off = [&](int jj) {
    const int c = 2 * jj + (tr_q >> 1);
    return (tr_row * CPR + (c ^ (tr_row % CPR))) * 16 + (tr_q & 1) * 8;
  };
#pragma unroll
  for (int t = 0; t < NT; t += 2) {
    u32x4 pp[RT], ppl[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      pp[r] = u32x4{pa[r][t][0], pa[r][t][1], pa[r][t + 1][0], pa[r][t + 1][1]};
      if constexpr (SPLIT)
        ppl[r] = u32x4{pl[r][t][0], pl[r][t][1], pl[r][t + 1][0], pl[r][t + 1][1]};
    }
#pragma unroll
    for (int jj = 0; jj < D / 16; ++jj) {
      u32x2 v0 = lds_read_tr16(reinterpret_cast<const char*>(tiles[t].v) + tr_off(jj));
      u32x2 v1 = lds_read_tr16(reinterpret_cast<const char*>(tiles[t + 1].v) + tr_off(jj));
      if constexpr (MASKED) {
        // what the slots past a tile's tokens hold must not reach P.V:
        // element k of this lane is token g + 4k
        const uint32_t m0 = (ln.g < lims[t] ? 0xffffu : 0u) | (ln.g + 4 < lims[t] ? 0xffff0000u : 0u);
        const uint32_t m1 = (ln.g + 8 < lims[t] ? 0xffffu : 0u) | (ln.g + 12 < lims[t] ? 0xffff0000u : 0u);
        const uint32_t n0 = (ln.g < lims[t + 1] ? 0xffffu : 0u) | (ln.g + 4 < lims[t + 1] ? 0xffff0000u : 0u);
        const uint32_t n1 = (ln.g + 8 < lims[t + 1] ? 0xffffu : 0u) | (ln.g + 12 < lims[t + 1] ? 0xffff0000u : 0u);
        v0 = u32x2{v0[0] & m0, v0[1] & m1};
        v1 = u32x2{v1[0] & n0, v1[1] & n1};
      }
      const u32x4 vb{v0[0], v0[1], v1[0], v1[1]};
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        st[r].o[jj] = mfma_qk<DT>(pp[r], vb, st[r].o[jj]);
        if constexpr (SPLIT) st[r].o[jj] = mfma_qk<DT>(ppl[r], vb, st[r].o[jj]);
      }
    }
  }
}

// Wide items: many query rows per KV head (long spans, large head groups).
// Each of the NW waves owns RT 16-row tiles of the item (up to NW * RT * 16
// rows) and folds every tile of the partition into them; the K/V tiles are
// loaded once per item, each wave loading one tile of every group of NW
// straight into double-buffered LDS (buffer loads with the LDS destination:
// no registers hold tiles in flight; one barrier per group), and read by
// all waves kFoldTiles<RT> at a time (fold_group: one max reduction and rescale
// test per run of tiles, row tiles interleaved).  A wave's rows are
// complete in its registers at the end: no merge.
template <int DT, int D, int NW, int BS, int RT>
__global__ __launch_bounds__(NW * 64, 2) void multi_query_wide_kernel(MultiQueryArgs ma) {
  using S = MfmaShape<DT, D>;
  using VT = typename S::VT;
  constexpr int EPL = S::EPL;
  constexpr int ROWS = NW * RT * 16;
  __shared__ WideTile<D> buf0[NW], buf1[NW];
  const DecodeArgs& a = ma.d;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int kvh = blockIdx.x % a.num_kv_heads, unit = blockIdx.x / a.num_kv_heads;
  const int s = longest_first(a, blockIdx.y), part = blockIdx.z;
  const int L = clamp_len(a, s);

  const int T = ma.num_query_tokens;
  const int t0 = ma.query_start[s];
  int nq = ma.query_start[s + 1] - t0;
  nq = (t0 < 0 || t0 > T) ? 0 : max(0, min(nq, min(ma.max_query_len, T - t0)));
  const int base_pos = L - nq;
  if (ma.token_lens != nullptr && kvh == 0 && unit == 0 && part == 0)
    for (int i = threadIdx.x; i < nq; i += NW * 64) ma.token_lens[t0 + i] = max(base_pos + i + 1, 0);

  const int r0 = unit * ROWS;
  if (r0 >= nq * G) return;  // past this sequence's rows
  const int rows = min(ROWS, nq * G - r0);
  const int span = max(base_pos + (r0 + rows - 1) / G + 1, 0);
  const int nblocks = (span + kBlockSize - 1) / kBlockSize;
  if (part >= parts_of(span, a.part_blocks)) return;

  const MfmaLane ln;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // This wave's row tiles: rows r0 + 16 (w RT + r) + n.
  int rows_t[RT], pos_first[RT], pos_last[RT], pos_n[RT];
  u32x4 qb[RT][S::NJ];
  MfmaState<D> st[RT];
  const u32x4* q = reinterpret_cast<const u32x4*>(a.q);
  static_for<0, RT>([&](auto rc) __attribute__((always_inline)) {
    constexpr int r = decltype(rc)::value;
    const int rb = r0 + 16 * (w * RT + r);
    rows_t[r] = max(0, min(16, rows - 16 * (w * RT + r)));
    pos_first[r] = base_pos + rb / G;
    pos_last[r] = base_pos + (rb + max(rows_t[r] - 1, 0)) / G;
    const bool active = ln.n < rows_t[r];
    const int rn = rb + (active ? ln.n : max(rows_t[r] - 1, 0));
    pos_n[r] = base_pos + rn / G;
    const int64_t qrow = (int64_t)(t0 + rn / G) * a.num_q_heads + kvh * G + rn % G;
#pragma unroll
    for (int jj = 0; jj < S::NJ; ++jj)
      qb[r][jj] = active ? q[qrow * S::CPR + 4 * jj + ln.g] : u32x4{0u, 0u, 0u, 0u};
    st[r].reset();
  });
  // fold_group takes a non-negative scale: scale * (q.k) = |scale| * ((-q).k),
  // and flipping the sign bits of the 16-bit q elements negates q exactly.
  const float sl = __builtin_fabsf(a.scale_log2);
  if (a.scale_log2 < 0.f) {
    static_for<0, RT>([&](auto rc) __attribute__((always_inline)) {
      constexpr int r = decltype(rc)::value;
#pragma unroll
      for (int jj = 0; jj < S::NJ; ++jj) qb[r][jj] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
    });
  }

  const int32_t* __restrict__ bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  const int jb = part * a.part_blocks;
  const int je = min(jb + a.part_blocks, nblocks);
  const int ngroups = je > jb ? (je - jb + NW - 1) / NW : 0;
  // Tile of group g this wave loads (index clamped into the item).
  // Every wave reads the block ids of all NW tiles of a group (scalar loads,
  // two groups ahead): it loads its own tile and knows every tile's token
  // count without a round trip through LDS.
  const TableRow btc = table_row(bt);
  struct GroupIds {
    TileIds<BS> t[NW];
  };
  auto ids_at = [&](int g) __attribute__((always_inline)) {
    GroupIds r;
#pragma unroll
    for (int t = 0; t < NW; ++t)
      r.t[t] = tile_ids<BS>(btc, min(jb + g * NW + t, je - 1), a.max_blocks_per_seq);
    return r;
  };
  // the wave's own tile of group g (a load of its own: picking it out of a
  // GroupIds by the wave index would index an array at run time)
  auto id_at = [&](int g) __attribute__((always_inline)) {
    return tile_ids<BS>(btc, min(jb + g * NW + w, je - 1), a.max_blocks_per_seq);
  };
  // LDS buffer B (0 or 1, known at compile time).
  auto buffer = [&](auto bc) __attribute__((always_inline)) {
    if constexpr (decltype(bc)::value == 0)
      return buf0;
    else
      return buf1;
  };
  // This wave's tile of group g into LDS buffer bc.
  auto load = [&](int g, const TileIds<BS>& ids, auto bc) __attribute__((always_inline)) {
    WideTile<D>* const dst = buffer(bc) + w;
    const int jt = jb + g * NW + w;
    const bool ok = g < ngroups && jt < je;
    const TileDesc<BS, S::TILE_BYTES> desc = tile_desc<BS, S::TILE_BYTES>(a, ids, jt, kvh, ok);
    // Buffer loads with the LDS destination: lane l of a load writes the 16
    // bytes at slot 64 jj + l of the load's KiB, no registers involved.  A K
    // load's lane fetches the chunk kswz puts at its slot; V keeps row order.
    // Which block part a load reads is known at compile time, as in load_tile.
    using Desc = TileDesc<BS, S::TILE_BYTES>;
    static_for<0, S::NJ>([&](auto jc) __attribute__((always_inline)) {
      constexpr int jj = decltype(jc)::value;
      constexpr int h = Desc::part(jj * 1024);
      const int p = jj * 64 + lane;
      const int r = p / S::CPR, c = (p % S::CPR) ^ (r % S::CPR);
      const int koff = (r * S::CPR + c) * 16 - h * Desc::HB, voff = koff;  // both kswz
      if (ma.reread) {
        load16_to_lds<PA_SHARED_LOAD_POLICY>(desc.k[h], dst->k + jj * 64, koff);
        load16_to_lds<PA_SHARED_LOAD_POLICY>(desc.v[h], dst->v + jj * 64, voff);
      } else {
        load16_to_lds<PA_KV_LOAD_POLICY>(desc.k[h], dst->k + jj * 64, koff);
        load16_to_lds<PA_KV_LOAD_POLICY>(desc.v[h], dst->v + jj * 64, voff);
      }
    });
  };

  GroupIds ids_g;
  TileIds<BS> next_id;
  // Group g, held in buffer bc: load group g + 1 into the other buffer, fold
  // group g, wait for the wave's own loads and meet the other waves.
  auto step = [&](int g, auto bc) __attribute__((always_inline)) {
      constexpr int B = decltype(bc)::value;
      WideTile<D>* const tiles = buffer(bc);
      const TileIds<BS> id = next_id;
      next_id = id_at(g + 2);
      // the other buffer was last read before the previous barrier
      load(g + 1, id, std::integral_constant<int, 1 - B>{});
      const int g_first = (jb + g * NW) * kBlockSize;  // first token of the group
      int lims[NW];
#pragma unroll
      for (int t = 0; t < NW; ++t) {
        const int jt = jb + g * NW + t;
        lims[t] = jt < je ? tile_limit<BS>(a, ids_g.t[t], span - jt * kBlockSize) : 0;
      }
      ids_g = ids_at(g + 1);
      bool any = false, whole = true;
#pragma unroll
      for (int t = 0; t < NW; ++t) whole = whole && lims[t] == kBlockSize;
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        any = any || (rows_t[r] > 0 && pos_last[r] >= g_first);
        whole = whole && (rows_t[r] == 0 || pos_first[r] + 1 >= g_first + NW * kBlockSize);
      }
      // the group in runs of FT tiles (registers: FT * 16 scores per row tile)
      if (any) {
        constexpr int FT = kFoldTiles<RT>;
        static_assert(NW % FT == 0, "a group is folded in whole runs");
        static_for<0, NW / FT>([&](auto hc) __attribute__((always_inline)) {
          constexpr int t0 = decltype(hc)::value * FT;
          const int(&lh)[FT] = *reinterpret_cast<const int(*)[FT]>(&lims[t0]);
          if (whole)
            fold_group<DT, D, FT, RT, false>(st, qb, pos_n, tiles + t0, lh,
                                             g_first + t0 * kBlockSize, sl, ln);
          else
            fold_group<DT, D, FT, RT, true>(st, qb, pos_n, tiles + t0, lh,
                                            g_first + t0 * kBlockSize, sl, ln);
        });
      }
      wait_lds_loads();
      __syncthreads();  // group g + 1 in the other buffer; every wave done with this one
  };
  if (ngroups > 0) {
    load(0, id_at(0), std::integral_constant<int, 0>{});
    ids_g = ids_at(0);
    next_id = id_at(1);
    wait_lds_loads();
    __syncthreads();
    for (int g = 0; g < ngroups; g += 2) {
      step(g, std::integral_constant<int, 0>{});
      if (g + 1 < ngroups) step(g + 1, std::integral_constant<int, 1>{});
    }
  }

  // Each wave writes its own rows: output row 4g+e of a row tile, dims
  // 16 jj + n (the P.V result layout).
  static_for<0, RT>([&](auto rc) __attribute__((always_inline)) {
    constexpr int r = decltype(rc)::value;
    if (rows_t[r] == 0) return;
    const int rb = r0 + 16 * (w * RT + r);
    float lsum = xor16_combine(st[r].lsum, AddOp{});
    lsum = xor32_combine(lsum, AddOp{});
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int hh = 4 * ln.g + e;
      const float lr = u2f((uint32_t)__builtin_amdgcn_ds_bpermute(hh << 2, (int)f2u(lsum)));
      if (hh >= rows_t[r]) continue;
      const int R = rb + hh, tok = R / G;
      const int row_parts = parts_of(max(base_pos + tok + 1, 0), a.part_blocks);
      if (part >= row_parts) continue;
      const float inv = lr > 0.f ? 1.f / lr : 0.f;
      const int64_t orow = (int64_t)(t0 + tok) * a.num_q_heads + kvh * G + R % G;
      if (row_parts <= 1) {
#pragma unroll
        for (int jj = 0; jj < EPL; ++jj)
          store_elem<DT>(a.out, orow * D + 16 * jj + ln.n, st[r].o[jj][e] * inv);
      } else {
        const int64_t prow = orow * a.max_partitions + part;
#pragma unroll
        for (int jj = 0; jj < EPL; ++jj) a.tmp_out[prow * D + 16 * jj + ln.n] = st[r].o[jj][e] * inv;
      }
    }
    // per-row max and sum of the partial, from the lanes holding row n
    if (ln.g == 0 && ln.n < rows_t[r]) {
      const int R = rb + ln.n, tok = R / G;
      const int row_parts = parts_of(max(base_pos + tok + 1, 0), a.part_blocks);
      if (row_parts > 1 && part < row_parts) {
        const int64_t prow =
            ((int64_t)(t0 + tok) * a.num_q_heads + kvh * G + R % G) * a.max_partitions + part;
        a.max_logits[prow] = st[r].m * kLn2;
        a.exp_sums[prow] = lsum;
      }
    }
  });
}

template <int DT, int D, int BS>
hipError_t launch_bs(const MultiQueryArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)(a.d.num_kv_heads * a.units), (unsigned)a.d.num_seqs,
                  (unsigned)a.d.max_partitions);
  if (a.wide && a.row_tiles == 2)
    hipLaunchKernelGGL((multi_query_wide_kernel<DT, D, 4, BS, 2>), grid, dim3(4 * 64), 0, stream,
                       a);
  else if (a.wide)
    hipLaunchKernelGGL((multi_query_wide_kernel<DT, D, 4, BS, 1>), grid, dim3(4 * 64), 0, stream,
                       a);
  else if (a.row_tiles == 2)
    hipLaunchKernelGGL((multi_query_kernel<DT, D, kMqWaves, kMqDepth, BS, 2>), grid,
                       dim3(kMqWaves * 64), 0, stream, a);
  else
    hipLaunchKernelGGL((multi_query_kernel<DT, D, kMqWaves, kMqDepth, BS, 1>), grid,
                       dim3(kMqWaves * 64), 0, stream, a);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_typed(const MultiQueryArgs& a, hipStream_t stream) {
  switch (a.d.block_size) {
    case 8: return launch_bs<DT, D, 8>(a, stream);
    case 32: return launch_bs<DT, D, 32>(a, stream);
    default: return launch_bs<DT, D, 16>(a, stream);
  }
}

}  // namespace

hipError_t launch_multi_query(const MultiQueryArgs& a, int dtype, int head_dim,
                              hipStream_t stream) {
  clear_stale_error();
  switch (dtype * 1000 + head_dim) {
    case kF16 * 1000 + 64: return launch_typed<kF16, 64>(a, stream);
    case kF16 * 1000 + 128: return launch_typed<kF16, 128>(a, stream);
    case kBF16 * 1000 + 64: return launch_typed<kBF16, 64>(a, stream);
    case kBF16 * 1000 + 128: return launch_typed<kBF16, 128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
