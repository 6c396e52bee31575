// Matrix-core tile primitives shared by the decode and shared-prefix kernels.
//
// Per 16-token block and KV head, with up to 16 query rows sharing the tile
// (the G query heads of a KV head, or the same head of sequences that share
// the block): S = K_blk (16 x D) . Q^T (D x 16 rows) and
// O += P (16 rows x 16 tokens) . V_blk (16 x D), both on MFMA:
//   S:  v_mfma_f32_16x16x32_{bf16,f16}, D/32 of them (rows = tokens,
//       columns = query rows, contraction over head_dim);
//   PV: v_mfma_f32_16x16x16_f16, D/16 of them (rows = query rows,
//       columns = output dims, contraction over the block's 16 tokens); for
//       bf16 v_mfma_f32_16x16x32_bf16 over the weights and their residuals
//       against the same V rows twice (fold_tile).
//
// Lane layouts (wave64, lane l, n = l % 16, g = l / 16):
//   MFMA 16x16xK operand A: row n, contraction slice g;  B: column n, slice g;
//   16x16 result: column n, rows 4g .. 4g+3.
// Orders are chosen so that the products chain without moving data:
//   * result row r of S stands for token tau(r) = r/4 + 4 (r%4), so lane l
//     ends up with the scores of tokens g + 4e (e = 0..3) for query row n --
//     exactly the P operand layout of the PV product (row = query row n,
//     contraction slice g = tokens g + 4e);
//   * the PV contraction over tokens uses the same order, so lane l needs
//     V rows g + 4e: four wave-wide loads of 4 whole rows each (coalesced 1 KiB
//     per instruction at D = 128), and output column n of PV product jj is
//     dim EPL*n + jj, the elements the lane loaded;
//   * the S contraction over head_dim visits 16-byte chunk 4j + g of a row in
//     product j (Q is read in the same order).  K is loaded as whole
//     contiguous KiB runs and reaches that layout through a per-wave LDS tile.
// Online softmax runs per query row in base 2; the running max of a row lives
// in the 4 lanes with that n, the output rows 4g..4g+3 fetch their rescale
// factor with a lane shuffle.
#pragma once

#include <type_traits>

#include "common.h"
#include "items.h"
#include "launch.h"

namespace pa {

template <int DT>
__device__ __forceinline__ f32x4 mfma_qk(const u32x4& a, const u32x4& b, const f32x4& c) {
  if constexpr (DT == kBF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <int DT>
__device__ __forceinline__ f32x4 mfma_pv(const u32x2& a, const u32x2& b, const f32x4& c) {
  if constexpr (DT == kBF16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                     __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

// Two floats -> packed pair of 16-bit elements (round to nearest even; one
// v_cvt_pk_{f16,bf16}_f32).
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  if constexpr (DT == kBF16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
}

// acc + the two 16-bit elements of w (a dot product with (1, 1): the
// products are exact).
template <int DT>
__device__ __forceinline__ float add_pair(uint32_t w, float acc) {
  if constexpr (DT == kBF16)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                           __builtin_bit_cast(bf16x2, 0x3f803f80u), acc, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), __builtin_bit_cast(f16x2, 0x3c003c00u),
                                  acc, false);
}

// The residuals p[e] - (p[e] as packed in pa), packed the same way: the
// subtraction is exact in fp32, so pa + residual holds each weight to about
// twice the 16-bit precision.
template <int DT>
__device__ __forceinline__ u32x2 residual_pack(const float (&p)[4], const u32x2& pa) {
  float r[4];
  unpack2<DT>(pa[0], r[0], r[1]);
  unpack2<DT>(pa[1], r[2], r[3]);
  return u32x2{pack2<DT>(p[0] - r[0], p[1] - r[1]), pack2<DT>(p[2] - r[2], p[3] - r[3])};
}

// acc + the four 16-bit weights of a packed P operand, exactly the values the
// matrix core multiplies with.
template <int DT>
__device__ __forceinline__ float packed_sum(const u32x2& w, float acc) {
  return add_pair<DT>(w[1], add_pair<DT>(w[0], acc));
}

// A row slice of EPL 16-bit elements; pair() puts element k of two rows
// side by side.
template <int EPL>
struct VSlice;
template <>
struct VSlice<8> {
  using T = u32x4;
  template <bool SHARED>
  __device__ static __forceinline__ T load(Rsrc r, int off) { return buf_load16<SHARED>(r, off); }
  // element k of x in the low half, of y in the high half (one byte permute)
  __device__ static __forceinline__ uint32_t pair(const T& x, const T& y, int k) {
    return __builtin_amdgcn_perm(y[k >> 1], x[k >> 1], (k & 1) ? 0x07060302u : 0x05040100u);
  }
};
template <>
struct VSlice<4> {
  using T = u32x2;
  template <bool SHARED>
  __device__ static __forceinline__ T load(Rsrc r, int off) { return buf_load8<SHARED>(r, off); }
  __device__ static __forceinline__ uint32_t pair(const T& x, const T& y, int k) {
    return __builtin_amdgcn_perm(y[k >> 1], x[k >> 1], (k & 1) ? 0x07060302u : 0x05040100u);
  }
};


// LDS of a workgroup whose NW waves share one item: per wave and query row
// the running max, sum and P.V accumulators; merge factors and totals.
// `fp` is the weight of an earlier (shared-prefix) part of the row.
template <int D, int NW>
struct MfmaLds {
  float m[NW][16], l[NW][16], f[NW][16], fp[16], tot[16], mx[16];
  float o[NW][16][D];
};

// Shapes of one (block, KV head) tile for the matrix-core path.
template <int DT, int D>
struct MfmaShape {
  static constexpr int NJ = D / 32;   // S products per block
  static constexpr int EPL = D / 16;  // V elements per lane per row = PV products
  static constexpr int CPR = D / 8;   // 16-byte chunks per row
  static constexpr int TILE_BYTES = kBlockSize * D * 2;
  using VS = VSlice<EPL>;
  using VT = typename VS::T;
};

// Lane coordinates inside the wave.
struct MfmaLane {
  int n, g, tok_k;  // column/row n, contraction slice g, token of S row n
  __device__ __forceinline__ MfmaLane() {
    const int lane = threadIdx.x & 63;
    n = lane & 15;
    g = lane >> 4;
    tok_k = (n >> 2) + 4 * (n & 3);
  }
};

// Softmax state of one wave for one item: running max of head n (base 2),
// this lane's share of head n's sum (tokens g + 4e), P.V accumulators
// (rows = heads 4g..4g+3, column n = dim EPL*n + jj).
template <int D>
struct MfmaState {
  float m, lsum;
  f32x4 o[D / 16];
  __device__ __forceinline__ void reset() {
    m = -INFINITY;
    lsum = 0.f;
#pragma unroll
    for (int jj = 0; jj < D / 16; ++jj) o[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
};

// The lane's share of one 16-token tile.  K: load jj is the tile's jj-th
// contiguous KiB (lane l takes its 16-byte chunk l), so every load reads
// whole cache lines; the rows reach the matrix-core layout through LDS
// (stage_k).  V: rows g + 4e, already in the P.V operand layout.  Which
// block part a load reads is known per load at compile time.
template <int DT, int D, bool SH, int BS, int TB>
__device__ __forceinline__ void load_tile(const TileDesc<BS, TB>& t, const MfmaLane& ln,
                                          u32x4 (&kr)[D / 32],
                                          typename MfmaShape<DT, D>::VT (&vr)[4]) {
  using S = MfmaShape<DT, D>;
  using Desc = TileDesc<BS, TB>;
  static_assert(TB == S::TILE_BYTES, "tile bytes");
  const int lane = ln.n + 16 * ln.g;
  static_for<0, S::NJ>([&](auto jc) {
    constexpr int jj = decltype(jc)::value;
    constexpr int h = Desc::part(jj * 1024);
    kr[jj] = buf_load16<SH>(t.k[h], (jj * 64 + lane) * 16 - h * Desc::HB);
  });
  static_for<0, 4>([&](auto ec) {
    constexpr int e = decltype(ec)::value;
    constexpr int h = Desc::part(4 * e * S::CPR * 16);  // rows 4e .. 4e+3
    vr[e] = S::VS::template load<SH>(t.v[h], ((ln.g + 4 * e) * 16 + ln.n) *
                                                 (int)sizeof(typename S::VT) - h * Desc::HB);
  });
}

// Force the wait for registers just loaded (an empty asm reading them).
template <int N>
__device__ __forceinline__ void wait_loaded(const u32x4 (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" ::"v"(x[i]));
}

// 16-byte slot of K chunk c of token row r in a wave's LDS staging tile.
// Rows are padded by one chunk: both the row-wise writes and the
// column-wise reads of the S operand then spread over the LDS banks, and
// every load/store of one lane differs from its others by a constant offset.
template <int D>
__device__ __forceinline__ int kslot(int r, int c) {
  return r * (D / 8 + 1) + c;
}
template <int D>
constexpr int kKStageSlots = kBlockSize * (D / 8 + 1);

// K tile as loaded (load jj, lane l = chunk jj*64 + l of the tile) into an
// LDS staging tile, row-major with padded rows.
template <int D>
__device__ __forceinline__ void put_k_stage(u32x4* kst, const u32x4 (&kr)[D / 32],
                                            const MfmaLane& ln) {
  constexpr int CPR = D / 8, NJ = D / 32;
  const int lane = ln.n + 16 * ln.g;
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) {
    const int idx = jj * 64 + lane;
    kst[kslot<D>(idx / CPR, idx % CPR)] = kr[jj];
  }
}

// The S operand layout out of a staging tile: lane (n, g) of product jj gets
// chunk 4jj + g of token row tau(n).
template <int D>
__device__ __forceinline__ void get_k_stage(const u32x4* kst, u32x4 (&kr)[D / 32],
                                            const MfmaLane& ln) {
#pragma unroll
  for (int jj = 0; jj < D / 32; ++jj) kr[jj] = kst[kslot<D>(ln.tok_k, 4 * jj + ln.g)];
}

// K tile through the wave's own LDS tile into the S operand layout, in
// place.  Only this wave touches `kst`, and its LDS accesses complete in
// order, so no barrier is needed.
template <int D>
__device__ __forceinline__ void stage_k(u32x4* kst, u32x4 (&kr)[D / 32], const MfmaLane& ln) {
  put_k_stage<D>(kst, kr, ln);
  get_k_stage<D>(kst, kr, ln);
}

// How many of a tile's 16 tokens count: all (kWhole); the first `limit`,
// per token (kTokens); all or none, the same for the whole wave
// (kWholeOrEmpty: an empty tile was loaded as zeros, so its V rows need no
// clearing, and its weights are dropped as a whole).
constexpr int kWhole = 0, kTokens = 1, kWholeOrEmpty = 2;

// B operands of the tile's P.V products (product jj: this lane's tokens
// g + 4e, element EPL*n + jj, packed in pairs), built once per tile; rows of
// tokens past `limit` are zeroed first (whatever those slots hold must not
// reach P.V, not even times a zero weight).
template <int DT, int D, int MASKED>
__device__ __forceinline__ void v_operands(typename MfmaShape<DT, D>::VT (&vr)[4], int limit,
                                           const MfmaLane& ln, u32x2 (&vb)[D / 16]) {
  using S = MfmaShape<DT, D>;
  using VT = typename S::VT;
  if constexpr (MASKED == kTokens) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (ln.g + 4 * e >= limit) vr[e] = VT{};
  }
#pragma unroll
  for (int jj = 0; jj < S::EPL; ++jj)
    vb[jj] = u32x2{S::VS::pair(vr[0], vr[1], jj), S::VS::pair(vr[2], vr[3], jj)};
}

// Fold one tile into the state: K already in the S operand layout
// (stage_k), V as P.V operands (v_operands), so several row tiles can share
// one tile.  Scores of tokens at or past `row_limit` (per lane: its query
// row n; the tile's token count, or less for causal rows of a multi-token
// query) are dropped.
template <int DT, int D, int MASKED>
__device__ __forceinline__ void fold_tile(MfmaState<D>& st, const u32x4 (&qb)[D / 32],
                                          const u32x4 (&kr)[D / 32], const u32x2 (&vb)[D / 16],
                                          int row_limit, float scale_log2, const MfmaLane& ln) {
  using S = MfmaShape<DT, D>;
  f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int jj = 0; jj < S::NJ; ++jj) sacc = mfma_qk<DT>(kr[jj], qb[jj], sacc);
  float sc[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    sc[e] = sacc[e] * scale_log2;
    if constexpr (MASKED == kTokens) sc[e] = ln.g + 4 * e < row_limit ? sc[e] : -INFINITY;
  }
  float mb = max_nn(max_nn(sc[0], sc[1]), max_nn(sc[2], sc[3]));
  mb = xor16_combine(mb, MaxNnOp{});
  mb = xor32_combine(mb, MaxNnOp{});
  if constexpr (MASKED == kWholeOrEmpty) mb = row_limit != 0 ? mb : -INFINITY;
  // The weights and the P.V products are written out in both arms of the
  // rescale branch: each arm's products then update the accumulators in
  // place.  With one copy after the branch the compiler keeps the rescaled
  // accumulators apart and copies every accumulator register on the path
  // without a rescale (the common one).
  auto weights_and_products = [&]() __attribute__((always_inline)) {
    float p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = fast_exp2(sc[e] - st.m);
    if constexpr (MASKED == kTokens) {
      if (st.m == -INFINITY) {  // no valid token of this head so far
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = 0.f;
      }
    }
    if constexpr (MASKED == kWholeOrEmpty) {
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = row_limit != 0 ? p[e] : 0.f;
    }
    const u32x2 pa{pack2<DT>(p[0], p[1]), pack2<DT>(p[2], p[3])};
    // The normaliser sums the weights as rounded for P.V, so numerator and
    // denominator weigh every token alike.
    st.lsum = packed_sum<DT>(pa, st.lsum);
    if constexpr (DT == kBF16) {
      // bf16 weights carry 8 significant bits: one weight's rounding moves the
      // output by up to 2^-8 of the spread of V, past the 1e-2 bound in the
      // tail of N(0,1) data.  Each weight's residual joins the product: a
      // 16x16x32 product over [weights, residuals] x [V rows, the same V rows]
      // (contraction slots 4..7 of a lane repeat its tokens g + 4e), so P.V
      // and the normaliser see the weights to ~2^-16 in one instruction.
      const u32x2 pl = residual_pack<DT>(p, pa);
      st.lsum = packed_sum<DT>(pl, st.lsum);
      const u32x4 pp{pa[0], pa[1], pl[0], pl[1]};
#pragma unroll
      for (int jj = 0; jj < S::EPL; ++jj)
        st.o[jj] = mfma_qk<DT>(pp, u32x4{vb[jj][0], vb[jj][1], vb[jj][0], vb[jj][1]}, st.o[jj]);
    } else {
#pragma unroll
      for (int jj = 0; jj < S::EPL; ++jj) st.o[jj] = mfma_pv<DT>(pa, vb[jj], st.o[jj]);
    }
  };
  // The running max moves once a score passes it by more than kRescaleSlack,
  // so every weight stays below 2^kRescaleSlack (for f16 the reference sits
  // kF16MaxOffset below the largest score: weights below 2^(slack + offset)).
  // The test is wave-uniform: any row's rise rescales all.
  constexpr float OFF = kMaxOffset<DT>;
  if (__builtin_amdgcn_ballot_w64(mb > st.m + (kRescaleSlack + OFF)) != 0) {
    const float mn = max_nn(st.m, mb - OFF);
    const float alpha = mn == -INFINITY ? 1.f : fast_exp2(st.m - mn);
    st.lsum *= alpha;
    st.m = mn;
    // output rows 4g .. 4g+3 are heads 4g+e: fetch their factors
    float arow[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      arow[e] = u2f((uint32_t)__builtin_amdgcn_ds_bpermute((4 * ln.g + e) << 2, (int)f2u(alpha)));
#pragma unroll
    for (int jj = 0; jj < S::EPL; ++jj)
#pragma unroll
      for (int e = 0; e < 4; ++e) st.o[jj][e] *= arow[e];
    weights_and_products();
  } else {
    weights_and_products();
  }
}

// Fold one tile (`limit` of its 16 tokens in the context) into the state:
// stage K, build the V operands, fold.
template <int DT, int D, int MASKED>
__device__ __forceinline__ void consume_tile(MfmaState<D>& st, const u32x4 (&qb)[D / 32],
                                             u32x4 (&kr)[D / 32],
                                             typename MfmaShape<DT, D>::VT (&vr)[4], int limit,
                                             float scale_log2, const MfmaLane& ln, u32x4* kst) {
  stage_k<D>(kst, kr, ln);
  u32x2 vb[D / 16];
  v_operands<DT, D, MASKED>(vr, limit, ln, vb);
  fold_tile<DT, D, MASKED>(st, qb, kr, vb, limit, scale_log2, ln);
}

template <int DT, int D>
__device__ __forceinline__ void consume_any(MfmaState<D>& st, const u32x4 (&qb)[D / 32],
                                            u32x4 (&kr)[D / 32],
                                            typename MfmaShape<DT, D>::VT (&vr)[4], int limit,
                                            float scale_log2, const MfmaLane& ln, u32x4* kst) {
  if (limit == kBlockSize)
    consume_tile<DT, D, false>(st, qb, kr, vr, limit, scale_log2, ln, kst);
  else
    consume_tile<DT, D, true>(st, qb, kr, vr, limit, scale_log2, ln, kst);
}

}  // namespace pa
