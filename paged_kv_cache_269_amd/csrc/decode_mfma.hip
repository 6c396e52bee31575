// Paged decode attention for grouped query heads on the gfx950 matrix cores.
//
// Same result as the vector-ALU kernel ("vLLM 2026 推理引擎全解"
// (chenxutan.com) §1.1 attention over the paged cache of §2.1-§2.2), for the
// case where G = Hq / Hkv query heads read one KV head.  Each K/V tile is
// then used by G heads, so the score and output products are real small
// matrix products: per 16-token block, S = K_blk (16 x D) . Q^T (D x 16 heads)
// and O += P (16 heads x 16 tokens) . V_blk (16 x D).  Both run on MFMA:
//   S:  v_mfma_f32_16x16x32_{bf16,f16}, D/32 of them (rows = tokens,
//       columns = heads, contraction over head_dim);
//   PV: v_mfma_f32_16x16x16_{bf16,f16}, D/16 of them (rows = heads,
//       columns = output dims, contraction over the block's 16 tokens).
// Up to 16 heads share one tile of work; G < 16 leaves rows idle (the
// matrix cores are far from the limit here, HBM is).
//
// Lane layouts (wave64, lane l, n = l % 16, g = l / 16):
//   MFMA 16x16xK operand A: row n, contraction slice g;  B: column n, slice g;
//   16x16 result: column n, rows 4g .. 4g+3.
// Orders are chosen so that no data moves between lanes:
//   * result row r of S stands for token tau(r) = r/4 + 4 (r%4), so lane l
//     ends up with the scores of tokens g + 4e (e = 0..3) for head n -- exactly
//     the P operand layout of the PV product (row = head n, contraction slice
//     g = tokens g + 4e);
//   * the PV contraction over tokens uses the same order, so lane l needs
//     V rows g + 4e: four wave-wide loads of 4 whole rows each (coalesced 1 KiB
//     per instruction at D = 128), and output column n of PV product jj is
//     dim EPL*n + jj, the elements the lane loaded;
//   * the S contraction over head_dim visits 16-byte chunk 4j + g of a row in
//     product j, so one K load instruction covers 64 contiguous bytes of each
//     of 16 rows and Q is read in the same order.
// Online softmax runs per head in base 2; the running max of a head lives in
// the 4 lanes with that n, the output rows 4g..4g+3 fetch their rescale
// factor with a lane shuffle.  Partial states of the NW waves are merged in
// LDS at the end of the partition.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace pa {

namespace {

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

// Two floats -> packed pair of 16-bit elements (round to nearest even).
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return (uint32_t)to_bits16<DT>(lo) | ((uint32_t)to_bits16<DT>(hi) << 16);
}

// 16-bit element k of a row slice held as EPL elements.
template <int EPL>
struct VSlice;
template <>
struct VSlice<8> {
  using T = u32x4;
  __device__ static __forceinline__ uint32_t half(const T& v, int k) {
    return (k & 1) ? (v[k >> 1] >> 16) : (v[k >> 1] & 0xffffu);
  }
};
template <>
struct VSlice<4> {
  using T = u32x2;
  __device__ static __forceinline__ uint32_t half(const T& v, int k) {
    return (k & 1) ? (v[k >> 1] >> 16) : (v[k >> 1] & 0xffffu);
  }
};

template <int DT, int D, int NW>
__global__ __launch_bounds__(NW * 64) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int NJ = D / 32;    // S products per block
  constexpr int EPL = D / 16;   // V elements per lane per row = PV products
  constexpr int CPR = D / 8;    // 16-byte chunks per row
  using VS = VSlice<EPL>;
  using VT = typename VS::T;

  const int part = blockIdx.x, hy = blockIdx.y, s = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int n = lane & 15, g = lane >> 4;
  const int group = a.num_q_heads / a.num_kv_heads;
  const int hchunks = (group + 15) >> 4;
  const int kvh = hy / hchunks;
  const int head0 = kvh * group + (hy % hchunks) * 16;
  const int nh = min(16, kvh * group + group - head0);

  int L = a.context_lens[s];
  L = L < 0 ? 0 : (L > a.max_len ? a.max_len : L);
  const int nblocks = (L + kBlockSize - 1) / kBlockSize;
  const int nparts = (nblocks + a.part_blocks - 1) / a.part_blocks;
  if (part > 0 && part >= nparts) return;
  const int64_t orow0 = (int64_t)s * a.num_q_heads + head0;
  if (L == 0) {
    for (int i = threadIdx.x; i < nh * D; i += NW * 64) store_elem<DT>(a.out, orow0 * D + i, 0.f);
    return;
  }

  // Q^T as the B operand of the S products: column n = head n, slice g of
  // product j = chunk 4j + g of the head's row.  Idle heads read nothing.
  u32x4 qb[NJ];
  {
    const u32x4* q = reinterpret_cast<const u32x4*>(a.q);
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj)
      qb[jj] = (n < nh) ? q[(orow0 + n) * CPR + 4 * jj + g] : u32x4{0u, 0u, 0u, 0u};
  }

  const u32x4* __restrict__ kc = reinterpret_cast<const u32x4*>(a.k_cache);
  const VT* __restrict__ vc = reinterpret_cast<const VT*>(a.v_cache);
  const int32_t* __restrict__ bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  const int jb = part * a.part_blocks;
  const int je = min(jb + a.part_blocks, nblocks);
  const int tok_k = (n >> 2) + 4 * (n & 3);  // token of S row n

  float m = -INFINITY;   // running max of head n (base 2)
  float lsum = 0.f;      // this lane's share of head n's sum (tokens g + 4e)
  f32x4 o[EPL];
#pragma unroll
  for (int jj = 0; jj < EPL; ++jj) o[jj] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto locate = [&](int j, int bid, int& limit) -> int64_t {  // tile base in elements
    limit = min(kBlockSize, L - j * kBlockSize);
    if ((uint32_t)bid >= (uint32_t)a.num_blocks_i32) {  // not a pool block: skip its tokens
      bid = 0;
      limit = 0;
    }
    return ((int64_t)bid * a.num_kv_heads + kvh) * (kBlockSize * D);
  };
  auto load = [&](int64_t base, u32x4 (&kr)[NJ], VT (&vr)[4]) {
    const u32x4* kt = kc + base / 8;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) kr[jj] = kt[tok_k * CPR + 4 * jj + g];
    const VT* vt = vc + base / EPL;
#pragma unroll
    for (int e = 0; e < 4; ++e) vr[e] = vt[(g + 4 * e) * 16 + n];
  };
  auto consume = [&](auto masked, const u32x4 (&kr)[NJ], VT (&vr)[4], int limit) {
    constexpr bool MASKED = decltype(masked)::value;
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) sacc = mfma_qk<DT>(kr[jj], qb[jj], sacc);
    float sc[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sc[e] = sacc[e] * a.scale_log2;
      if constexpr (MASKED) {
        const bool ok = g + 4 * e < limit;
        sc[e] = ok ? sc[e] : -INFINITY;
        if (!ok) vr[e] = VT{};  // whatever the slot holds must not reach P.V
      }
    }
    float mb = __builtin_fmaxf(__builtin_fmaxf(sc[0], sc[1]), __builtin_fmaxf(sc[2], sc[3]));
    mb = xor16_combine(mb, MaxOp{});
    mb = xor32_combine(mb, MaxOp{});
    const float mn = __builtin_fmaxf(m, mb);
    float alpha = fast_exp2(m - mn);
    float p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = fast_exp2(sc[e] - mn);
    if constexpr (MASKED) {
      if (mn == -INFINITY) {  // no valid token of this head so far
        alpha = 1.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = 0.f;
      }
    }
    lsum = lsum * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    m = mn;
    // output rows 4g .. 4g+3 are heads 4g+e: fetch their factors
    float arow[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      arow[e] = u2f((uint32_t)__builtin_amdgcn_ds_bpermute((4 * g + e) << 2, (int)f2u(alpha)));
    const u32x2 pa{pack2<DT>(p[0], p[1]), pack2<DT>(p[2], p[3])};
#pragma unroll
    for (int jj = 0; jj < EPL; ++jj) {
      const u32x2 vb{VS::half(vr[0], jj) | (VS::half(vr[1], jj) << 16),
                     VS::half(vr[2], jj) | (VS::half(vr[3], jj) << 16)};
      f32x4 c = o[jj];
#pragma unroll
      for (int e = 0; e < 4; ++e) c[e] *= arow[e];
      o[jj] = mfma_pv<DT>(pa, vb, c);
    }
  };
  auto consume_block = [&](const u32x4 (&kr)[NJ], VT (&vr)[4], int limit) {
    if (limit == kBlockSize)
      consume(std::false_type{}, kr, vr, limit);
    else
      consume(std::true_type{}, kr, vr, limit);
  };

  // Ping-pong register sets: block k+1 loads in flight while block k is
  // consumed; the pool id of block k+2 is fetched (scalar load) before that.
  u32x4 kA[NJ], kB[NJ];
  VT vA[4], vB[4];
  const int j0 = jb + w;
  const int nk = je > j0 ? (je - j0 + NW - 1) / NW : 0;
  if (nk > 0) {
    int id1 = nk > 1 ? bt[j0 + NW] : 0;
    int limA, limB = 0;
    load(locate(j0, bt[j0], limA), kA, vA);
    for (int k = 0;; k += 2) {
      const int id2 = k + 2 < nk ? bt[j0 + (k + 2) * NW] : 0;
      if (k + 1 < nk) load(locate(j0 + (k + 1) * NW, id1, limB), kB, vB);
      consume_block(kA, vA, limA);
      if (k + 1 >= nk) break;
      id1 = k + 3 < nk ? bt[j0 + (k + 3) * NW] : 0;
      if (k + 2 < nk) load(locate(j0 + (k + 2) * NW, id2, limA), kA, vA);
      consume_block(kB, vB, limB);
      if (k + 2 >= nk) break;
    }
  }

  // Per-head totals of this wave, then the cross-wave merge through LDS.
  lsum = xor16_combine(lsum, AddOp{});
  lsum = xor32_combine(lsum, AddOp{});
  __shared__ float s_m[NW][16], s_l[NW][16], s_f[NW][16], s_tot[16], s_max[16];
  __shared__ float s_o[NW][16][D];
  if (g == 0) {
    s_m[w][n] = m;
    s_l[w][n] = lsum;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int jj = 0; jj < EPL; ++jj) s_o[w][4 * g + e][EPL * n + jj] = o[jj][e];
  __syncthreads();
  if (threadIdx.x < 16) {
    const int hh = threadIdx.x;
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < NW; ++i) M = __builtin_fmaxf(M, s_m[i][hh]);
    float tot = 0.f;
    float f[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      f[i] = (s_m[i][hh] == -INFINITY) ? 0.f : fast_exp2(s_m[i][hh] - M);
      tot += s_l[i][hh] * f[i];
    }
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) s_f[i][hh] = f[i] * inv;
    s_tot[hh] = tot;
    s_max[hh] = M;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nh * D; i += NW * 64) {
    const int hh = i / D, d = i % D;
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < NW; ++k) v += s_o[k][hh][d] * s_f[k][hh];
    if (nparts <= 1) {
      store_elem<DT>(a.out, (orow0 + hh) * D + d, v);
    } else {
      const int64_t prow = (orow0 + hh) * a.max_partitions + part;
      a.tmp_out[prow * D + d] = v;
      if (d == 0) {
        a.max_logits[prow] = s_max[hh] * kLn2;
        a.exp_sums[prow] = s_tot[hh];
      }
    }
  }
}

template <int DT, int D>
hipError_t launch_typed(const DecodeArgs& a, int num_seqs, hipStream_t stream) {
  constexpr int NW = 4;
  const int group = a.num_q_heads / a.num_kv_heads;
  dim3 grid(a.max_partitions, a.num_kv_heads * ((group + 15) / 16), num_seqs);
  hipLaunchKernelGGL((decode_mfma_kernel<DT, D, NW>), grid, dim3(NW * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, int dtype, int head_dim, int num_seqs,
                              hipStream_t stream) {
  switch (dtype * 1000 + head_dim) {
    case kF16 * 1000 + 64: return launch_typed<kF16, 64>(a, num_seqs, stream);
    case kF16 * 1000 + 128: return launch_typed<kF16, 128>(a, num_seqs, stream);
    case kBF16 * 1000 + 64: return launch_typed<kBF16, 64>(a, num_seqs, stream);
    case kBF16 * 1000 + 128: return launch_typed<kBF16, 128>(a, num_seqs, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
