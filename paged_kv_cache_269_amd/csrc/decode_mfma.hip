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
#include "items.h"
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
  template <bool SHARED>
  __device__ static __forceinline__ T load(Rsrc r, int off) { return buf_load16<SHARED>(r, off); }
  __device__ static __forceinline__ uint32_t half(const T& v, int k) {
    return (k & 1) ? (v[k >> 1] >> 16) : (v[k >> 1] & 0xffffu);
  }
};
template <>
struct VSlice<4> {
  using T = u32x2;
  template <bool SHARED>
  __device__ static __forceinline__ T load(Rsrc r, int off) { return buf_load8<SHARED>(r, off); }
  __device__ static __forceinline__ uint32_t half(const T& v, int k) {
    return (k & 1) ? (v[k >> 1] >> 16) : (v[k >> 1] & 0xffffu);
  }
};

template <int D, int NW>
struct MfmaLds {
  float m[NW][16], l[NW][16], f[NW][16], tot[16], mx[16];
  float o[NW][16][D];
};

// One item: head tile hy (a KV head and up to 16 of its query heads) of
// sequence s over partition `part` (context L).
template <int DT, int D, int NW, int DEPTH>
__device__ __forceinline__ void mfma_item(const DecodeArgs& a, const int hy, const int s,
                                          const int part, const int L, MfmaLds<D, NW>& sm) {
  constexpr int NJ = D / 32;    // S products per block
  constexpr int EPL = D / 16;   // V elements per lane per row = PV products
  constexpr int CPR = D / 8;    // 16-byte chunks per row
  using VS = VSlice<EPL>;
  using VT = typename VS::T;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int n = lane & 15, g = lane >> 4;
  const int group = a.num_q_heads / a.num_kv_heads;
  const int hchunks = (group + 15) >> 4;
  const int kvh = hy / hchunks;
  const int head0 = kvh * group + (hy % hchunks) * 16;
  const int nh = min(16, kvh * group + group - head0);
  const int nblocks = (L + kBlockSize - 1) / kBlockSize;
  const int nparts = (nblocks + a.part_blocks - 1) / a.part_blocks;
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

  constexpr int TILE_BYTES = kBlockSize * D * 2;
  const char* kbase = static_cast<const char*>(a.k_cache);
  const char* vbase = static_cast<const char*>(a.v_cache);
  const int32_t* __restrict__ bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  const int jb = part * a.part_blocks;
  const int je = min(jb + a.part_blocks, nblocks);
  const int j0 = jb + w;                                  // this wave: blocks j0, j0+NW, ...
  const int nk = je > j0 ? (je - j0 + NW - 1) / NW : 0;  // how many
  const int tok_k = (n >> 2) + 4 * (n & 3);               // token of S row n

  float m = -INFINITY;   // running max of head n (base 2)
  float lsum = 0.f;      // this lane's share of head n's sum (tokens g + 4e)
  f32x4 o[EPL];
#pragma unroll
  for (int jj = 0; jj < EPL; ++jj) o[jj] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Pool id of the wave's kk-th block (index clamped into the table row).
  auto id_at = [&](int kk) -> int { return bt[j0 + min(kk, nk - 1) * NW]; };
  // Descriptors of the wave's kk-th tile and the number of its tokens in the
  // context; empty past the wave's last block or for an id outside the pool.
  auto tile = [&](int kk, int bid, int& limit, Rsrc& rk, Rsrc& rv) {
    const int j = j0 + min(kk, nk - 1) * NW;
    const bool ok = kk < nk && (uint32_t)bid < (uint32_t)a.num_blocks_i32;
    limit = ok ? min(kBlockSize, L - j * kBlockSize) : 0;
    const int64_t off = ((int64_t)(ok ? bid : 0) * a.num_kv_heads + kvh) * TILE_BYTES;
    rk = make_rsrc(kbase + off, ok ? TILE_BYTES : 0);
    rv = make_rsrc(vbase + off, ok ? TILE_BYTES : 0);
  };
  auto load = [&](auto shared, Rsrc rk, Rsrc rv, u32x4 (&kr)[NJ], VT (&vr)[4]) {
    constexpr bool SH = decltype(shared)::value;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) kr[jj] = buf_load16<SH>(rk, (tok_k * CPR + 4 * jj + g) * 16);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      vr[e] = VS::template load<SH>(rv, ((g + 4 * e) * 16 + n) * (int)sizeof(VT));
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

  // Software pipeline over the wave's blocks: DEPTH register sets; while
  // block k is consumed, the loads of blocks k+1 .. k+DEPTH-1 are in flight,
  // and the pool id of the next block to issue is already being fetched.
  // Every step issues its loads (empty past the end) so that the wait counts
  // are the same on every path -- no branch around a load -- and a
  // past-the-end step consumes nothing.
  u32x4 kr[DEPTH][NJ];
  VT vr[DEPTH][4];
  int lim[DEPTH];
  auto pipeline = [&](auto shared) {
    static_for<0, DEPTH - 1>([&](auto dc) {
      constexpr int d = decltype(dc)::value;
      Rsrc rk, rv;
      tile(d, id_at(d), lim[d], rk, rv);
      load(shared, rk, rv, kr[d], vr[d]);
    });
    int next_id = id_at(DEPTH - 1);
    for (int k = 0; k < nk; k += DEPTH) {
      static_for<0, DEPTH>([&](auto dc) {
        constexpr int d = decltype(dc)::value;
        constexpr int dn = (d + DEPTH - 1) % DEPTH;
        const int kn = k + d + DEPTH - 1;  // block whose loads are issued now
        const int id = next_id;
        next_id = id_at(kn + 1);
        Rsrc rk, rv;
        tile(kn, id, lim[dn], rk, rv);
        load(shared, rk, rv, kr[dn], vr[dn]);
        consume_block(kr[d], vr[d], lim[d]);
      });
    }
  };
  if (nk > 0) {
    // Shared prefix pages are re-read by every sequence that maps them: an
    // item whose first block the neighbouring sequence's table maps to the
    // same physical block loads with the cache-allocating policy; all other
    // items stream their tiles non-temporally.
    const int32_t* nb = a.num_seqs > 1 ? a.block_tables +
                            (int64_t)(s > 0 ? s - 1 : s + 1) * a.max_blocks_per_seq : nullptr;
    if (nb != nullptr && nb[j0] == bt[j0])
      pipeline(std::true_type{});
    else
      pipeline(std::false_type{});
  }

  // Per-head totals of this wave, then the cross-wave merge through LDS.
  lsum = xor16_combine(lsum, AddOp{});
  lsum = xor32_combine(lsum, AddOp{});
  if (g == 0) {
    sm.m[w][n] = m;
    sm.l[w][n] = lsum;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int jj = 0; jj < EPL; ++jj) sm.o[w][4 * g + e][EPL * n + jj] = o[jj][e];
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
  for (int i = threadIdx.x; i < nh * D; i += NW * 64) {
    const int hh = i / D, d = i % D;
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < NW; ++k) v += sm.o[k][hh][d] * sm.f[k][hh];
    if (nparts <= 1) {
      store_elem<DT>(a.out, (orow0 + hh) * D + d, v);
    } else {
      const int64_t prow = (orow0 + hh) * a.max_partitions + part;
      a.tmp_out[prow * D + d] = v;
      if (d == 0) {
        a.max_logits[prow] = sm.mx[hh] * kLn2;
        a.exp_sums[prow] = sm.tot[hh];
      }
    }
  }
}

// One workgroup per item.  Head units vary fastest across the grid:
// workgroups are dealt to the 8 XCDs round-robin, so the equal-sized items of
// one (sequence, partition) spread evenly over the XCDs, and one head unit of
// every sequence stays on one XCD (shared prefix pages then hit its L2).
template <int DT, int D, int NW, int DEPTH>
__global__ __launch_bounds__(NW * 64) void decode_mfma_kernel(DecodeArgs a) {
  __shared__ MfmaLds<D, NW> sm;
  const int unit = blockIdx.x, s = blockIdx.y, part = blockIdx.z;
  const int L = clamp_len(a, s);
  if (part >= parts_of(L, a.part_blocks)) return;  // past this sequence's end
  mfma_item<DT, D, NW, DEPTH>(a, unit, s, part, L, sm);
}

// Launch shapes: items of at least kLongItemBlocks blocks get 8 waves,
// shorter ones 4 (more workgroups resident per CU).
constexpr int kLongItemBlocks = 128;

template <int DT, int D, int NW, int DEPTH>
hipError_t launch_shape(const DecodeArgs& a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  const dim3 grid(a.num_kv_heads * ((group + 15) / 16), a.num_seqs, a.max_partitions);
  hipLaunchKernelGGL((decode_mfma_kernel<DT, D, NW, DEPTH>), grid, dim3(NW * 64), 0, stream, a);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  return a.part_blocks >= kLongItemBlocks ? launch_shape<DT, D, 8, 2>(a, stream)
                                          : launch_shape<DT, D, 4, 2>(a, stream);
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, int dtype, int head_dim, hipStream_t stream) {
  switch (dtype * 1000 + head_dim) {
    case kF16 * 1000 + 64: return launch_typed<kF16, 64>(a, stream);
    case kF16 * 1000 + 128: return launch_typed<kF16, 128>(a, stream);
    case kBF16 * 1000 + 64: return launch_typed<kBF16, 64>(a, stream);
    case kBF16 * 1000 + 128: return launch_typed<kBF16, 128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
