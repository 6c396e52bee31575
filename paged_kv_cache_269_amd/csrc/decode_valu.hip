// Paged decode attention on the vector ALU (one query head per workgroup).
//
// What is computed -- "vLLM 2026 推理引擎全解" (chenxutan.com), §1.1:
// o = softmax(scale * q K^T) V over every cached token of the sequence;
// §2.1-§2.2 of the same page: the tokens live in 16-token pages found through
// the sequence's page table, pool layout [pages, heads, 16, head_dim].  The
// vLLM manual (doramagic.ai), PagedAttention V1/V2 kernels, names the ideas
// reused here in gfx950 form: paged K/V reads, wavefront reductions, one
// fused kernel, wide vector loads.
//
// Work split (gfx950, wave64):
//   workgroup = (partition, query head, sequence), NW waves;
//   wave w takes blocks w, w+NW, ... of its partition;
//   one (block, kv head) tile is 16 rows of head_dim elements, contiguous in
//   HBM (16 * D * e bytes).  A wave-wide 16-byte-per-lane load covers TPL =
//   64 / LPT whole rows (LPT lanes per row), so every load instruction reads
//   one contiguous 1 KiB run; a tile takes NLD = 16 / TPL such loads for K
//   and as many for V.  The next block's loads are issued before the current
//   block is consumed.
//   Each group of LPT lanes owns one token row per load: it forms the q.k dot
//   product on its 16-byte slices (v_dot2 for f16/bf16) and finishes it with
//   a DPP butterfly, keeps its own running max / sum / output slice (online
//   softmax in base 2), and accumulates p * v for the dims it loaded.
//   The TPL rows x NW waves partial states are merged once, through LDS, at
//   the end of the partition.
// Tail tokens (>= context length) of the last block are removed by
// selection, never by multiplying, so whatever they hold (NaN included)
// cannot reach the result.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace pa {

namespace {

template <int DT, int D>
struct ValuShape {
  static constexpr int VEC = 16 / Elem<DT>::bytes;  // elements per 16-byte chunk
  static constexpr int LPT = D / VEC;               // lanes per token row
  static constexpr int TPL = 64 / LPT;              // token rows per wave load
  static constexpr int NLD = kBlockSize / TPL;      // loads per tile per lane
  static constexpr int CPT = kBlockSize * D / VEC;  // 16-byte chunks per tile
  static_assert(LPT >= 2 && LPT <= 32 && TPL * LPT == 64, "unsupported head_dim");
};

template <int DT, int D, int NW>
__global__ __launch_bounds__(NW * 64) void decode_valu_kernel(DecodeArgs a) {
  using S = ValuShape<DT, D>;
  constexpr int VEC = S::VEC, LPT = S::LPT, TPL = S::TPL, NLD = S::NLD;

  const int part = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int row = lane / LPT, c = lane % LPT;
  const int group = a.num_q_heads / a.num_kv_heads;
  const int kvh = h / group;

  int L = a.context_lens[s];
  L = L < 0 ? 0 : (L > a.max_len ? a.max_len : L);
  const int nblocks = (L + kBlockSize - 1) / kBlockSize;
  const int nparts = (nblocks + a.part_blocks - 1) / a.part_blocks;
  if (part > 0 && part >= nparts) return;
  const int64_t orow = (int64_t)s * a.num_q_heads + h;
  if (L == 0) {
    for (int d = threadIdx.x; d < D; d += NW * 64) store_elem<DT>(a.out, orow * D + d, 0.f);
    return;
  }

  const u32x4 qv = reinterpret_cast<const u32x4*>(a.q)[orow * (D / VEC) + c];
  const u32x4* __restrict__ kc = reinterpret_cast<const u32x4*>(a.k_cache);
  const u32x4* __restrict__ vc = reinterpret_cast<const u32x4*>(a.v_cache);
  const int32_t* __restrict__ bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  const int jb = part * a.part_blocks;
  const int je = min(jb + a.part_blocks, nblocks);

  float m = -INFINITY, l = 0.f;
  float acc[VEC];
#pragma unroll
  for (int k = 0; k < VEC; ++k) acc[k] = 0.f;

  // Tile base (in 16-byte chunks) of block j whose pool id is bid, and the
  // number of its tokens that belong to the context.
  auto locate = [&](int j, int bid, int& limit) -> int64_t {
    limit = min(kBlockSize, L - j * kBlockSize);
    if ((uint32_t)bid >= (uint32_t)a.num_blocks_i32) {  // not a pool block: skip its tokens
      bid = 0;
      limit = 0;
    }
    return ((int64_t)bid * a.num_kv_heads + kvh) * S::CPT;
  };
  auto load = [&](int64_t base, u32x4 (&kr)[NLD], u32x4 (&vr)[NLD]) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) kr[i] = kc[base + i * 64 + lane];
#pragma unroll
    for (int i = 0; i < NLD; ++i) vr[i] = vc[base + i * 64 + lane];
  };
  auto consume = [&](auto masked, const u32x4 (&kr)[NLD], const u32x4 (&vr)[NLD], int limit) {
    constexpr bool MASKED = decltype(masked)::value;
    float sc[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      sc[i] = group_sum<LPT>(dot16<DT>(qv, kr[i], 0.f)) * a.scale_log2;
      if constexpr (MASKED) sc[i] = (i * TPL + row < limit) ? sc[i] : -INFINITY;
    }
    float mb = sc[0];
#pragma unroll
    for (int i = 1; i < NLD; ++i) mb = __builtin_fmaxf(mb, sc[i]);
    const float mn = __builtin_fmaxf(m, mb);
    if constexpr (MASKED) {
      if (mn == -INFINITY) return;  // nothing valid for this row yet
    }
    const float alpha = fast_exp2(m - mn);
    float p[NLD];
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      p[i] = fast_exp2(sc[i] - mn);
      ps += p[i];
    }
    l = l * alpha + ps;
#pragma unroll
    for (int k = 0; k < VEC; ++k) acc[k] *= alpha;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      if (!MASKED || i * TPL + row < limit) axpy16<DT>(p[i], vr[i], acc);
    }
    m = mn;
  };
  auto consume_block = [&](const u32x4 (&kr)[NLD], const u32x4 (&vr)[NLD], int limit) {
    if (limit == kBlockSize)
      consume(std::false_type{}, kr, vr, limit);
    else
      consume(std::true_type{}, kr, vr, limit);
  };

  // Two register sets, ping-pong: the loads of block k+1 are in flight while
  // block k is consumed, and the pool id of block k+2 is fetched (scalar
  // load) before block k is consumed.
  u32x4 kA[NLD], vA[NLD], kB[NLD], vB[NLD];
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

  // Merge the TPL x NW partial states of this partition.
  constexpr int R = NW * TPL;
  __shared__ float s_m[R], s_l[R];
  __shared__ float s_acc[R * D];
  const int r = w * TPL + row;
  if (c == 0) {
    s_m[r] = m;
    s_l[r] = l;
  }
#pragma unroll
  for (int k = 0; k < VEC; ++k) s_acc[r * D + c * VEC + k] = acc[k];
  __syncthreads();

  for (int d = threadIdx.x; d < D; d += NW * 64) {
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < R; ++i) M = __builtin_fmaxf(M, s_m[i]);
    float lsum = 0.f, o = 0.f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const float f = (s_m[i] == -INFINITY) ? 0.f : fast_exp2(s_m[i] - M);
      lsum += s_l[i] * f;
      o += s_acc[i * D + d] * f;
    }
    o = lsum > 0.f ? o / lsum : 0.f;
    if (nparts <= 1) {
      store_elem<DT>(a.out, orow * D + d, o);
    } else {
      const int64_t prow = orow * a.max_partitions + part;
      a.tmp_out[prow * D + d] = o;
      if (d == 0) {
        a.max_logits[prow] = M * kLn2;  // back to natural-log units
        a.exp_sums[prow] = lsum;
      }
    }
  }
}

template <int DT, int D>
hipError_t launch_typed(const DecodeArgs& a, int num_seqs, hipStream_t stream) {
  constexpr int NW = 4;
  dim3 grid(a.max_partitions, a.num_q_heads, num_seqs);
  hipLaunchKernelGGL((decode_valu_kernel<DT, D, NW>), grid, dim3(NW * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_valu(const DecodeArgs& a, int dtype, int head_dim, int num_seqs,
                              hipStream_t stream) {
  switch (dtype * 1000 + head_dim) {
    case kF32 * 1000 + 64: return launch_typed<kF32, 64>(a, num_seqs, stream);
    case kF32 * 1000 + 128: return launch_typed<kF32, 128>(a, num_seqs, stream);
    case kF16 * 1000 + 64: return launch_typed<kF16, 64>(a, num_seqs, stream);
    case kF16 * 1000 + 128: return launch_typed<kF16, 128>(a, num_seqs, stream);
    case kBF16 * 1000 + 64: return launch_typed<kBF16, 64>(a, num_seqs, stream);
    case kBF16 * 1000 + 128: return launch_typed<kBF16, 128>(a, num_seqs, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
