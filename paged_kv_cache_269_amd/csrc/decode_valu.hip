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
//   workgroup = (query head, sequence, partition), NW waves;
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
// One-call decode step (DecodeArgs::new_slots set): the new token of each
// sequence is written by the item that owns its KV head's last partition,
// and every item whose context ends with that slot takes the row from
// registers instead of the cache (same page §1.1: o_t attends over K_{1:t}
// with token t included), so no item waits for the write.
#include <type_traits>

#include "common.h"
#include "items.h"
#include "launch.h"

namespace pa {

namespace {

template <int DT, int D>
struct ValuShape {
  static constexpr int VEC = 16 / Elem<DT>::bytes;  // elements per 16-byte chunk
  static constexpr int LPT = D / VEC;               // lanes per token row
  static constexpr int TPL = 64 / LPT;              // token rows per wave load
  static constexpr int NLD = kBlockSize / TPL;      // loads per tile per lane
  static constexpr int TILE_BYTES = kBlockSize * D * Elem<DT>::bytes;  // one (block, head) tile
  static_assert(LPT >= 2 && LPT <= 32 && TPL * LPT == 64, "unsupported head_dim");
};

// Shared memory of one workgroup: the per-row partial states of an item.
template <int DT, int D, int NW>
struct ValuLds {
  static constexpr int R = NW * ValuShape<DT, D>::TPL;
  float m[R], l[R];
  float acc[R * D];
};

// One item: query head h of sequence s over partition `part` (context L).
// WAVE_ITEM: the calling wave alone processes the whole partition and merges
// its rows in registers (no LDS, no barrier); otherwise the NW waves of the
// workgroup share the partition's blocks and merge through LDS.
template <int DT, int D, int NW, int DEPTH, bool WAVE_ITEM, int BS = kBlockSize>
__device__ __forceinline__ void valu_item(const DecodeArgs& a, const int h, const int s,
                                          const int part, const int L, ValuLds<DT, D, NW>* sm) {
  using S = ValuShape<DT, D>;
  constexpr int VEC = S::VEC, LPT = S::LPT, TPL = S::TPL, NLD = S::NLD;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int row = lane / LPT, c = lane % LPT;
  const int group = a.num_q_heads / a.num_kv_heads;
  const int kvh = h / group;
  const int nblocks = (L + kBlockSize - 1) / kBlockSize;
  const int nparts = (nblocks + a.part_blocks - 1) / a.part_blocks;
  const int64_t orow = (int64_t)s * a.num_q_heads + h;
  const int32_t* __restrict__ bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;

  // Fused KV write: the first query head of each KV head, in the partition
  // holding the context's end, stores the new token's row (lanes of row 0,
  // chunk c each); every item takes the row from registers where its context
  // ends with that slot.
  constexpr int RB = D * Elem<DT>::bytes;  // bytes of one K or V row
  const NewToken nt = new_token<BS>(a, bt, s, kvh, L, h % group == 0 && part == max(nparts, 1) - 1,
                                    RB);
  const u32x4 nkc = buf_load16(new_row_rsrc(a, a.new_k, s, kvh, RB), c * 16);
  const u32x4 nvc = buf_load16(new_row_rsrc(a, a.new_v, s, kvh, RB), c * 16);
  auto store_new = [&]() {
    if (nt.store && (WAVE_ITEM || w == 0) && row == 0) {
      store_row_part(a.k_cache, nt.off + c * 16, nkc);
      store_row_part(a.v_cache, nt.off + c * 16, nvc);
    }
  };

  if (L == 0) {
    const int t0 = WAVE_ITEM ? lane : (int)threadIdx.x, tn = WAVE_ITEM ? 64 : NW * 64;
    for (int d = t0; d < D; d += tn) store_elem<DT>(a.out, orow * D + d, 0.f);
    store_new();
    return;
  }

  const u32x4 qv = reinterpret_cast<const u32x4*>(a.q)[orow * (D / VEC) + c];
  // Shared-prefix launches (one pass): the leading `pre` blocks were done by
  // the prefix kernel; their state joins the merge below.
  const int pre = (!WAVE_ITEM && a.prefix_blocks != nullptr) ? a.prefix_blocks[s] : 0;
  const int jb = max(part * a.part_blocks, pre);
  const int je = min(part * a.part_blocks + a.part_blocks, nblocks);
  constexpr int STRIDE = WAVE_ITEM ? 1 : NW;
  const int j0 = jb + (WAVE_ITEM ? 0 : w);                         // blocks j0, j0+STRIDE, ...
  const int nk = je > j0 ? (je - j0 + STRIDE - 1) / STRIDE : 0;  // how many

  float m = -INFINITY, l = 0.f;
  float acc[VEC];
#pragma unroll
  for (int k = 0; k < VEC; ++k) acc[k] = 0.f;

  using Desc = TileDesc<BS, S::TILE_BYTES>;
  // Pool ids of the wave's kk-th 16-token tile (index clamped into the row).
  auto id_at = [&](int kk) {
    return tile_ids<BS>(bt, j0 + min(kk, nk - 1) * STRIDE, a.max_blocks_per_seq);
  };
  // Descriptors of the wave's kk-th tile and the number of its tokens in the
  // context; past the wave's last tile the descriptors are empty and no
  // token counts, nor do tokens in a block whose id lies outside the pool.
  auto tile = [&](int kk, const TileIds<BS>& ids, int& limit, int& tj) {
    const int j = j0 + min(kk, nk - 1) * STRIDE;
    const bool ok = kk < nk;
    limit = ok ? tile_limit<BS>(a, ids, L - j * kBlockSize) : 0;
    tj = ok ? j : -1;
    return tile_desc<BS, S::TILE_BYTES>(a, ids, j, kvh, ok);
  };
  // Load i covers the tile's i-th KiB (TPL whole rows); which block part it
  // reads is known per load at compile time.
  auto load = [&](auto shared, const Desc& t, u32x4 (&kr)[NLD], u32x4 (&vr)[NLD]) {
    constexpr bool SH = decltype(shared)::value;
    static_for<0, NLD>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr int h = Desc::part(i * 1024);
      kr[i] = buf_load16<SH>(t.k[h], (i * 64 + lane) * 16 - h * Desc::HB);
    });
    static_for<0, NLD>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr int h = Desc::part(i * 1024);
      vr[i] = buf_load16<SH>(t.v[h], (i * 64 + lane) * 16 - h * Desc::HB);
    });
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
  auto consume_block = [&](u32x4 (&kr)[NLD], u32x4 (&vr)[NLD], int limit, int tj) {
    if (nt.sub && tj == nt.tile) {  // the context's last token is the new one
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        if (i * TPL + row == nt.row) {
          kr[i] = nkc;
          vr[i] = nvc;
        }
      }
    }
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
  u32x4 kr[DEPTH][NLD], vr[DEPTH][NLD];
  int lim[DEPTH], tjs[DEPTH];
  auto pipeline = [&](auto shared) {
    static_for<0, DEPTH - 1>([&](auto dc) {
      constexpr int d = decltype(dc)::value;
      load(shared, tile(d, id_at(d), lim[d], tjs[d]), kr[d], vr[d]);
    });
    TileIds<BS> next_id = id_at(DEPTH - 1);
    for (int k = 0; k < nk; k += DEPTH) {
      static_for<0, DEPTH>([&](auto dc) {
        constexpr int d = decltype(dc)::value;
        constexpr int dn = (d + DEPTH - 1) % DEPTH;
        const int kn = k + d + DEPTH - 1;  // tile whose loads are issued now
        const TileIds<BS> id = next_id;
        next_id = id_at(kn + 1);
        load(shared, tile(kn, id, lim[dn], tjs[dn]), kr[dn], vr[dn]);
        consume_block(kr[d], vr[d], lim[d], tjs[d]);
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
    if (nb != nullptr && tile_ids<BS>(nb, j0, a.max_blocks_per_seq).id[0] ==
                             tile_ids<BS>(bt, j0, a.max_blocks_per_seq).id[0])
      pipeline(std::true_type{});
    else
      pipeline(std::false_type{});
  }
  store_new();

  if constexpr (WAVE_ITEM) {
    // Merge this wave's TPL row states in registers; row 0 writes.
    const float M = across_groups<LPT>(m, MaxOp{});
    const float f = (m == -INFINITY) ? 0.f : fast_exp2(m - M);
    const float lsum = across_groups<LPT>(l * f, AddOp{});
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    float o[VEC];
#pragma unroll
    for (int k = 0; k < VEC; ++k) o[k] = across_groups<LPT>(acc[k] * f, AddOp{}) * inv;
    if (row == 0) {
      if (nparts <= 1) {
        store16<DT>(a.out, orow * D + c * VEC, o);
      } else {
        const int64_t prow = orow * a.max_partitions + part;
#pragma unroll
        for (int k = 0; k < VEC; k += 4)  // fp32 partials: 16 bytes = 4 values per store
          store16<kF32>(a.tmp_out, prow * D + c * VEC + k, o + k);
        if (c == 0) {
          a.max_logits[prow] = M * kLn2;  // back to natural-log units
          a.exp_sums[prow] = lsum;
        }
      }
    }
    return;
  }

  // Merge the TPL x NW partial states of this partition.
  constexpr int R = NW * TPL;
  const int r = w * TPL + row;
  if (c == 0) {
    sm->m[r] = m;
    sm->l[r] = l;
  }
#pragma unroll
  for (int k = 0; k < VEC; ++k) sm->acc[r * D + c * VEC + k] = acc[k];
  __syncthreads();

  const float pm = pre > 0 ? a.prefix_m[orow] : -INFINITY;
  const float pl = pre > 0 ? a.prefix_l[orow] : 0.f;
  for (int d = threadIdx.x; d < D; d += NW * 64) {
    float M = pm;
#pragma unroll
    for (int i = 0; i < R; ++i) M = __builtin_fmaxf(M, sm->m[i]);
    float lsum = 0.f, o = 0.f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const float f = (sm->m[i] == -INFINITY) ? 0.f : fast_exp2(sm->m[i] - M);
      lsum += sm->l[i] * f;
      o += sm->acc[i * D + d] * f;
    }
    if (pre > 0) {
      const float wp = pl * fast_exp2(pm - M);
      lsum += wp;
      o += wp * a.prefix_o[orow * D + d];
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

// One workgroup per item.  Head units vary fastest across the grid:
// workgroups are dealt to the 8 XCDs round-robin, so the equal-sized items of
// one (sequence, partition) spread evenly over the XCDs, and one head unit of
// every sequence stays on one XCD (shared prefix pages then hit its L2).
template <int DT, int D, int NW, int DEPTH, int BS>
__global__ __launch_bounds__(NW * 64) void decode_valu_kernel(DecodeArgs a) {
  __shared__ ValuLds<DT, D, NW> sm;
  const int unit = blockIdx.x, s = longest_first(a, blockIdx.y), part = blockIdx.z;
  const int L = clamp_len(a, s);
  if (part >= parts_of(L, a.part_blocks)) return;  // past this sequence's end
  valu_item<DT, D, NW, DEPTH, false, BS>(a, unit, s, part, L, &sm);
}

// One wave per item: wave w of workgroup z takes partition z * NW + w, for
// launches with many partitions per sequence (each wave then streams a whole
// partition; there is no cross-wave merge).
template <int DT, int D, int NW, int DEPTH>
__global__ __launch_bounds__(NW * 64) void decode_valu_wave_kernel(DecodeArgs a) {
  const int unit = blockIdx.x, s = longest_first(a, blockIdx.y);
  const int part = blockIdx.z * NW + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int L = clamp_len(a, s);
  if (part >= parts_of(L, a.part_blocks)) return;  // past this sequence's end
  valu_item<DT, D, NW, DEPTH, true>(a, unit, s, part, L, nullptr);
}

#ifndef PA_WAVE_ITEM_WAVES
#define PA_WAVE_ITEM_WAVES 4  // waves (= partitions) per workgroup, one-wave items
#endif
#ifndef PA_WAVE_ITEM_DEPTH
#define PA_WAVE_ITEM_DEPTH 3  // tiles per wave in the load pipeline, one-wave items
#endif

// Workgroup-per-item launches: 4 waves, 2 tiles in flight per wave.  On the
// LLaMA-7B shape (items of 32-128 blocks) this measured 201 us per call
// against 206-209 us for 8 waves with 3 tiles in flight, and 203-205 us for
// 8 x 2, 4 x 3 and 4 x 4: more, smaller workgroups per CU balance better.
constexpr int kItemWaves = 4;
constexpr int kItemDepth = 2;

template <int DT, int D, int NW, int DEPTH, int BS = kBlockSize>
hipError_t launch_shape(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.num_q_heads, a.num_seqs, a.max_partitions);
  hipLaunchKernelGGL((decode_valu_kernel<DT, D, NW, DEPTH, BS>), grid, dim3(NW * 64), 0, stream,
                     a);
  return hipGetLastError();
}

// Launches with at least kWaveItemParts partitions take one wave per item.
#ifndef PA_WAVE_ITEM_PARTS
#define PA_WAVE_ITEM_PARTS 8
#endif
constexpr int kWaveItemParts = PA_WAVE_ITEM_PARTS;

template <int DT, int D, int NW, int DEPTH>
hipError_t launch_wave_shape(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.num_q_heads, a.num_seqs, (a.max_partitions + NW - 1) / NW);
  hipLaunchKernelGGL((decode_valu_wave_kernel<DT, D, NW, DEPTH>), grid, dim3(NW * 64), 0, stream,
                     a);
  return hipGetLastError();
}

#ifndef PA_CASCADE_WAVES
#define PA_CASCADE_WAVES 2  // waves per item after a shared-prefix pass
#endif
#ifndef PA_CASCADE_DEPTH
#define PA_CASCADE_DEPTH 2
#endif

template <int DT, int D>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  // 8- and 32-token blocks: workgroup-per-item kernels for every launch.
  if (a.block_size == 8) return launch_shape<DT, D, kItemWaves, kItemDepth, 8>(a, stream);
  if (a.block_size == 32) return launch_shape<DT, D, kItemWaves, kItemDepth, 32>(a, stream);
  // After a shared-prefix pass the items hold only the private blocks.
  if (a.prefix_blocks != nullptr)
    return launch_shape<DT, D, PA_CASCADE_WAVES, PA_CASCADE_DEPTH>(a, stream);
  if (a.max_partitions >= kWaveItemParts) return launch_wave_shape<DT, D, PA_WAVE_ITEM_WAVES, PA_WAVE_ITEM_DEPTH>(a, stream);
  return launch_shape<DT, D, kItemWaves, kItemDepth>(a, stream);
}

}  // namespace

hipError_t launch_decode_valu(const DecodeArgs& a, int dtype, int head_dim, hipStream_t stream) {
  clear_stale_error();
  switch (dtype * 1000 + head_dim) {
    case kF32 * 1000 + 64: return launch_typed<kF32, 64>(a, stream);
    case kF32 * 1000 + 128: return launch_typed<kF32, 128>(a, stream);
    case kF16 * 1000 + 64: return launch_typed<kF16, 64>(a, stream);
    case kF16 * 1000 + 128: return launch_typed<kF16, 128>(a, stream);
    case kBF16 * 1000 + 64: return launch_typed<kBF16, 64>(a, stream);
    case kBF16 * 1000 + 128: return launch_typed<kBF16, 128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
