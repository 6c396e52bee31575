// Paged decode attention for grouped query heads on the gfx950 matrix cores.
//
// Same result as the vector-ALU kernel ("vLLM 2026 推理引擎全解"
// (chenxutan.com) §1.1 attention over the paged cache of §2.1-§2.2), for the
// case where G = Hq / Hkv query heads read one KV head.  Each K/V tile is
// then used by G heads, so the score and output products are real small
// matrix products (mfma_tile.h); up to 16 heads share one tile of work, and
// G < 16 leaves rows idle (the matrix cores are far from the limit here, HBM
// is).  Partial states of the NW waves of a workgroup are merged in LDS at
// the end of the partition; one-wave items and the streaming kernel write
// theirs from registers.  Every kernel here also does the one-call step's
// KV write (items.h, new_token).
#include <type_traits>

#include "common.h"
#include "items.h"
#include "launch.h"
#include "mfma_tile.h"

namespace pa {

namespace {


// Head tile of an item: KV head and its first query head / count.
struct HeadTile {
  int kvh, nh;
  int64_t orow0;  // (s, first query head) row index
};

__device__ __forceinline__ HeadTile head_tile(const DecodeArgs& a, int unit, int s) {
  const int group = a.num_q_heads / a.num_kv_heads;
  const int hchunks = (group + 15) >> 4;
  HeadTile t;
  t.kvh = unit / hchunks;
  const int head0 = t.kvh * group + (unit % hchunks) * 16;
  t.nh = min(16, t.kvh * group + group - head0);
  t.orow0 = (int64_t)s * a.num_q_heads + head0;
  return t;
}

// Q^T as the B operand of the S products: column n = head n, slice g of
// product j = chunk 4j + g of the head's row.  Idle heads read nothing.
template <int DT, int D>
__device__ __forceinline__ void load_q(const DecodeArgs& a, const HeadTile& t, const MfmaLane& ln,
                                       u32x4 (&qb)[D / 32]) {
  using S = MfmaShape<DT, D>;
  const u32x4* q = reinterpret_cast<const u32x4*>(a.q);
#pragma unroll
  for (int jj = 0; jj < S::NJ; ++jj)
    qb[jj] = (ln.n < t.nh) ? q[(t.orow0 + ln.n) * S::CPR + 4 * jj + ln.g] : u32x4{0u, 0u, 0u, 0u};
}

// A wave's finished item (the whole partition), written from registers:
// the output row when the sequence has one partition, else its partial.
template <int DT, int D>
__device__ __forceinline__ void write_wave_item(const DecodeArgs& a, MfmaState<D>& st,
                                                const HeadTile& t, int part, int nparts,
                                                const MfmaLane& ln) {
  constexpr int EPL = D / 16;
  float lsum = xor16_combine(st.lsum, AddOp{});
  lsum = xor32_combine(lsum, AddOp{});
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int hh = 4 * ln.g + e;
    const float lr = u2f((uint32_t)__builtin_amdgcn_ds_bpermute(hh << 2, (int)f2u(lsum)));
    const float inv = lr > 0.f ? 1.f / lr : 0.f;
    if (hh < t.nh) {
      if (nparts <= 1) {
#pragma unroll
        for (int jj = 0; jj < EPL; ++jj)
          store_elem<DT>(a.out, (t.orow0 + hh) * D + EPL * ln.n + jj, st.o[jj][e] * inv);
      } else {
        const int64_t prow = (t.orow0 + hh) * a.max_partitions + part;
#pragma unroll
        for (int jj = 0; jj < EPL; ++jj) a.tmp_out[prow * D + EPL * ln.n + jj] = st.o[jj][e] * inv;
      }
    }
  }
  if (nparts > 1 && ln.g == 0 && ln.n < t.nh) {
    const int64_t prow = (t.orow0 + ln.n) * a.max_partitions + part;
    a.max_logits[prow] = st.m * kLn2;
    a.exp_sums[prow] = lsum;
  }
}

// Partitions p0 .. p1 of a head tile hold no result of their own (their
// tokens were folded into an earlier slot): weight zero for the reduce.
__device__ __forceinline__ void mark_empty(const DecodeArgs& a, const HeadTile& t, int p0, int p1,
                                           const MfmaLane& ln) {
  if (ln.n >= t.nh) return;
  const int64_t row = (t.orow0 + ln.n) * a.max_partitions;
  for (int p = p0 + ln.g; p <= p1; p += 4) a.exp_sums[row + p] = 0.f;
}

// One item: head tile `unit` of sequence s over partition `part` (context
// L).  WAVE_ITEM: the calling wave alone processes the whole partition and
// writes its result from registers (no merge, no barrier); otherwise the NW
// waves share the partition's blocks and merge through LDS.  `kst` is the
// calling wave's K staging tile.
template <int DT, int D, int NW, int DEPTH, bool WAVE_ITEM, int BS = kBlockSize>
__device__ __forceinline__ void mfma_item(const DecodeArgs& a, const int unit, const int s,
                                          const int part, const int L, MfmaLds<D, NW>* sm,
                                          u32x4* kst) {
  using S = MfmaShape<DT, D>;
  using VT = typename S::VT;
  constexpr int EPL = S::EPL;
  const MfmaLane ln;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const HeadTile t = head_tile(a, unit, s);
  const int nblocks = (L + kBlockSize - 1) / kBlockSize;
  const int nparts = (nblocks + a.part_blocks - 1) / a.part_blocks;
  const int32_t* __restrict__ bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;

  // Fused KV write: the first head tile of each KV head, in the partition
  // holding the context's end, stores the new token's row; every item takes
  // the row from registers where its context ends with that slot.  K: this
  // lane's chunk of the row in the load layout (chunk lane % CPR); V: its
  // slice n in the P.V operand layout.
  constexpr int RB = D * 2;  // bytes of one K or V row
  const int hchunks = (a.num_q_heads / a.num_kv_heads + 15) >> 4;
  const NewToken nt = new_token<BS>(a, bt, s, t.kvh, L,
                                    unit % hchunks == 0 && part == max(nparts, 1) - 1, RB);
  const int lane = ln.n + 16 * ln.g;
  const u32x4 nkc = buf_load16(new_row_rsrc(a, a.new_k, s, t.kvh, RB), (lane % S::CPR) * 16);
  const VT nvc = S::VS::template load<false>(new_row_rsrc(a, a.new_v, s, t.kvh, RB),
                                             EPL * ln.n * 2);
  auto store_new = [&]() {
    if (nt.store && (WAVE_ITEM || w == 0)) {
      if (lane < S::CPR) store_row_part(a.k_cache, nt.off + lane * 16, nkc);
      if (ln.g == 0) store_row_part(a.v_cache, nt.off + EPL * ln.n * 2, nvc);
    }
  };

  if (L == 0) {
    const int t0 = WAVE_ITEM ? (int)(threadIdx.x & 63) : (int)threadIdx.x;
    const int tn = WAVE_ITEM ? 64 : NW * 64;
    for (int i = t0; i < t.nh * D; i += tn) store_elem<DT>(a.out, t.orow0 * D + i, 0.f);
    store_new();
    return;
  }
  u32x4 qb[S::NJ];
  load_q<DT, D>(a, t, ln, qb);
  // Shared-prefix launches (one pass): the leading `pre` blocks were done by
  // the prefix kernel; their state joins the merge below.
  const int pre = (!WAVE_ITEM && a.prefix_blocks != nullptr) ? a.prefix_blocks[s] : 0;
  const int jb = max(part * a.part_blocks, pre);
  const int je = min(part * a.part_blocks + a.part_blocks, nblocks);
  constexpr int STRIDE = WAVE_ITEM ? 1 : NW;
  const int j0 = jb + (WAVE_ITEM ? 0 : w);                         // blocks j0, j0+STRIDE, ...
  const int nk = je > j0 ? (je - j0 + STRIDE - 1) / STRIDE : 0;  // how many

  MfmaState<D> st;
  st.reset();

  // Pool ids of the wave's kk-th 16-token tile (index clamped into the row).
  auto id_at = [&](int kk) {
    return tile_ids<BS>(bt, j0 + min(kk, nk - 1) * STRIDE, a.max_blocks_per_seq);
  };
  // Descriptors of the wave's kk-th tile and the number of its tokens in the
  // context; empty past the wave's last tile, and tokens in a block outside
  // the pool do not count.
  auto tile = [&](int kk, const TileIds<BS>& ids, int& limit, int& tj) {
    const int j = j0 + min(kk, nk - 1) * STRIDE;
    const bool ok = kk < nk;
    limit = ok ? tile_limit<BS>(a, ids, L - j * kBlockSize) : 0;
    tj = ok ? j : -1;
    return tile_desc<BS, S::TILE_BYTES>(a, ids, j, t.kvh, ok);
  };
  // The context's last token is the new one: its K row (load jj, lane l =
  // row (64 jj + l) / CPR) and V row (slice e = row g + 4e) come from registers.
  auto substitute = [&](u32x4 (&kr)[S::NJ], VT (&vr)[4], int tj) {
    if (nt.sub && tj == nt.tile) {
#pragma unroll
      for (int jj = 0; jj < S::NJ; ++jj)
        if ((jj * 64 + lane) / S::CPR == nt.row) kr[jj] = nkc;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (ln.g + 4 * e == nt.row) vr[e] = nvc;
    }
  };

  // Software pipeline over the wave's blocks: DEPTH register sets; while
  // block k is consumed, the loads of blocks k+1 .. k+DEPTH-1 are in flight,
  // and the pool id of the next block to issue is already being fetched.
  // Every step issues its loads (empty past the end) so that the wait counts
  // are the same on every path -- no branch around a load -- and a
  // past-the-end step consumes nothing.
  u32x4 kr[DEPTH][S::NJ];
  VT vr[DEPTH][4];
  int lim[DEPTH], tjs[DEPTH];
  auto pipeline = [&](auto shared) {
    constexpr bool SH = decltype(shared)::value;
    static_for<0, DEPTH - 1>([&](auto dc) {
      constexpr int d = decltype(dc)::value;
      load_tile<DT, D, SH>(tile(d, id_at(d), lim[d], tjs[d]), ln, kr[d], vr[d]);
    });
    TileIds<BS> next_id = id_at(DEPTH - 1);
    for (int k = 0; k < nk; k += DEPTH) {
      static_for<0, DEPTH>([&](auto dc) {
        constexpr int d = decltype(dc)::value;
        constexpr int dn = (d + DEPTH - 1) % DEPTH;
        const int kn = k + d + DEPTH - 1;  // tile whose loads are issued now
        const TileIds<BS> id = next_id;
        next_id = id_at(kn + 1);
        load_tile<DT, D, SH>(tile(kn, id, lim[dn], tjs[dn]), ln, kr[dn], vr[dn]);
        substitute(kr[d], vr[d], tjs[d]);
        consume_any<DT, D>(st, qb, kr[d], vr[d], lim[d], a.scale_log2, ln, kst);
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
    write_wave_item<DT, D>(a, st, t, part, nparts, ln);
    return;
  }
  // Per-head totals of this wave, then the cross-wave merge through LDS.
  const int n = ln.n, g = ln.g;
  float lsum = xor16_combine(st.lsum, AddOp{});
  lsum = xor32_combine(lsum, AddOp{});
  if (g == 0) {
    sm->m[w][n] = st.m;
    sm->l[w][n] = lsum;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int jj = 0; jj < EPL; ++jj) sm->o[w][4 * g + e][EPL * n + jj] = st.o[jj][e];
  __syncthreads();
  if (threadIdx.x < 16) {
    const int hh = threadIdx.x;
    const bool hp = pre > 0 && hh < t.nh;
    const float pm = hp ? a.prefix_m[t.orow0 + hh] : -INFINITY;
    float M = pm;
#pragma unroll
    for (int i = 0; i < NW; ++i) M = __builtin_fmaxf(M, sm->m[i][hh]);
    float tot = 0.f;
    float f[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      f[i] = (sm->m[i][hh] == -INFINITY) ? 0.f : fast_exp2(sm->m[i][hh] - M);
      tot += sm->l[i][hh] * f[i];
    }
    const float wp = hp ? a.prefix_l[t.orow0 + hh] * fast_exp2(pm - M) : 0.f;
    tot += wp;
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) sm->f[i][hh] = f[i] * inv;
    sm->fp[hh] = wp * inv;
    sm->tot[hh] = tot;
    sm->mx[hh] = M;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < t.nh * D; i += NW * 64) {
    const int hh = i / D, d = i % D;
    float v = pre > 0 ? sm->fp[hh] * a.prefix_o[(t.orow0 + hh) * D + d] : 0.f;
#pragma unroll
    for (int k = 0; k < NW; ++k) v += sm->o[k][hh][d] * sm->f[k][hh];
    if (nparts <= 1) {
      store_elem<DT>(a.out, (t.orow0 + hh) * D + d, v);
    } else {
      const int64_t prow = (t.orow0 + hh) * a.max_partitions + part;
      a.tmp_out[prow * D + d] = v;
      if (d == 0) {
        a.max_logits[prow] = sm->mx[hh] * kLn2;
        a.exp_sums[prow] = sm->tot[hh];
      }
    }
  }
}

// One workgroup per item.  Head units vary fastest across the grid:
// workgroups are dealt to the 8 XCDs round-robin, so the equal-sized items of
// one (sequence, partition) spread evenly over the XCDs, and one head unit of
// every sequence stays on one XCD (shared prefix pages then hit its L2).
template <int DT, int D, int NW, int DEPTH, int BS>
__global__ __launch_bounds__(NW * 64) void decode_mfma_kernel(DecodeArgs a) {
  __shared__ MfmaLds<D, NW> sm;
  __shared__ u32x4 kst[NW][kKStageSlots<D>];
  const int unit = blockIdx.x, s = longest_first(a, blockIdx.y), part = blockIdx.z;
  const int L = clamp_len(a, s);
  if (part >= parts_of(L, a.part_blocks)) return;  // past this sequence's end
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  mfma_item<DT, D, NW, DEPTH, false, BS>(a, unit, s, part, L, &sm, kst[w]);
}

// One wave per item: wave w of workgroup z takes partition z * NW + w, for
// launches with many partitions per sequence.
template <int DT, int D, int NW, int DEPTH>
__global__ __launch_bounds__(NW * 64) void decode_mfma_wave_kernel(DecodeArgs a) {
  __shared__ u32x4 kst[NW][kKStageSlots<D>];
  const int unit = blockIdx.x, s = longest_first(a, blockIdx.y);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int part = blockIdx.z * NW + w;
  const int L = clamp_len(a, s);
  if (part >= parts_of(L, a.part_blocks)) return;  // past this sequence's end
  mfma_item<DT, D, NW, DEPTH, true>(a, unit, s, part, L, nullptr, kst[w]);
}

// Streaming mode: position of a worker in the compact item list
// (sequence-major, then head unit, then partition) and in the blocks of the
// current item.  Every field is wave-uniform; the per-block step is one
// increment and compare, everything else happens at item boundaries.
//
// The table and length pointers come from the kernel's __restrict__
// arguments: the loop also stores results, and only loads known not to alias
// those stores become scalar loads (a vector load of a block id would make
// every step wait for all tile loads in flight).
struct StreamCursor {
  int s, unit, part, nparts, len, nblocks;
  int j, jend;    // current block, end of the item's blocks (>= j + 1)
  int left;       // items of the worker's range from the current one on
  int kvh;        // KV head of `unit`
  bool new_tile;  // the head tile changed at the last item boundary
  int64_t row;    // offset of sequence s's block-table row (an offset, not a pointer:
                  // loads must stay visibly based on the kernel argument)

  __device__ __forceinline__ void enter_item(const DecodeArgs& a) {
    j = part * a.part_blocks;
    jend = max(j + 1, min(j + a.part_blocks, nblocks));  // an empty context still takes a step
  }
  __device__ __forceinline__ void enter_seq(const DecodeArgs& a, const int32_t* tables,
                                            const int32_t* lens) {
    len = min(max(lens[s], 0), a.max_len);
    nblocks = (len + kBlockSize - 1) / kBlockSize;
    nparts = parts_of(len, a.part_blocks);
    row = (int64_t)s * a.max_blocks_per_seq;
  }
  __device__ __forceinline__ bool last_block() const { return j + 1 >= jend; }
  // Step to the next block (and item, head unit, sequence as they end).
  __device__ __forceinline__ void advance(const DecodeArgs& a, const int32_t* tables,
                                          const int32_t* lens, int units, int hchunks) {
    if (++j < jend) return;
    --left;
    if (++part == nparts) {
      part = 0;
      new_tile = true;
      if (++unit == units) {
        unit = 0;
        if (s + 1 < a.num_seqs) ++s;
        enter_seq(a, tables, lens);
      }
      kvh = unit / hchunks;
    }
    enter_item(a);
  }
};

// Inclusive prefix sum over the 64 lanes of the wave.
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __builtin_amdgcn_ds_bpermute(((lane - off) & 63) << 2, x);
    x += lane >= off ? y : 0;
  }
  return x;
}

// Streaming mode, for launches with many partitions and few sequences: every
// resident wave is a worker that takes an equal contiguous share of the
// compact item list and streams the blocks of all its items through one
// load pipeline, writing each item's partial (or output row) as soon as its
// last block is consumed.  No workgroup is ever empty, no item pays a
// pipeline start-up, and the partitions stay exactly the ones the reduce
// merges.  The launch keeps the item count below 2^31.
template <int DT, int D, int NW, int DEPTH>
#ifndef PA_STREAM_MIN_WAVES
#define PA_STREAM_MIN_WAVES 2  // waves per SIMD the register budget must allow
#endif
__global__ __launch_bounds__(NW * 64, PA_STREAM_MIN_WAVES) void decode_mfma_stream_kernel(
    DecodeArgs a, const int32_t* __restrict__ tables, const int32_t* __restrict__ lens) {
  using S = MfmaShape<DT, D>;
  using VT = typename S::VT;
  __shared__ u32x4 kst_all[NW][kKStageSlots<D>];
  const MfmaLane ln;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int group = a.num_q_heads / a.num_kv_heads;
  const int hchunks = (group + 15) >> 4;
  const int units = a.num_kv_heads * hchunks;
  u32x4* kst = kst_all[w];

  // Item counts of the sequences, 64 at a time, summed across the lanes:
  // the total, then the sequence holding this worker's first item.
  int total = 0;
  for (int s0 = 0; s0 < a.num_seqs; s0 += 64) {
    const int s = s0 + lane;
    const int n = s < a.num_seqs ? units * parts_of(min(max(lens[s], 0), a.max_len), a.part_blocks)
                                 : 0;
    total += __builtin_amdgcn_readlane(wave_inclusive_sum(n), 63);
  }
  const int workers = gridDim.x * NW;
  const int wid = blockIdx.x * NW + w;
  const int i0 = (int)((int64_t)total * wid / workers);
  const int i1 = (int)((int64_t)total * (wid + 1) / workers);
  if (i0 >= i1) return;

  StreamCursor lc;  // load cursor (runs DEPTH-1 steps ahead of the consume cursor)
  {
    int cum = 0, seq = a.num_seqs - 1;
    for (int s0 = 0; s0 < a.num_seqs; s0 += 64) {
      const int s = s0 + lane;
      const int n = s < a.num_seqs
                        ? units * parts_of(min(max(lens[s], 0), a.max_len), a.part_blocks)
                        : 0;
      const int incl = cum + wave_inclusive_sum(n);
      // sequences of this chunk that end at or before item i0
      const uint64_t done = __builtin_amdgcn_ballot_w64(s < a.num_seqs && incl <= i0);
      const int k = __builtin_popcountll(done);
      if (k < 64) {  // sequence s0 + k holds item i0
        seq = s0 + k;
        cum = k > 0 ? __builtin_amdgcn_readlane(incl, k - 1) : cum;
        break;
      }
      cum = __builtin_amdgcn_readlane(incl, 63);
    }
    lc.s = min(seq, a.num_seqs - 1);
    lc.enter_seq(a, tables, lens);
    const int r = i0 - cum;
    lc.unit = r / lc.nparts;
    lc.part = r % lc.nparts;
    lc.kvh = lc.unit / hchunks;
    lc.left = i1 - i0;
    lc.new_tile = false;
    lc.enter_item(a);
  }
  StreamCursor cc = lc;  // consume cursor

  // Fused KV write (as in the items): each head tile's sequence's new row
  // for the tile's KV head is loaded just before the tile's query (so the
  // wait for q covers it); the tile holding the context's last position
  // takes the row from registers where the slot is that position, and the
  // item of the last partition of the KV head's first head chunk stores it.
  constexpr int RB = D * 2;  // bytes of one K or V row
  NewToken nt;
  u32x4 nkc;
  VT nvc;
  auto new_row = [&]() {
    nt = new_token<kBlockSize>(a, tables + cc.row, cc.s, cc.kvh, cc.len, true, RB);
    nkc = buf_load16(new_row_rsrc(a, a.new_k, cc.s, cc.kvh, RB), (lane % S::CPR) * 16);
    nvc = S::VS::template load<false>(new_row_rsrc(a, a.new_v, cc.s, cc.kvh, RB),
                                      S::EPL * ln.n * 2);
  };
  new_row();
  HeadTile t = head_tile(a, cc.unit, cc.s);
  u32x4 qb[S::NJ];
  load_q<DT, D>(a, t, ln, qb);
  MfmaState<D> st;
  st.reset();
  int seg_part0 = cc.part;  // first partition of the open segment

  u32x4 kr[DEPTH][S::NJ];
  VT vr[DEPTH][4];
  int lim[DEPTH];
  // Issue the loads of the load cursor's block (empty once past this
  // worker's range) and step the cursor.
  auto issue = [&](int slot, int bid) {
    const bool live = lc.left > 0;
    const bool ok = live && lc.j < lc.nblocks && (uint32_t)bid < (uint32_t)a.num_blocks_i32;
    lim[slot] = ok ? min(kBlockSize, lc.len - lc.j * kBlockSize) : 0;
    load_tile<DT, D, false>(tile_desc<kBlockSize, S::TILE_BYTES>(a, TileIds<kBlockSize>{{bid}},
                                                                 lc.j, lc.kvh, ok),
                            ln, kr[slot], vr[slot]);
    if (live) lc.advance(a, tables, lens, units, hchunks);
  };
  auto id_of = [&](const StreamCursor& c) -> int {
    return (c.left > 0 && c.j < c.nblocks) ? tables[c.row + c.j] : 0;
  };

  static_for<0, DEPTH - 1>([&](auto dc) { issue(decltype(dc)::value, id_of(lc)); });
  int next_id = id_of(lc);
  bool running = true;
  while (running) {
    static_for<0, DEPTH>([&](auto dc) {
      constexpr int d = decltype(dc)::value;
      constexpr int dn = (d + DEPTH - 1) % DEPTH;
      const int id = next_id;
      issue(dn, id);
      next_id = id_of(lc);
      if (running) {
        if (cc.new_tile) {  // a new head tile: its query (and new row)
          new_row();
          t = head_tile(a, cc.unit, cc.s);
          load_q<DT, D>(a, t, ln, qb);
          // Wait for q here, on this rare path: left pending past the
          // branch, it would make every step wait for all loads in flight.
          wait_loaded(qb);
          cc.new_tile = false;
        }
        if (nt.sub && cc.j == nt.tile) {  // the context's last token is the new one
#pragma unroll
          for (int jj = 0; jj < S::NJ; ++jj)
            if ((jj * 64 + lane) / S::CPR == nt.row) kr[d][jj] = nkc;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (ln.g + 4 * e == nt.row) vr[d][e] = nvc;
        }
        consume_any<DT, D>(st, qb, kr[d], vr[d], lim[d], a.scale_log2, ln, kst);
        bool closed = false;
        if (cc.last_block()) {
          // Consecutive partitions of one head tile in this worker's range
          // are one segment: the softmax state runs on, and the segment's
          // merged partial goes to the slot of its first partition, the
          // others marked empty.  Stores are few (one partial per head tile
          // per worker) and so are the waits that follow them.
          const bool more = cc.left > 1;
          if (!(more && cc.part + 1 < cc.nparts)) {
            if (cc.len == 0) {  // empty context: zero row
              for (int i = lane; i < t.nh * D; i += 64)
                store_elem<DT>(a.out, t.orow0 * D + i, 0.f);
            } else {
              write_wave_item<DT, D>(a, st, t, seg_part0, cc.nparts, ln);
              mark_empty(a, t, seg_part0 + 1, cc.part, ln);
            }
            if (nt.store && cc.unit % hchunks == 0 && cc.part == cc.nparts - 1) {
              if (lane < S::CPR) store_row_part(a.k_cache, nt.off + lane * 16, nkc);
              if (ln.g == 0) store_row_part(a.v_cache, nt.off + S::EPL * ln.n * 2, nvc);
            }
            st.reset();
            running = more;
            closed = true;
          }
        }
        cc.advance(a, tables, lens, units, hchunks);
        if (closed) seg_part0 = cc.part;
      }
    });
  }
}

#ifndef PA_MFMA_WAVE_ITEM_WAVES
#define PA_MFMA_WAVE_ITEM_WAVES 4  // waves (= partitions) per workgroup, one-wave items
#endif
#ifndef PA_MFMA_WAVE_ITEM_DEPTH
#define PA_MFMA_WAVE_ITEM_DEPTH 3  // tiles per wave in the load pipeline, one-wave items
#endif

// Launch shapes: items of at least kLongItemBlocks blocks get 8 waves,
// shorter ones 4 (more workgroups resident per CU).
constexpr int kLongItemBlocks = 128;
#ifndef PA_MFMA_LONG_WAVES
#define PA_MFMA_LONG_WAVES 8
#endif
#ifndef PA_MFMA_LONG_DEPTH
#define PA_MFMA_LONG_DEPTH 2
#endif

template <int DT, int D, int NW, int DEPTH, int BS = kBlockSize>
hipError_t launch_shape(const DecodeArgs& a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  const dim3 grid(a.num_kv_heads * ((group + 15) / 16), a.num_seqs, a.max_partitions);
  hipLaunchKernelGGL((decode_mfma_kernel<DT, D, NW, DEPTH, BS>), grid, dim3(NW * 64), 0, stream,
                     a);
  return hipGetLastError();
}

// Launches with at least kWaveItemParts partitions take one wave per item;
// with at most kStreamMaxSeqs sequences as well, the streaming mode.
#ifndef PA_WAVE_ITEM_PARTS
#define PA_WAVE_ITEM_PARTS 8
#endif
constexpr int kWaveItemParts = PA_WAVE_ITEM_PARTS;
#ifndef PA_STREAM_MAX_SEQS
#define PA_STREAM_MAX_SEQS 64
#endif
#ifndef PA_MFMA_STREAM_WAVES
#define PA_MFMA_STREAM_WAVES 4  // waves per workgroup, streaming mode
#endif
#ifndef PA_MFMA_STREAM_DEPTH
#define PA_MFMA_STREAM_DEPTH 2  // tiles per wave in the load pipeline, streaming mode
#endif
constexpr int kStreamMaxSeqs = PA_STREAM_MAX_SEQS;

template <int DT, int D, int NW, int DEPTH>
hipError_t launch_wave_shape(const DecodeArgs& a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  const dim3 grid(a.num_kv_heads * ((group + 15) / 16), a.num_seqs,
                  (a.max_partitions + NW - 1) / NW);
  hipLaunchKernelGGL((decode_mfma_wave_kernel<DT, D, NW, DEPTH>), grid, dim3(NW * 64), 0, stream,
                     a);
  return hipGetLastError();
}

#ifndef PA_STREAM_WG_PER_CU
#define PA_STREAM_WG_PER_CU 1  // streaming workgroups per compute unit
#endif

// One streaming workgroup per compute unit (never more than are resident):
// measured on the long-context shape, fewer workers with longer ranges beat
// filling every wave slot, and a grid that is not a multiple of the CU count
// leaves some CUs with twice the work.
template <int DT, int D, int NW, int DEPTH>
hipError_t launch_stream_shape(const DecodeArgs& a, int64_t items, hipStream_t stream) {
  const auto kernel = decode_mfma_stream_kernel<DT, D, NW, DEPTH>;
  static ResidentCache cache;
  const int resident = resident_workgroups(reinterpret_cast<const void*>(kernel), NW * 64, cache);
  const int cus = compute_units();
  if (resident <= 0 || cus <= 0) return hipErrorInvalidValue;
  const int grid = std::min(resident, cus * PA_STREAM_WG_PER_CU);
  const int64_t need = (items + NW - 1) / NW;  // never more workers than items
  hipLaunchKernelGGL(kernel, dim3((unsigned)(need < grid ? need : grid)), dim3(NW * 64), 0,
                     stream, a, a.block_tables, a.context_lens);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  // 8- and 32-token blocks: workgroup-per-item kernels for every launch.
  if (a.block_size == 8)
    return a.part_blocks >= kLongItemBlocks ? launch_shape<DT, D, 8, 2, 8>(a, stream)
                                            : launch_shape<DT, D, 4, 2, 8>(a, stream);
  if (a.block_size == 32)
    return a.part_blocks >= kLongItemBlocks ? launch_shape<DT, D, 8, 2, 32>(a, stream)
                                            : launch_shape<DT, D, 4, 2, 32>(a, stream);
  const int group = a.num_q_heads / a.num_kv_heads;
  const int64_t items = (int64_t)a.num_kv_heads * ((group + 15) / 16) * a.num_seqs *
                        a.max_partitions;
  if (decode_mfma_streams(a)) {
    return launch_stream_shape<DT, D, PA_MFMA_STREAM_WAVES, PA_MFMA_STREAM_DEPTH>(a, items, stream);
  }
  if (a.max_partitions >= kWaveItemParts)
    return launch_wave_shape<DT, D, PA_MFMA_WAVE_ITEM_WAVES, PA_MFMA_WAVE_ITEM_DEPTH>(a, stream);
  return a.part_blocks >= kLongItemBlocks
             ? launch_shape<DT, D, PA_MFMA_LONG_WAVES, PA_MFMA_LONG_DEPTH>(a, stream)
             : launch_shape<DT, D, 4, 2>(a, stream);
}

}  // namespace

bool decode_mfma_streams(const DecodeArgs& a) {
  if (a.block_size != kBlockSize) return false;
  const int group = a.num_q_heads / a.num_kv_heads;
  const int64_t items = (int64_t)a.num_kv_heads * ((group + 15) / 16) * a.num_seqs *
                        a.max_partitions;
  return a.max_partitions >= kWaveItemParts && a.num_seqs <= kStreamMaxSeqs && items < INT32_MAX;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int dtype, int head_dim, hipStream_t stream) {
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
