// Shared-prefix pass of a cascade decode.
//
// The pages' prefix sharing ("vLLM 2026 推理引擎全解" (chenxutan.com) §2.1 and
// §2.3; the vLLM manual (doramagic.ai), "sharing mechanism") maps the same
// physical blocks into the tables of many sequences.  Attention over such a
// block is the same small product for every sequence that maps it, with only
// the query changing, so it can be done once for a group of sequences with
// their queries as the rows of one matrix-core tile: S = K_blk . Q^T over
// (sequence, query head) rows, O += P . V_blk (mfma_tile.h).
//
// Groups are fixed runs of 16 / G consecutive sequences (G query heads per
// KV head, G <= 8): a tile's 16 rows are the G heads of those sequences.  A
// group's prefix is the number of leading table entries that all members
// share and that lie inside every member's context as whole blocks.  Groups
// with fewer than kMinPrefixBlocks such blocks (or a single member) leave
// everything to the decode kernel.  Each (KV head, group) workgroup writes,
// per row, the base-2 max, the sum of exponentials and the normalised output
// of the prefix part, and per sequence the prefix length in blocks; the
// decode kernel then covers the remaining blocks and merges the two parts
// with the same log-sum-exp rule as the split-K reduce.
#include <climits>
#include <type_traits>

#include "common.h"
#include "items.h"
#include "launch.h"
#include "mfma_tile.h"

namespace pa {

namespace {

constexpr int kMinPrefixBlocks = 4;

// Most sequences in one run (16 query rows, at least one head each).
constexpr int kMaxRunSeqs = 16;

// Leading full blocks that sequences s0 .. s0+ns-1 all map to the same
// physical blocks (0 when fewer than kMinPrefixBlocks or ns < 2).  Every wave
// computes it: the members' lengths and the first 128 entries of all their
// table rows are loaded together (one round trip: every load is issued
// before the first compare; rows past the run repeat its last member),
// mismatches found with ballots; longer shared parts continue 64 entries at
// a time.  No barrier is needed.
__device__ __forceinline__ int group_prefix_blocks(const DecodeArgs& a, int s0, int ns) {
  if (ns < 2) return 0;
  const int lane = threadIdx.x & 63;
  const int M = a.max_blocks_per_seq;
  const int32_t* r0 = a.block_tables + (int64_t)s0 * M;
  const int lb = lane < ns ? clamp_len(a, s0 + lane) / kBlockSize : INT_MAX;
  const int c0 = min(lane, M - 1), c1 = min(64 + lane, M - 1);  // entries, clamped into the row
  const int ref0 = r0[c0], ref1 = r0[c1];
  int e0[kMaxRunSeqs - 1], e1[kMaxRunSeqs - 1];
#pragma unroll
  for (int i = 1; i < kMaxRunSeqs; ++i) {
    const int32_t* r = r0 + (int64_t)min(i, ns - 1) * M;
    e0[i - 1] = r[c0];
    e1[i - 1] = r[c1];
  }
  bool d0 = false, d1 = false;
#pragma unroll
  for (int i = 1; i < kMaxRunSeqs; ++i) {
    d0 |= e0[i - 1] != ref0;
    d1 |= e1[i - 1] != ref1;
  }
  d0 = d0 && lane < M;
  d1 = d1 && 64 + lane < M;
  int full = M;  // whole blocks in every member's context
  for (int i = 0; i < ns; ++i) full = min(full, __builtin_amdgcn_readlane(lb, i));
  if (full < kMinPrefixBlocks) return 0;
  int P = full;
  const uint64_t m0 = __builtin_amdgcn_ballot_w64(d0 && lane < full);
  const uint64_t m1 = __builtin_amdgcn_ballot_w64(d1 && 64 + lane < full);
  if (m0 != 0) {
    P = __builtin_ctzll(m0);
  } else if (m1 != 0) {
    P = 64 + __builtin_ctzll(m1);
  } else {
    for (int j0 = 128; j0 < full; j0 += 64) {
      const int j = j0 + lane;
      bool diff = false;
      if (j < full) {
        const int ref = r0[j];
        for (int i = 1; i < ns; ++i) diff |= r0[(int64_t)i * M + j] != ref;
      }
      const uint64_t mask = __builtin_amdgcn_ballot_w64(diff);
      if (mask != 0) {
        P = j0 + __builtin_ctzll(mask);
        break;
      }
    }
  }
  return P >= kMinPrefixBlocks ? P : 0;
}

template <int DT, int D, int NW, int DEPTH>
__global__ __launch_bounds__(NW * 64) void prefix_kernel(DecodeArgs a, PrefixOut out, KvWrite kw) {
  using S = MfmaShape<DT, D>;
  using VT = typename S::VT;
  __shared__ MfmaLds<D, NW> sm;
  __shared__ u32x4 kst_all[NW][kKStageSlots<D>];
  const MfmaLane ln;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  u32x4* kst = kst_all[w];
  const int G = a.num_q_heads / a.num_kv_heads;
  const int rs = 16 / G;  // sequences per tile
  const int kvh = blockIdx.x;
  const int s0 = blockIdx.y * rs;
  const int ns = min(rs, a.num_seqs - s0);
  // Query rows: row n is head kvh*G + n % G of sequence s0 + n / G (loaded
  // while the shared part is being measured).
  const int nrows = ns * G;
  const int64_t qrow = (int64_t)(s0 + ln.n / G) * a.num_q_heads + kvh * G + ln.n % G;
  u32x4 qb[S::NJ];
  {
    const u32x4* q = reinterpret_cast<const u32x4*>(a.q);
#pragma unroll
    for (int jj = 0; jj < S::NJ; ++jj)
      qb[jj] = ln.n < nrows ? q[qrow * S::CPR + 4 * jj + ln.g] : u32x4{0u, 0u, 0u, 0u};
  }
  // The step's KV write for this run's sequences and KV head kvh: the new K
  // and V rows to their slots (slot = block * 16 + offset, "vLLM 2026
  // 推理引擎全解" §2.2), one 16-byte chunk per work-item and row half.  Its
  // loads are issued with the table reads of the measurement below, whose
  // wait covers them.
  constexpr int WCH = kMaxRunSeqs * 2 * S::CPR;  // chunks of a full run (K and V)
  constexpr int WPT = (WCH + NW * 64 - 1) / (NW * 64);
  u32x4 wv[WPT];
  int64_t wdst[WPT];
  bool wk[WPT], wok[WPT];
  if (kw.slots != nullptr) {
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
      const int i = (int)threadIdx.x + j * NW * 64;
      const int tok = i / (2 * S::CPR), c = i % S::CPR;
      wk[j] = (i / S::CPR) % 2 == 0;
      wok[j] = tok < ns;
      if (wok[j]) {
        const int s = s0 + tok;
        const int64_t src = ((int64_t)s * a.num_kv_heads + kvh) * S::CPR + c;
        const u32x4* row = static_cast<const u32x4*>(wk[j] ? kw.key : kw.value);
        wv[j] = row[src];
        const int64_t slot = kw.slots[s];
        wok[j] = slot >= 0 && slot < kw.num_slots;
        wdst[j] = (((slot / kBlockSize) * a.num_kv_heads + kvh) * kBlockSize + slot % kBlockSize) *
                      S::CPR + c;
      }
    }
  }
  const int P = group_prefix_blocks(a, s0, ns);
  if (kw.slots != nullptr) {
#pragma unroll
    for (int j = 0; j < WPT; ++j)
      if (wok[j]) static_cast<u32x4*>(wk[j] ? kw.k_cache : kw.v_cache)[wdst[j]] = wv[j];
  }
  if (kvh == 0 && (int)threadIdx.x < ns) out.prefix_blocks[s0 + threadIdx.x] = P;
  if (P == 0) return;

  // Wave w takes prefix blocks w, w+NW, ... through a DEPTH-deep register
  // pipeline (every step issues its loads; past the end they are empty).
  // The pages are re-read by the other groups' workgroups: cached loads.
  const int32_t* bt = a.block_tables + (int64_t)s0 * a.max_blocks_per_seq;
  const int nk = w < P ? (P - w + NW - 1) / NW : 0;
  MfmaState<D> st;
  st.reset();
  u32x4 kr[DEPTH][S::NJ];
  VT vr[DEPTH][4];
  int lim[DEPTH];
  const TableRow btc = table_row(bt);
  auto id_at = [&](int kk) -> int { return btc[w + min(kk, max(nk - 1, 0)) * NW]; };
  auto issue = [&](int kk, int bid, int slot) {
    const bool ok = kk < nk && (uint32_t)bid < (uint32_t)a.num_blocks_i32;
    lim[slot] = __builtin_amdgcn_readfirstlane(ok ? kBlockSize : 0);
    load_tile<DT, D, true>(tile_desc<kBlockSize, S::TILE_BYTES>(a, TileIds<kBlockSize>{{bid}},
                                                                w + kk * NW, kvh, ok),
                           ln, kr[slot], vr[slot]);
  };
  if (nk > 0) {
    static_for<0, DEPTH - 1>([&](auto dc) {
      constexpr int d = decltype(dc)::value;
      issue(d, id_at(d), d);
    });
    int next_id = id_at(DEPTH - 1);
    for (int k = 0; k < nk; k += DEPTH) {
      static_for<0, DEPTH>([&](auto dc) {
        constexpr int d = decltype(dc)::value;
        constexpr int dn = (d + DEPTH - 1) % DEPTH;
        const int kn = k + d + DEPTH - 1;
        const int id = next_id;
        next_id = id_at(kn + 1);
        issue(kn, id, dn);
        // a tile is whole or empty (past the end, or a block outside the
        // pool): an empty one adds nothing to any row.  Folded either way
        // (with its weights dropped), so the accumulators stay in place.
        consume_tile<DT, D, kWholeOrEmpty>(st, qb, kr[d], vr[d], lim[d], a.scale_log2, ln, kst);
      });
    }
  }

  // Merge the NW waves' states per row through LDS; write the prefix state.
  float lsum = xor16_combine(st.lsum, AddOp{});
  lsum = xor32_combine(lsum, AddOp{});
  constexpr int EPL = S::EPL;
  if (ln.g == 0) {
    sm.m[w][ln.n] = st.m;
    sm.l[w][ln.n] = lsum;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int jj = 0; jj < EPL; ++jj) sm.o[w][4 * ln.g + e][EPL * ln.n + jj] = st.o[jj][e];
  __syncthreads();
  if (threadIdx.x < 16) {
    const int r = threadIdx.x;
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < NW; ++i) M = __builtin_fmaxf(M, sm.m[i][r]);
    float tot = 0.f, f[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      f[i] = (sm.m[i][r] == -INFINITY) ? 0.f : fast_exp2(sm.m[i][r] - M);
      tot += sm.l[i][r] * f[i];
    }
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) sm.f[i][r] = f[i] * inv;
    if (r < nrows) {
      const int64_t row = (int64_t)(s0 + r / G) * a.num_q_heads + kvh * G + r % G;
      out.m[row] = M;
      out.l[row] = tot;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nrows * D; i += NW * 64) {
    const int r = i / D, d = i % D;
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < NW; ++k) v += sm.o[k][r][d] * sm.f[k][r];
    const int64_t row = (int64_t)(s0 + r / G) * a.num_q_heads + kvh * G + r % G;
    out.o[row * D + d] = v;
  }
}

#ifndef PA_PREFIX_WAVES
#define PA_PREFIX_WAVES 4
#endif
#ifndef PA_PREFIX_DEPTH
#define PA_PREFIX_DEPTH 2
#endif

template <int DT, int D>
hipError_t launch_typed(const DecodeArgs& a, const PrefixOut& o, const KvWrite& w,
                        hipStream_t stream) {
  const int G = a.num_q_heads / a.num_kv_heads;
  const int rs = 16 / G;
  const dim3 grid(a.num_kv_heads, (a.num_seqs + rs - 1) / rs);
  hipLaunchKernelGGL((prefix_kernel<DT, D, PA_PREFIX_WAVES, PA_PREFIX_DEPTH>), grid,
                     dim3(PA_PREFIX_WAVES * 64), 0, stream, a, o, w);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefix(const DecodeArgs& a, const PrefixOut& o, const KvWrite& w, int dtype,
                         int head_dim, hipStream_t stream) {
  clear_stale_error();
  const int G = a.num_q_heads / a.num_kv_heads;
  if (G > 8) return hipErrorInvalidValue;
  switch (dtype * 1000 + head_dim) {
    case kF16 * 1000 + 64: return launch_typed<kF16, 64>(a, o, w, stream);
    case kF16 * 1000 + 128: return launch_typed<kF16, 128>(a, o, w, stream);
    case kBF16 * 1000 + 64: return launch_typed<kBF16, 64>(a, o, w, stream);
    case kBF16 * 1000 + 128: return launch_typed<kBF16, 128>(a, o, w, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
