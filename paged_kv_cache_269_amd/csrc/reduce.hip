// Split-K merge of partition partials (log-sum-exp reduce).
//
// Each partition p of a (sequence, query head) row leaves its score max m_p,
// its sum l_p = sum exp(z - m_p) and its normalised output o_p.  Because
// exp(z - M) = exp(z - m_p) exp(m_p - M), softmax over the whole context is
//   out = sum_p w_p o_p / sum_p w_p,   w_p = l_p exp(m_p - M),  M = max_p m_p.
// This is the merge the long-context path needs once a context is cut into
// partitions processed in parallel; it runs after the decode kernel on the
// same stream.
//
// Up to 64 partitions per row: one wave per row (reduce_rows_kernel).
// More: one workgroup (512 lanes) per (query head, sequence): of up to 512
// partitions at a time, those with weight are compacted into LDS (index and
// weight; slots left empty by a kernel that folded several partitions into
// one are never read), then 512 / head_dim lane groups each sweep a share of
// them over all head_dim columns (coalesced reads of tmp_out rows, kUnroll
// independent loads in flight per lane), and the shares are added at the
// end.
#include "common.h"
#include "launch.h"

namespace pa {

namespace {

constexpr int kThreads = 512;
constexpr int kUnroll = 8;

__device__ __forceinline__ float block_max(float x, float* scratch) {
  x = group_reduce<64>(x, MaxOp{});
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) scratch[w] = x;
  __syncthreads();
  float r = scratch[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) r = __builtin_fmaxf(r, scratch[i]);
  __syncthreads();
  return r;
}

template <int DT, int D>
__global__ __launch_bounds__(kThreads) void reduce_kernel(ReduceArgs a) {
  constexpr int SPLIT = kThreads / D;
  const int h = blockIdx.x, s = blockIdx.y;
  const int tid = threadIdx.x;
  int L = a.context_lens[s];
  L = L < 0 ? 0 : (L > a.max_len ? a.max_len : L);
  const int P = (L + a.partition_size - 1) / a.partition_size;
  if (a.skip_single && P <= 1) return;
  const int64_t orow = (int64_t)s * a.num_q_heads + h;
  const int64_t base = orow * a.max_partitions;

  __shared__ float s_w[kThreads];
  __shared__ int s_p[kThreads];
  __shared__ int s_cnt[kThreads / 64];
  __shared__ float s_red[kThreads / 64];
  __shared__ float s_o[SPLIT][D];
  __shared__ float s_ws[SPLIT];

  float mx = -INFINITY;
  for (int p = tid; p < P; p += kThreads) {
    const float l = a.exp_sums[base + p];
    if (l > 0.f) mx = __builtin_fmaxf(mx, a.max_logits[base + p]);
  }
  const float M = block_max(mx, s_red);

  const int d = tid % D, share = tid / D;
  const int lane = tid & 63, wave = tid >> 6;
  float o = 0.f, wsum = 0.f;
  for (int p0 = 0; p0 < P; p0 += kThreads) {
    const int p = p0 + tid;
    float wv = 0.f;
    if (p < P) {
      const float l = a.exp_sums[base + p];
      if (l > 0.f) wv = l * fast_exp2((a.max_logits[base + p] - M) * kLog2e);
    }
    // Compact the partitions with weight into s_w / s_p (in partition
    // order): weightless ones -- the empty slots of folded partitions --
    // are not read at all.
    const uint64_t has = __builtin_amdgcn_ballot_w64(wv > 0.f);
    if (lane == 0) s_cnt[wave] = __builtin_popcountll(has);
    __syncthreads();
    int before = 0, cnt = 0;
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) {
      before += i < wave ? s_cnt[i] : 0;
      cnt += s_cnt[i];
    }
    if (wv > 0.f) {
      const int k = before + __builtin_amdgcn_mbcnt_hi((uint32_t)(has >> 32),
                                                       __builtin_amdgcn_mbcnt_lo((uint32_t)has, 0));
      s_w[k] = wv;
      s_p[k] = p;
    }
    __syncthreads();
    for (int k = share; k < cnt; k += SPLIT * kUnroll) {
      float t[kUnroll], wk[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {  // loads issued unconditionally (index kept in range)
        const int kk = k + u * SPLIT;
        const bool in = kk < cnt;
        const int ki = in ? kk : share;
        wk[u] = in ? s_w[ki] : 0.f;
        t[u] = a.tmp_out[(base + s_p[ki]) * D + d];
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        wsum += wk[u];
        o += wk[u] * t[u];
      }
    }
    __syncthreads();
  }
  s_o[share][d] = o;
  if (d == 0) s_ws[share] = wsum;
  __syncthreads();
  if (tid < D) {
    float ot = 0.f, wt = 0.f;
#pragma unroll
    for (int i = 0; i < SPLIT; ++i) {
      ot += s_o[i][tid];
      wt += s_ws[i];
    }
    store_elem<DT>(a.out, orow * D + tid, wt > 0.f ? ot / wt : 0.f);
  }
}

// Many rows with few partitions each (multi-token queries: a row per query
// token and head): one wave per row, kRowsPerGroup rows per workgroup.  Lane
// l holds columns kCols l .. kCols l + kCols - 1; partition p's weight is
// computed by lane p % 64 and broadcast; kRowUnroll partition rows are
// loaded at a time.  Slots without weight (empty, possibly never written)
// are dropped by selection, never multiplied in.
constexpr int kRowsPerGroup = 4;
constexpr int kRowUnroll = 4;
constexpr int kRowsMaxPartitions = 64;

template <int DT, int D>
__global__ __launch_bounds__(64 * kRowsPerGroup) void reduce_rows_kernel(ReduceArgs a,
                                                                          int num_rows) {
  constexpr int C = D / 64;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerGroup + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= num_rows) return;
  const int s = row / a.num_q_heads;
  int L = a.context_lens[s];
  L = L < 0 ? 0 : (L > a.max_len ? a.max_len : L);
  const int P = (L + a.partition_size - 1) / a.partition_size;
  if (a.skip_single && P <= 1) return;
  const int64_t base = (int64_t)row * a.max_partitions;

  // P <= kRowsMaxPartitions: one partition per lane
  const bool mine = lane < P;
  const float l = mine ? a.exp_sums[base + lane] : 0.f;
  const float m = mine ? a.max_logits[base + lane] : -INFINITY;
  const float M = group_reduce<64>(l > 0.f ? m : -INFINITY, MaxOp{});
  const float wv = l > 0.f ? l * fast_exp2((m - M) * kLog2e) : 0.f;
  const float wsum = group_sum<64>(wv);

  float o[C];
#pragma unroll
  for (int c = 0; c < C; ++c) o[c] = 0.f;
  const float* __restrict__ t0 = a.tmp_out + base * D + C * lane;
  for (int p0 = 0; p0 < P; p0 += kRowUnroll) {
    float t[kRowUnroll][C], w[kRowUnroll];
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {  // loads issued unconditionally (index kept in range)
      const int p = min(p0 + u, P - 1);
      w[u] = p0 + u < P ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                        __builtin_bit_cast(int, wv), p))
                        : 0.f;
#pragma unroll
      for (int c = 0; c < C; ++c) t[u][c] = t0[(int64_t)p * D + c];
    }
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u)
#pragma unroll
      for (int c = 0; c < C; ++c) o[c] += w[u] > 0.f ? w[u] * t[u][c] : 0.f;
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
  for (int c = 0; c < C; ++c) store_elem<DT>(a.out, (int64_t)row * D + C * lane + c, o[c] * inv);
}

template <int DT, int D>
hipError_t launch_typed(const ReduceArgs& a, int num_seqs, hipStream_t stream) {
  if (a.max_partitions <= kRowsMaxPartitions) {
    const int rows = num_seqs * a.num_q_heads;
    hipLaunchKernelGGL((reduce_rows_kernel<DT, D>),
                       dim3((rows + kRowsPerGroup - 1) / kRowsPerGroup), dim3(64 * kRowsPerGroup),
                       0, stream, a, rows);
  } else {
    hipLaunchKernelGGL((reduce_kernel<DT, D>), dim3(a.num_q_heads, num_seqs), dim3(kThreads), 0,
                       stream, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs& a, int dtype, int head_dim, int num_seqs,
                         hipStream_t stream) {
  clear_stale_error();
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
