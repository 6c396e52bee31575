// Device-side helpers shared by the gfx950 kernels of libpagedattn:
// element-type traits, 16-byte vector access, wave64 cross-lane reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace pa {

enum Dtype : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

constexpr int kBlockSize = 16;   // tokens per tile the kernels work on (= pool block by default)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Online softmax of the matrix-core folds: how far (base 2) a tile's max may
// pass the running max before the running max -- and with it the
// accumulators' scale -- moves.  Weights then stay below 2^slack before
// they are rounded to the 16-bit P operand.  The normaliser sums the weights
// as rounded, so the output is a weighted mean of V whose weights are off by
// their own rounding only, relative to each weight whatever its size (f16:
// 11 bits; bf16: weight and residual, ~16 bits): the slack sets how often
// the accumulators are rescaled, not the accuracy.
#ifndef PA_RESCALE_SLACK
#define PA_RESCALE_SLACK 8
#endif
constexpr float kRescaleSlack = PA_RESCALE_SLACK;
// f16 weights (5 exponent bits) fall below the smallest subnormal, 2^-24,
// 24 below the running max.  For f16 the running max is therefore kept
// kF16MaxOffset below the largest score seen: the largest weight is 2^7 (and
// with the slack at most 2^15, under the f16 limit of 65504), and a weight
// only underflows 31 below it.  The state stays self-consistent (the sum is
// taken against the same reference), so merges and exports are unchanged.
// bf16 has the exponent range of f32 and keeps the plain running max.
constexpr float kF16MaxOffset = 7.f;
template <int DT>
constexpr float kMaxOffset = DT == kF16 ? kF16MaxOffset : 0.f;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

template <int DT> struct Elem;
template <> struct Elem<kF32> { static constexpr int bytes = 4; };
template <> struct Elem<kF16> { static constexpr int bytes = 2; };
template <> struct Elem<kBF16> { static constexpr int bytes = 2; };

// ---------------------------------------------------------------------------
// element <-> float
//
// Reinterpreting casts go through these by-value helpers: with this hipcc,
// __builtin_bit_cast applied directly to an ext_vector element (v[k], v.z)
// reads element 0 instead of element k, so a vector element is always first
// copied into a scalar.

__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ f16x2 u2h2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ __forceinline__ bf16x2 u2b2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

// The two 16-bit elements of a 32-bit word, as floats (low half first).
template <int DT>
__device__ __forceinline__ void unpack2(uint32_t w, float& lo, float& hi) {
  if constexpr (DT == kF16) {
    const f16x2 h = u2h2(w);
    lo = (float)h.x;
    hi = (float)h.y;
  } else {
    lo = u2f(w << 16);
    hi = u2f(w & 0xffff0000u);
  }
}

// float -> 16-bit storage, round to nearest even.
template <int DT>
__device__ __forceinline__ uint16_t to_bits16(float x) {
  if constexpr (DT == kF16) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  } else {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
  }
}

// Store one float result into an element array of type DT.
template <int DT>
__device__ __forceinline__ void store_elem(void* base, int64_t idx, float x) {
  if constexpr (DT == kF32) {
    reinterpret_cast<float*>(base)[idx] = x;
  } else {
    reinterpret_cast<uint16_t*>(base)[idx] = to_bits16<DT>(x);
  }
}

// Dot product of two 16-byte chunks (4 f32 or 8 f16/bf16 elements), fp32
// accumulation onto acc.
template <int DT>
__device__ __forceinline__ float dot16(const u32x4& a, const u32x4& b, float acc) {
  if constexpr (DT == kF32) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      acc = __builtin_fmaf(u2f(a[k]), u2f(b[k]), acc);
  } else if constexpr (DT == kF16) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      acc = __builtin_amdgcn_fdot2(u2h2(a[k]), u2h2(b[k]), acc, false);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      acc = __builtin_amdgcn_fdot2_f32_bf16(u2b2(a[k]), u2b2(b[k]), acc, false);
  }
  return acc;
}

// acc[0..VEC) += p * chunk, VEC = 16 / element bytes.
template <int DT>
__device__ __forceinline__ void axpy16(float p, const u32x4& v, float* acc) {
  if constexpr (DT == kF32) {
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] = __builtin_fmaf(p, u2f(v[k]), acc[k]);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float lo, hi;
      unpack2<DT>(v[k], lo, hi);
      acc[2 * k] = __builtin_fmaf(p, lo, acc[2 * k]);
      acc[2 * k + 1] = __builtin_fmaf(p, hi, acc[2 * k + 1]);
    }
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// buffer loads
//
// A tile is read through a buffer descriptor covering exactly its bytes.  A
// descriptor with zero records makes every load through it return zeros
// without touching memory, so loads can be issued unconditionally (no branch
// around them -- which keeps the load counters exact) for tiles past the end
// of a wave's work or with an invalid block id.

typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kBufferWord3 = 0x00020000;  // raw 32-bit data format, no swizzle

// Cache policy of the K/V tile loads (the instruction's cache-policy bits).
// A private tile is read once per call, so it is loaded non-temporally (nt:
// streamed past cache allocation, which measurably raises gather bandwidth).
// A tile shared by several sequences (a common prefix) is re-read by each of
// them and is loaded with the default, cache-allocating policy.
#ifndef PA_KV_LOAD_POLICY
#define PA_KV_LOAD_POLICY 2   // nt
#endif
#ifndef PA_SHARED_LOAD_POLICY
#define PA_SHARED_LOAD_POLICY 0
#endif

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kBufferWord3);
}
template <bool SHARED = false>
__device__ __forceinline__ u32x4 buf_load16(Rsrc r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(
      r, (int)byte_off, 0, SHARED ? PA_SHARED_LOAD_POLICY : PA_KV_LOAD_POLICY);
}
template <bool SHARED = false>
__device__ __forceinline__ u32x2 buf_load8(Rsrc r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b64(
      r, (int)byte_off, 0, SHARED ? PA_SHARED_LOAD_POLICY : PA_KV_LOAD_POLICY);
}


// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time
// (register arrays indexed by I stay in fixed registers).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// ---------------------------------------------------------------------------
// wave64 cross-lane reductions

// DPP row controls (a DPP row is 16 lanes).
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRowMirror = 0x140; // lane i <-> 15 - i within a row
constexpr int kDppHalfMirror = 0x141;// lane i <-> 7 - i within each half row
constexpr int kDppRowRor8 = 0x128;   // lane i <-> i ^ 8 within a row (rotate by 8)

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return u2f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f2u(x), CTRL, 0xF, 0xF, false));
}

// Exchange with lane ^ 16 / lane ^ 32, combined through op.  The gfx950
// permlane swaps hand back both halves of the exchange; combining the two
// results lane-wise gives op(x[l], x[l ^ 16]) (resp. ^ 32) in every lane.
template <typename Op>
__device__ __forceinline__ float xor16_combine(float x, Op op) {
  auto r = __builtin_amdgcn_permlane16_swap(f2u(x), f2u(x), false, false);
  const uint32_t a = r[0], b = r[1];
  return op(u2f(a), u2f(b));
}
template <typename Op>
__device__ __forceinline__ float xor32_combine(float x, Op op) {
  auto r = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
  const uint32_t a = r[0], b = r[1];
  return op(u2f(a), u2f(b));
}

struct AddOp {
  __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};
struct MaxOp {
  __device__ __forceinline__ float operator()(float a, float b) const { return __builtin_fmaxf(a, b); }
};
// Maximum of operands that are never NaN (scores after masking, running
// maxima).  The NaN-propagating form (v_maximum3_f32 on gfx950) needs no
// quieting of its inputs, which fmaxf costs one extra instruction per
// operand that the compiler cannot prove quiet (matrix-core results, lane
// shuffles).
__device__ __forceinline__ float max_nn(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}
struct MaxNnOp {
  __device__ __forceinline__ float operator()(float a, float b) const { return max_nn(a, b); }
};

// Reduction over aligned groups of N lanes (N in {2,4,8,16,32,64}); every
// lane of a group receives the group's result.  Within a 16-lane row the
// butterfly is xor 1, xor 2, then the half-row and row mirrors (each pairs
// every lane with one from the other half of its current group).
template <int N, typename Op>
__device__ __forceinline__ float group_reduce(float x, Op op) {
  static_assert(N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group size");
  x = op(x, dpp<kDppQuadXor1>(x));
  if constexpr (N >= 4) x = op(x, dpp<kDppQuadXor2>(x));
  if constexpr (N >= 8) x = op(x, dpp<kDppHalfMirror>(x));
  if constexpr (N >= 16) x = op(x, dpp<kDppRowMirror>(x));
  if constexpr (N >= 32) x = xor16_combine(x, op);
  if constexpr (N >= 64) x = xor32_combine(x, op);
  return x;
}

template <int N>
__device__ __forceinline__ float group_sum(float x) {
  return group_reduce<N>(x, AddOp{});
}

// Reduction across the 64 / N aligned groups of N lanes: every lane receives
// op over all lanes with the same index within their group (N in {8,16,32}).
template <int N, typename Op>
__device__ __forceinline__ float across_groups(float x, Op op) {
  static_assert(N == 8 || N == 16 || N == 32, "group size");
  if constexpr (N == 8) x = op(x, dpp<kDppRowRor8>(x));
  if constexpr (N <= 16) x = xor16_combine(x, op);
  x = xor32_combine(x, op);
  return x;
}

// Store n = 4 (fp32) or 8 (fp16/bf16) consecutive results as one 16-byte
// store; base + idx must be 16-byte aligned.
template <int DT>
__device__ __forceinline__ void store16(void* base, int64_t idx, const float* v) {
  if constexpr (DT == kF32) {
    *reinterpret_cast<u32x4*>(reinterpret_cast<float*>(base) + idx) =
        u32x4{f2u(v[0]), f2u(v[1]), f2u(v[2]), f2u(v[3])};
  } else {
    u32x4 w;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = (uint32_t)to_bits16<DT>(v[2 * k]) | ((uint32_t)to_bits16<DT>(v[2 * k + 1]) << 16);
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(base) + idx) = w;
  }
}

}  // namespace pa
