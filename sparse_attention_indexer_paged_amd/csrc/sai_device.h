// Device-side building blocks shared by the gfx950 indexer kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sai.h"
#include "sai_profile.h"

namespace sai {

constexpr int kHeads = SAI_HEADS;          // 64
constexpr int kDim = SAI_HEAD_DIM;         // 128
constexpr int kBlock = SAI_BLOCK_SIZE;     // 64 tokens
constexpr int kValueBytes = kBlock * kDim; // 8192
constexpr int kBlockBytes = SAI_BLOCK_BYTES;
constexpr int kWave = 64;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- fp8
// float32 -> fp8 e4m3fn, round to nearest even, saturating at +-448, sign
// kept (so -0.0 -> 0x80).  Normal range: round the float32 mantissa to 3 bits
// on the bit pattern and rebias the exponent (127 -> 7); subnormal range
// (|y| < 2^-6): the code is the integer round(|y| * 2^9) in 0..8, where 8 is
// the smallest normal 2^-6.  Input must not be NaN.
__device__ __forceinline__ uint32_t f32_to_e4m3fn(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fminf(fabsf(y), 448.0f);
  uint32_t mag;
  if (a >= 0.015625f) {
    const uint32_t u = __float_as_uint(a);
    const uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);
    mag = (r >> 20) - (120u << 3);
  } else {
    mag = (uint32_t)rintf(a * 512.0f);
  }
  return sign | mag;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// quantiser scale: max(amax * fl32(1/448), FLT_MIN), float32
__device__ __forceinline__ float fp8_scale(float amax) {
  return fmaxf(amax * (1.0f / 448.0f), 1.17549435e-38f);
}

// y[i] = fl32(x[i] / s), the correctly rounded quotients.  For a scale
// 2^-93 <= s <= FLT_MAX they come from r = fl32(1 / s) by Markstein's
// correction (P. Markstein, "Computation of elementary functions on the IBM
// RISC System/6000 processor", IBM J. Res. Dev. 34(1), 1990): q = fl(x r)
// is within an ulp of x / s, the residual x - s q is then exact in one fused
// multiply-add, and fl(q + (x - s q) r) is the correctly rounded quotient.
// The residual is a multiple of 2^(e - 46) for |x| in [2^e, 2^(e + 1)),
// exact as long as e >= -103; a smaller x has a quotient below 2^-10 (as
// s >= 2^-93), which every float32 near it rounds to the same e4m3 code,
// zero.  The result takes the sign of x, so that a zero keeps its own sign
// (the correction would turn -0 into +0).  Other scales take the IEEE
// division.
template <int N>
__device__ __forceinline__ void quotients_by_scale(const float (&x)[N], float s, float (&y)[N]) {
  if (s >= 0x1p-93f && s <= 3.40282347e38f) {
    const float r = 1.0f / s;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const float q = x[i] * r;
      // the sign of x: a zero x gives a zero of its own sign, as x / s does
      y[i] = __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q, s, x[i]), r, q), x[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) y[i] = x[i] / s;
  }
}

// Order-preserving float -> uint32 key (larger float, larger key).  -0.0 is
// folded onto +0.0 so the two tie.  Every NaN (either sign, any payload)
// gets key 0, below -inf (key 0x007FFFFF): NaNs rank last and tie with each
// other, so ties among them go to the lower index like any other tie.
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (u & 0x7FFFFFFFu) > 0x7F800000u ? 0u : k;
}

// ---------------------------------------------------------------- wave ops
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive scan over a whole workgroup of NT threads (NT multiple of 64,
// at most 64 waves).  `scratch` holds NT/64 + 1 ints of LDS.  Returns the
// exclusive prefix of `v`; *total receives the workgroup sum.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = wave_inclusive_scan(v);
  if (lane == 63) scratch[w] = inc;
  __syncthreads();
  if (w == 0) {
    int s = lane < NW ? scratch[lane] : 0;
    int si = wave_inclusive_scan(s);
    if (lane < NW) scratch[lane] = si - s;
    if (lane == NW - 1) scratch[NW] = si;
  }
  __syncthreads();
  int res = scratch[w] + inc - v;
  *total = scratch[NW];
  __syncthreads();
  return res;
}

// ---------------------------------------------------------------- launches
// Every kernel goes through launch().  When the calling thread has armed a
// start/stop event pair (sai_time_next_launch), its next launch carries the
// pair in its own dispatch, so their elapsed time is that kernel's execution
// alone; a separate hipEventRecord would add marker packets to the stream.
// A span (sai_time_span) stays armed until the caller disarms it: its first
// launch carries start and every launch carries stop, so the pair ends with
// the last kernel of the calls made meanwhile.
struct LaunchTiming {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
  bool span = false;
};
inline thread_local LaunchTiming g_launch_timing;

template <typename F, typename... Args>
inline void launch(F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t s, Args... args) {
  LaunchTiming& t = g_launch_timing;
  const hipEvent_t start = t.start, stop = t.stop;
  if (t.span) t.start = nullptr;
  else t = LaunchTiming{};
  hipExtLaunchKernelGGL(kernel, grid, block, lds, s, start, stop, 0u, args...);
}

}  // namespace sai
