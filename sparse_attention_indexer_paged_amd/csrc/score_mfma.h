// Pieces shared by the indexer logits kernels (paged decode in logits.hip,
// contiguous prefill in prefill.hip): the fp8 MFMA operand and accumulator
// layouts of v_mfma_f32_16x16x128_f8f6f4 with A = 16 heads of one query row
// and B = 16 keys, the fused ReLU / head-weight epilogue, the cross-lane
// head reduction and the masked logit stores.
//
// Operand layout: lane l = 16*g + n holds row/column n and 32 bytes of the
// 128-long contraction; lane (g, n) takes bytes [16g, 16g+16) and
// [64+16g, 64+16g+16) of its head or key row (any order works as long as A
// and B agree).  Accumulator layout: lane (g, n), register i = head 4g + i of
// the head group, key n.
#pragma once

#include "sai_device.h"

namespace sai {
namespace score {

// Masking by integer select on the bit patterns, so the choice is never an
// fp operation the no-NaN compile mode may reason about.
__device__ __forceinline__ float select_f(bool c, float a, uint32_t b_bits) {
  return __uint_as_float(c ? __float_as_uint(a) : b_bits);
}
constexpr uint32_t kNegInfBits = 0xFF800000u;

// Logits are written once and read by the next kernel.  NT streams them past
// the caches (non-temporal); plain stores leave them in L2 and the
// memory-side cache, where a top-k that follows finds a small logits buffer
// sooner.
template <bool NT = true>
__device__ __forceinline__ void store_logit(float* p, float v) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}
typedef float f32x4 __attribute__((ext_vector_type(4)));
template <bool NT = true>
__device__ __forceinline__ void store_logit4(float* p, float4 v) {
  const f32x4 x = {v.x, v.y, v.z, v.w};
  if constexpr (NT)
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p));
  else
    *reinterpret_cast<f32x4*>(p) = x;
}
constexpr uint32_t kNaNBits = 0x7FC00000u;

__device__ __forceinline__ int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
__device__ __forceinline__ int64_t max64(int64_t a, int64_t b) { return a > b ? a : b; }

__device__ __forceinline__ int cdiv_i(int a, int b) { return (a + b - 1) / b; }

static inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Key tile t of a 64-key block covers keys tile_key(t) .. tile_key(t)+15.
// After the reduce-scatter, tiles 0,2,1,3 land in lanes 0-15, 16-31, 32-47,
// 48-63; with this assignment lane l holds key l.
__device__ __forceinline__ int tile_key(int t) { return ((t & 1) << 5) | ((t & 2) << 3); }

__device__ __forceinline__ v8i make_v8i(uint4 a, uint4 b) {
  v8i r;
  r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
  r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
  return r;
}

// A operands of one query row ([64 heads][128] codes): head group hg holds
// heads 16hg .. 16hg+15.
__device__ __forceinline__ void load_qfrag(v8i (&qa)[4], const uint8_t* __restrict__ qrow) {
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
#pragma unroll
  for (int hg = 0; hg < 4; ++hg) {
    const uint8_t* p = qrow + (16 * hg + n) * kDim + 16 * g;
    qa[hg] = make_v8i(*reinterpret_cast<const uint4*>(p), *reinterpret_cast<const uint4*>(p + 64));
  }
}

// Head weights matching the accumulator layout: lane (g, n) needs heads
// 16hg + 4g + i, i = 0..3.
__device__ __forceinline__ void load_wfrag(float4 (&wv)[4], const float* __restrict__ wrow) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int hg = 0; hg < 4; ++hg) wv[hg] = *reinterpret_cast<const float4*>(wrow + 16 * hg + 4 * g);
}

__device__ __forceinline__ float relu_dot4(const float4 w, const v4f c, float acc) {
  acc = fmaf(w.x, fmaxf(c[0], 0.0f), acc);
  acc = fmaf(w.y, fmaxf(c[1], 0.0f), acc);
  acc = fmaf(w.z, fmaxf(c[2], 0.0f), acc);
  acc = fmaf(w.w, fmaxf(c[3], 0.0f), acc);
  return acc;
}

// Sum the four lanes {n, n+16, n+32, n+48} of each of the 4 key tiles and
// scatter: lanes 16p + n receive tile [0, 2, 1, 3][p], column n.
__device__ __forceinline__ float reduce_scatter4(float p0, float p1, float p2, float p3) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(p2), __float_as_uint(p3), false, false);
  const float x01 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const float x23 = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(x01), __float_as_uint(x23), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

}  // namespace score
}  // namespace sai
