// fp8 MLA cache ("fp8_ds_mla" layout) and its writer.
//
// One cache entry per token, 656 bytes (prhub summary of vLLM PR #47090, key
// source excerpt of _fused_norm_rope_kernel, MLA_CACHE_DS_MLA branch):
//   [0, 512)    the 512 latent values as fp8 e4m3fn codes, one dynamic scale
//               per 128-value tile
//   [512, 528)  the 4 tile scales, fp32
//   [528, 656)  the 64 RoPE values, bf16
// Token slot s is entry s % block_size of block s / block_size.
#include "sai_device.h"

using namespace sai;

namespace {

constexpr int kMlaKv = 512;
constexpr int kMlaTile = 128;
constexpr int kMlaRope = 64;
constexpr int kMlaScaleOff = kMlaKv;                    // 512
constexpr int kMlaRopeOff = kMlaKv + 4 * (kMlaKv / kMlaTile);  // 528
constexpr int kMlaEntry = kMlaRopeOff + 2 * kMlaRope;   // 656
static_assert(kMlaEntry == 656 && kMlaEntry % 16 == 0, "16-byte aligned entries");

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// One wave per token (4 per workgroup).  Lane l holds latent values
// [8l, 8l+8), so the 16 lanes of a row group are one 128-value tile and the
// tile amax is a 16-lane reduction; lanes 0..31 also carry RoPE values 2l, 2l+1.
__global__ __launch_bounds__(256) void mla_cache_write_kernel(
    const uint16_t* __restrict__ kv, int64_t kv_stride, const uint16_t* __restrict__ kpe,
    int64_t kpe_stride, const int64_t* __restrict__ slots, int64_t n, uint8_t* __restrict__ cache,
    int64_t num_slots, int64_t block_size, int64_t block_stride) {
  const int64_t tok = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (tok >= n) return;  // wave-uniform
  const int64_t slot = slots[tok];
  if (slot < 0 || slot >= num_slots) return;
  const uint4 raw = *reinterpret_cast<const uint4*>(kv + tok * kv_stride + lane * 8);
  float x[8];
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    x[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
  const float scale = fp8_scale(amax);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) lo |= f32_to_e4m3fn(x[i] / scale) << (8 * i);
#pragma unroll
  for (int i = 0; i < 4; ++i) hi |= f32_to_e4m3fn(x[4 + i] / scale) << (8 * i);
  uint8_t* e = cache + (slot / block_size) * block_stride + (slot % block_size) * kMlaEntry;
  *reinterpret_cast<uint2*>(e + lane * 8) = make_uint2(lo, hi);
  if ((lane & 15) == 0) *reinterpret_cast<float*>(e + kMlaScaleOff + 4 * (lane >> 4)) = scale;
  if (lane < kMlaRope / 2)
    *reinterpret_cast<uint32_t*>(e + kMlaRopeOff + 4 * lane) =
        *reinterpret_cast<const uint32_t*>(kpe + tok * kpe_stride + 2 * lane);
}

}  // namespace

extern "C" int mla_cache_write(const void* kv_bf16, int64_t kv_row_stride, const void* kpe_bf16,
                               int64_t kpe_row_stride, const int64_t* slot_mapping, int64_t n,
                               void* cache, int64_t num_blocks, int32_t block_size,
                               hipStream_t stream) {
  if (n < 0 || num_blocks < 0 || block_size <= 0) return SAI_EINVAL;
  if (n == 0) return SAI_OK;
  if (kv_row_stride < kMlaKv || (kv_row_stride & 7) || kpe_row_stride < kMlaRope || (kpe_row_stride & 1))
    return SAI_EINVAL;
  if (!kv_bf16 || !kpe_bf16 || !slot_mapping || !cache) return SAI_EINVAL;
  if (!aligned16(kv_bf16) || !aligned4(kpe_bf16) || !aligned16(cache)) return SAI_EINVAL;
  const int64_t grid = (n + 3) / 4;
  if (grid > 0x7FFFFFFF || num_blocks > INT64_MAX / (block_size * (int64_t)kMlaEntry)) return SAI_EUNSUPPORTED;
  launch(mla_cache_write_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
         (const uint16_t*)kv_bf16, kv_row_stride, (const uint16_t*)kpe_bf16, kpe_row_stride,
         slot_mapping, n, (uint8_t*)cache, num_blocks * (int64_t)block_size, (int64_t)block_size,
         (int64_t)block_size * kMlaEntry);
  return hipGetLastError() == hipSuccess ? SAI_OK : SAI_ELAUNCH;
}
