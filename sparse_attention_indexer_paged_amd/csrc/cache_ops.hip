// K-cache write, query producer, paged->contiguous gather and slot-id map.
//
// All four are bandwidth/latency-bound byte movers with a little fp32 math;
// none is a contraction, so they use no MFMA: 16-byte vector loads and stores
// laid out so consecutive lanes touch consecutive bytes.
#include "sai_device.h"

using namespace sai;

extern "C" const char* sai_status_string(int status) {
  switch (status) {
    case SAI_OK: return "SAI_OK";
    case SAI_EINVAL: return "SAI_EINVAL: invalid argument";
    case SAI_EUNSUPPORTED: return "SAI_EUNSUPPORTED: unsupported shape";
    case SAI_EWORKSPACE: return "SAI_EWORKSPACE: workspace missing or too small";
    case SAI_ELAUNCH: return "SAI_ELAUNCH: kernel launch failed";
    case SAI_ESCRATCH: return "SAI_ESCRATCH: problem needs more than the built-in scratch buffer";
    default: return "SAI: unknown status";
  }
}

extern "C" int sai_time_next_launch(hipEvent_t start, hipEvent_t stop) {
  if ((start == nullptr) != (stop == nullptr)) return SAI_EINVAL;
  g_launch_timing = LaunchTiming{start, stop, false};
  return SAI_OK;
}

extern "C" int sai_time_span(hipEvent_t start, hipEvent_t stop) {
  if ((start == nullptr) != (stop == nullptr)) return SAI_EINVAL;
  g_launch_timing = LaunchTiming{start, stop, start != nullptr};
  return SAI_OK;
}

static inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static inline int launch_status() {
  return hipGetLastError() == hipSuccess ? SAI_OK : SAI_ELAUNCH;
}

// ---------------------------------------------------------------- rotation
// Rotates the pair (x1, x2) by the angle whose cosine and sine are (c, s):
// r1 = x1 c - x2 s, r2 = x2 c + x1 s, every product and sum rounded to
// float32 on its own (no fused multiply-add), so the codes the quantiser
// makes of the result are reproducible bit for bit.
__device__ __forceinline__ void rope_pair(float& x1, float& x2, float c, float s) {
#pragma clang fp contract(off)
  const float a = x1 * c, b = x2 * s, d = x2 * c, e = x1 * s;
  x1 = a - b;
  x2 = d + e;
}

// Rotary tables of the fused producers: cos/sin [rows, half] fp32, row p =
// token position p; pair j of a row (values 2j, 2j + 1) uses column j.
struct Rope {
  const int64_t* pos;
  const float* cos_t;
  const float* sin_t;
  int64_t rows;
  int half;  // rope_dim / 2
};

// The table entries of pairs j0 .. j0+N-1 of row p (0 <= p < rows), every
// load issued before any is used: pairs past the row's half re-read its
// last entry (the caller ignores them), so the loads are unconditional and
// go out together instead of one round trip per pair.
// When half is a multiple of 4 (and j0 too) the entries come as 16-byte
// loads of whole groups of four.
template <int N>
__device__ __forceinline__ void rope_load(const Rope& rope, int64_t p, int j0, float (&c)[N], float (&s)[N]) {
  static_assert(N % 4 == 0, "groups of four pairs");
  const float* cr = rope.cos_t + p * rope.half;
  const float* sr = rope.sin_t + p * rope.half;
  if ((rope.half & 3) == 0) {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const int j = min(j0 + i, rope.half - 4);
      const float4 cv = *reinterpret_cast<const float4*>(cr + j);
      const float4 sv = *reinterpret_cast<const float4*>(sr + j);
      c[i] = cv.x; c[i + 1] = cv.y; c[i + 2] = cv.z; c[i + 3] = cv.w;
      s[i] = sv.x; s[i + 1] = sv.y; s[i + 2] = sv.z; s[i + 3] = sv.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int j = min(j0 + i, rope.half - 1);
      c[i] = cr[j];
      s[i] = sr[j];
    }
  }
}

// ---------------------------------------------------------------- K1
// 8 lanes per token row: lane i of the group holds values [16i, 16i+16)
// (two 16-byte loads in flight per lane), i.e. rotary pairs 8i .. 8i+7.
// One 256-thread workgroup writes 32 tokens.  With ROPE the first 2*half
// values are rotated by the token's position before the quantiser sees
// them; a position outside the table writes NaN codes and a NaN scale.
template <bool ROPE>
__global__ __launch_bounds__(256) void k_cache_write_kernel(
    const uint16_t* __restrict__ k, int64_t row_stride, const int64_t* __restrict__ slots,
    int64_t n, uint8_t* __restrict__ cache, int64_t num_blocks, Rope rope) {
  const int64_t tok = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  const int sub = threadIdx.x & 7;
  const bool live = tok < n;
  uint4 raw[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
  int64_t slot = -1;
  int64_t p = 0;
  if (live) {
    raw[0] = *reinterpret_cast<const uint4*>(k + tok * row_stride + sub * 16);
    raw[1] = *reinterpret_cast<const uint4*>(k + tok * row_stride + sub * 16 + 8);
    slot = slots[tok];
    if (ROPE) p = rope.pos[tok];
  }
  float x[16];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t w[4] = {raw[h].x, raw[h].y, raw[h].z, raw[h].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[8 * h + 2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
      x[8 * h + 2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
  }
  bool pos_ok = true;
  if constexpr (ROPE) {
    pos_ok = p >= 0 && p < rope.rows;
    if (live && pos_ok && 8 * sub < rope.half) {
      float c[8], sn[8];
      rope_load<8>(rope, p, 8 * sub, c, sn);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (8 * sub + i < rope.half) rope_pair(x[2 * i], x[2 * i + 1], c[i], sn[i]);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
  for (int o = 4; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 8));
  float scale = fp8_scale(amax);
  float y[16];
  quotients_by_scale(x, scale, y);
  uint32_t pk[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    pk[q] = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) pk[q] |= f32_to_e4m3fn(y[4 * q + i]) << (8 * i);
  }
  if (!pos_ok) {
    pk[0] = pk[1] = pk[2] = pk[3] = 0x7F7F7F7Fu;
    scale = __uint_as_float(0x7FC00000u);
  }
  if (!live || slot < 0 || slot >= num_blocks * kBlock) return;
  uint8_t* blk = cache + (slot / kBlock) * kBlockBytes;
  const int off = (int)(slot % kBlock);
  *reinterpret_cast<uint4*>(blk + off * kDim + sub * 16) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  if (sub == 0) *reinterpret_cast<float*>(blk + kValueBytes + 4 * off) = scale;
}

extern "C" int indexer_k_cache_write(const void* k_bf16, int64_t k_row_stride,
                                     const int64_t* slot_mapping, int64_t n, void* kv_cache,
                                     int64_t num_blocks, hipStream_t stream) {
  if (n < 0 || num_blocks < 0) return SAI_EINVAL;
  if (n == 0) return SAI_OK;
  if (k_row_stride < kDim || (k_row_stride & 7)) return SAI_EINVAL;
  if (!k_bf16 || !slot_mapping || !kv_cache || !aligned16(k_bf16) || !aligned16(kv_cache))
    return SAI_EINVAL;
  const int64_t grid = (n + 31) / 32;
  if (grid > 0x7FFFFFFF) return SAI_EUNSUPPORTED;
  launch(k_cache_write_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream,
         (const uint16_t*)k_bf16, k_row_stride, slot_mapping, n, (uint8_t*)kv_cache, num_blocks,
         Rope{nullptr, nullptr, nullptr, 0, 0});
  return launch_status();
}

// Host checks shared by the two fused producers: rope_dim even in [0, 128];
// tables and positions present when something is rotated.
static int check_rope(const int64_t* positions, const float* cos_t, const float* sin_t,
                      int64_t table_rows, int32_t rope_dim) {
  if (rope_dim < 0 || rope_dim > kDim || (rope_dim & 1) || table_rows < 0) return SAI_EINVAL;
  if (rope_dim > 0 && (!positions || !cos_t || !sin_t)) return SAI_EINVAL;
  if (table_rows > (int64_t)1 << 40) return SAI_EUNSUPPORTED;
  return SAI_OK;
}

extern "C" int indexer_k_rope_cache_write(const void* k_bf16, int64_t k_row_stride,
                                          const int64_t* positions, const float* cos_table,
                                          const float* sin_table, int64_t table_rows,
                                          int32_t rope_dim, const int64_t* slot_mapping, int64_t n,
                                          void* kv_cache, int64_t num_blocks, hipStream_t stream) {
  if (n < 0 || num_blocks < 0) return SAI_EINVAL;
  const int rc = check_rope(positions, cos_table, sin_table, table_rows, rope_dim);
  if (rc != SAI_OK) return rc;
  if (n == 0) return SAI_OK;
  if (k_row_stride < kDim || (k_row_stride & 7)) return SAI_EINVAL;
  if (!k_bf16 || !slot_mapping || !kv_cache || !aligned16(k_bf16) || !aligned16(kv_cache))
    return SAI_EINVAL;
  const int64_t grid = (n + 31) / 32;
  if (grid > 0x7FFFFFFF) return SAI_EUNSUPPORTED;
  if (rope_dim == 0)
    launch(k_cache_write_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream,
           (const uint16_t*)k_bf16, k_row_stride, slot_mapping, n, (uint8_t*)kv_cache, num_blocks,
           Rope{nullptr, nullptr, nullptr, 0, 0});
  else
    launch(k_cache_write_kernel<true>, dim3((unsigned)grid), dim3(256), 0, stream,
           (const uint16_t*)k_bf16, k_row_stride, slot_mapping, n, (uint8_t*)kv_cache, num_blocks,
           Rope{positions, cos_table, sin_table, table_rows, rope_dim / 2});
  return launch_status();
}

// ---------------------------------------------------------------- q producer
// One 256-thread workgroup per query token (64 heads x 128 = 8192 values):
// thread t owns values [32t, 32t+32) as four 16-byte loads, i.e. head t/4,
// in-head values 32 (t % 4) .. +31 (rotary pairs 16 (t % 4) .. +15).  With
// ROPE every head's first 2*half values are rotated by the token's position
// before the token's scale is taken; a position outside the table gives
// NaN codes, scale and weights.
template <bool ROPE>
__global__ __launch_bounds__(256) void q_quant_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ wts, uint8_t* __restrict__ q8,
    float* __restrict__ w_eff, float* __restrict__ q_scale, Rope rope) {
  __shared__ float s_amax[4];
  __shared__ float s_cs[2][ROPE ? 64 : 1];  // the token's cos and sin table row
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x;
  const uint16_t* src = q + row * (kHeads * kDim) + t * 32;
  uint4 raw[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) raw[v] = *reinterpret_cast<const uint4*>(src + v * 8);
  // The token's table row goes to LDS (threads 0..half-1 load the
  // cosines, 64..64+half-1 the sines) while the row's loads are in flight.
  bool pos_ok = true;
  if constexpr (ROPE) {
    const int64_t p = rope.pos[row];
    pos_ok = p >= 0 && p < rope.rows;
    const int64_t pc = pos_ok ? p : 0;
    if (t < 64 && t < rope.half) s_cs[0][t] = rope.cos_t[pc * rope.half + t];
    else if (t >= 64 && t < 128 && t - 64 < rope.half) s_cs[1][t - 64] = rope.sin_t[pc * rope.half + t - 64];
  }
  float x[32];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const uint32_t w[4] = {raw[v].x, raw[v].y, raw[v].z, raw[v].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[v * 8 + 2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
      x[v * 8 + 2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
  }
  if constexpr (ROPE) {
    __syncthreads();  // the table row
    if (pos_ok) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = 16 * (t & 3) + i;
        if (j < rope.half) rope_pair(x[2 * i], x[2 * i + 1], s_cs[0][j], s_cs[1][j]);
      }
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
  amax = wave_max(amax);
  if ((t & 63) == 0) s_amax[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_amax[0], s_amax[1]), fmaxf(s_amax[2], s_amax[3]));
  float scale = fp8_scale(amax);
  float y[32];
  quotients_by_scale(x, scale, y);
  uint32_t packed[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t pk = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) pk |= f32_to_e4m3fn(y[4 * i + j]) << (8 * j);
    packed[i] = pos_ok ? pk : 0x7F7F7F7Fu;
  }
  if (!pos_ok) scale = __uint_as_float(0x7FC00000u);
  uint8_t* dst = q8 + row * (kHeads * kDim) + t * 32;
  *reinterpret_cast<uint4*>(dst) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  *reinterpret_cast<uint4*>(dst + 16) = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  if (t < kHeads) w_eff[row * kHeads + t] = wts[row * kHeads + t] * scale;
  if (t == 0 && q_scale) q_scale[row] = scale;
}

extern "C" int indexer_q_quant(const void* q_bf16, const float* weights, int64_t rows,
                               void* q_fp8, float* w_eff, float* q_scale, hipStream_t stream) {
  if (rows < 0) return SAI_EINVAL;
  if (rows == 0) return SAI_OK;
  if (!q_bf16 || !weights || !q_fp8 || !w_eff || !aligned16(q_bf16) || !aligned16(q_fp8))
    return SAI_EINVAL;
  if (rows > 0x7FFFFFFF) return SAI_EUNSUPPORTED;
  launch(q_quant_kernel<false>, dim3((unsigned)rows), dim3(256), 0, stream,
         (const uint16_t*)q_bf16, weights, (uint8_t*)q_fp8, w_eff, q_scale,
         Rope{nullptr, nullptr, nullptr, 0, 0});
  return launch_status();
}

extern "C" int indexer_q_rope_quant(const void* q_bf16, const int64_t* positions,
                                    const float* cos_table, const float* sin_table,
                                    int64_t table_rows, int32_t rope_dim, const float* weights,
                                    int64_t rows, void* q_fp8, float* w_eff, float* q_scale,
                                    hipStream_t stream) {
  if (rows < 0) return SAI_EINVAL;
  const int rc = check_rope(positions, cos_table, sin_table, table_rows, rope_dim);
  if (rc != SAI_OK) return rc;
  if (rows == 0) return SAI_OK;
  if (!q_bf16 || !weights || !q_fp8 || !w_eff || !aligned16(q_bf16) || !aligned16(q_fp8))
    return SAI_EINVAL;
  if (rows > 0x7FFFFFFF) return SAI_EUNSUPPORTED;
  if (rope_dim == 0)
    launch(q_quant_kernel<false>, dim3((unsigned)rows), dim3(256), 0, stream,
           (const uint16_t*)q_bf16, weights, (uint8_t*)q_fp8, w_eff, q_scale,
           Rope{nullptr, nullptr, nullptr, 0, 0});
  else
    launch(q_quant_kernel<true>, dim3((unsigned)rows), dim3(256), 0, stream,
           (const uint16_t*)q_bf16, weights, (uint8_t*)q_fp8, w_eff, q_scale,
           Rope{positions, cos_table, sin_table, table_rows, rope_dim / 2});
  return launch_status();
}

// ---------------------------------------------------------------- gather
// 8 lanes per destination token (16 bytes each); 32 tokens per workgroup.
// The owning request of a destination row is found by binary search of
// cu_seq_lens, so the launch needs only host sizes.
__global__ __launch_bounds__(256) void gather_kernel(
    const uint8_t* __restrict__ cache, int64_t num_blocks, const int32_t* __restrict__ bt,
    int64_t bt_stride, const int32_t* __restrict__ cu, int32_t batch, int64_t total,
    uint8_t* __restrict__ out_k, float* __restrict__ out_s) {
  const int64_t row = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  const int sub = threadIdx.x & 7;
  if (row >= total) return;
  if (row < cu[0] || row >= cu[batch]) return;
  int lo = 0, hi = batch;  // largest b with cu[b] <= row
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= row) lo = mid; else hi = mid;
  }
  const int b = lo;
  const int64_t t = row - cu[b];
  const int64_t c = t / kBlock;
  if (c >= bt_stride) return;
  const int32_t blk = bt[(int64_t)b * bt_stride + c];
  const int off = (int)(t % kBlock);
  uint4 v = make_uint4(0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu);
  float s = __uint_as_float(0x7FC00000u);
  if (blk >= 0 && blk < num_blocks) {
    const uint8_t* src = cache + (int64_t)blk * kBlockBytes;
    v = *reinterpret_cast<const uint4*>(src + off * kDim + sub * 16);
    if (sub == 0) s = *reinterpret_cast<const float*>(src + kValueBytes + 4 * off);
  }
  *reinterpret_cast<uint4*>(out_k + row * kDim + sub * 16) = v;
  if (sub == 0) out_s[row] = s;
}

extern "C" int gather_indexer_k(const void* kv_cache, int64_t num_blocks, const int32_t* block_table,
                                int64_t bt_stride, const int32_t* cu_seq_lens, int32_t batch,
                                int64_t total_tokens, void* out_k_fp8, float* out_scale,
                                hipStream_t stream) {
  if (batch < 0 || total_tokens < 0 || num_blocks < 0 || bt_stride < 0) return SAI_EINVAL;
  if (batch == 0 || total_tokens == 0) return SAI_OK;
  if (!kv_cache || !block_table || !cu_seq_lens || !out_k_fp8 || !out_scale) return SAI_EINVAL;
  if (!aligned16(kv_cache) || !aligned16(out_k_fp8)) return SAI_EINVAL;
  const int64_t grid = (total_tokens + 31) / 32;
  if (grid > 0x7FFFFFFF) return SAI_EUNSUPPORTED;
  launch(gather_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     (const uint8_t*)kv_cache, num_blocks, block_table, bt_stride, cu_seq_lens,
                     batch, total_tokens, (uint8_t*)out_k_fp8, out_scale);
  return launch_status();
}

// ---------------------------------------------------------------- slot ids
// One 256-thread workgroup per row: the row's top-k indices are loaded into
// registers while the request's block-table row is staged in LDS, so each
// index maps to its slot with an LDS lookup instead of a dependent global
// gather.  Tables wider than kSlotLdsEntries use the elementwise kernel.
constexpr int kSlotLdsEntries = 8192;
constexpr int kSlotPerThread = 8;  // k <= 2048 = 256 threads x 8

__global__ __launch_bounds__(256) void slots_row_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ row_req,
    const int32_t* __restrict__ bt, int64_t bt_stride, int32_t batch, int32_t k,
    int32_t* __restrict__ out) {
  __shared__ int32_t s_bt[kSlotLdsEntries];
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x;
  int32_t iv[kSlotPerThread];
#pragma unroll
  for (int e = 0; e < kSlotPerThread; ++e) {
    const int j = tid + 256 * e;
    iv[e] = j < k ? idx[r * k + j] : -1;
  }
  const int32_t b = row_req[r];
  const bool okb = b >= 0 && b < batch;
  for (int64_t c = tid; c < bt_stride; c += 256) s_bt[c] = okb ? bt[(int64_t)b * bt_stride + c] : -1;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < kSlotPerThread; ++e) {
    const int j = tid + 256 * e;
    if (j >= k) break;
    const int32_t i = iv[e];
    int32_t slot = -1;
    if (i >= 0 && (i / kBlock) < bt_stride) {
      const int32_t blk = s_bt[i / kBlock];
      if (blk >= 0) slot = blk * kBlock + (i % kBlock);
    }
    out[r * k + j] = slot;
  }
}

// One thread per output element (tables wider than the LDS stage).
__global__ __launch_bounds__(256) void slots_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ row_req,
    const int32_t* __restrict__ bt, int64_t bt_stride, int32_t batch, int64_t total, int32_t k,
    int32_t* __restrict__ out) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= total) return;
  const int64_t r = e / k;
  const int32_t i = idx[e];
  int32_t slot = -1;
  if (i >= 0) {
    const int32_t b = row_req[r];
    const int64_t c = i / kBlock;
    if (b >= 0 && b < batch && c < bt_stride) {
      const int32_t blk = bt[(int64_t)b * bt_stride + c];
      if (blk >= 0) slot = blk * kBlock + (i % kBlock);
    }
  }
  out[e] = slot;
}

extern "C" int topk_to_global_slots(const int32_t* topk_idx, const int32_t* row_req,
                                    const int32_t* block_table, int64_t bt_stride, int32_t batch,
                                    int32_t rows, int32_t k, int32_t* out_slots,
                                    hipStream_t stream) {
  if (rows < 0 || k < 0 || batch < 0 || bt_stride < 0) return SAI_EINVAL;
  if (rows == 0 || k == 0) return SAI_OK;
  if (!topk_idx || !row_req || !block_table || !out_slots) return SAI_EINVAL;
  if (k <= 256 * kSlotPerThread && bt_stride <= kSlotLdsEntries) {
    launch(slots_row_kernel, dim3(rows), dim3(256), 0, stream, topk_idx, row_req,
                       block_table, bt_stride, batch, k, out_slots);
    return launch_status();
  }
  const int64_t total = (int64_t)rows * k;
  const int64_t grid = (total + 255) / 256;
  if (grid > 0x7FFFFFFF) return SAI_EUNSUPPORTED;
  launch(slots_kernel, dim3(grid), dim3(256), 0, stream, topk_idx, row_req,
                     block_table, bt_stride, batch, total, k, out_slots);
  return launch_status();
}
