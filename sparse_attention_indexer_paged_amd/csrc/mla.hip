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
  // every load goes out before the slot is known: the values, the RoPE
  // piece and the slot arrive in one round trip
  const int64_t slot = slots[tok];
  const uint4 raw = *reinterpret_cast<const uint4*>(kv + tok * kv_stride + lane * 8);
  const uint32_t pe = *reinterpret_cast<const uint32_t*>(kpe + tok * kpe_stride + 2 * (lane & 31));
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
  float y[8];
  quotients_by_scale(x, scale, y);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) lo |= f32_to_e4m3fn(y[i]) << (8 * i);
#pragma unroll
  for (int i = 0; i < 4; ++i) hi |= f32_to_e4m3fn(y[4 + i]) << (8 * i);
  if (slot < 0 || slot >= num_slots) return;
  uint8_t* e = cache + (slot / block_size) * block_stride + (slot % block_size) * kMlaEntry;
  *reinterpret_cast<uint2*>(e + lane * 8) = make_uint2(lo, hi);
  if ((lane & 15) == 0) *reinterpret_cast<float*>(e + kMlaScaleOff + 4 * (lane >> 4)) = scale;
  if (lane < kMlaRope / 2) *reinterpret_cast<uint32_t*>(e + kMlaRopeOff + 4 * lane) = pe;
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

// ------------------------------------------------------------ sparse decode
// Sparse MLA decode over the fp8 cache (the consumer of the global slot ids;
// ROCm/ATOM PR #1094, Technical Details).  For query row t and head h, over
// the row's valid slots j:
//   s_j = sm_scale * (q_nope[t,h] . kv_j + q_pe[t,h] . kpe_j),
//   out[t,h] = sum_j softmax(s)_j kv_j,  lse[t,h] = log sum_j exp(s_j),
// kv_j the dequantised latent (code * tile scale), kpe_j the stored RoPE part.
//
// Two kernels share the gather below: the 64-head (wide) kernel, described
// at its definition (it stages chunks as bf16), for head counts in groups of
// 64, and the 16-head (narrow) kernel described here for the rest.
//
// Narrow: workgroup = one query row x 16 heads x one split of the slot list,
// 4 waves.  Slots go through in chunks of 32: the chunk's entries are gathered one
// chunk ahead into registers, then written to LDS twice -- codes
// token-major (the B operand of Q.K^T: 8 consecutive dims of one token per
// lane) and dim-major (the B operand of P.V: 8 consecutive tokens of one dim
// per lane), the latter through 4x4 byte transposes in registers.  Wave w
// owns latent tile w (128 dims): it scores the chunk against its tile with
// bf16 MFMAs on exactly converted fp8 codes, scales each token's partial by
// its tile scale, and adds one of the four RoPE MFMAs; the four partials are
// summed through LDS.  Every wave then runs the same online softmax and
// multiplies P (times its tile's scales, in bf16) by its tile of V.  With
// several splits the partial (m, l, O) go to a workspace and a second
// kernel combines them.

typedef __bf16 v8bf16 __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));
typedef __bf16 v4bf16 __attribute__((ext_vector_type(4)));

constexpr int kMlaHg = 16;     // heads per workgroup (narrow kernel) and per wave (wide)
constexpr int kMlaWideHeads = 64;  // heads per workgroup of the wide kernel
constexpr int kMlaChunk = 32;  // slots per chunk
constexpr int kMlaKmPitch = kMlaKv + 8;   // token-major LDS row pitch (bytes): 130 words, so 16 rows' 8-byte operand reads cover the 32 banks once
constexpr int kMlaVtPitch = kMlaKv + 16;  // dim-major slab pitch (words)
constexpr int kMlaPePitch = kMlaRope + 8;  // RoPE LDS row pitch (bf16 values)

namespace {

// 8 fp8 e4m3fn codes -> 8 bf16 (exact: every e4m3 value is a bf16 value)
__device__ __forceinline__ v8bf16 fp8x8_to_bf16(uint2 c) {
  const v2bf16 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.x, 1.0f, false);
  const v2bf16 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.x, 1.0f, true);
  const v2bf16 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.y, 1.0f, false);
  const v2bf16 e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.y, 1.0f, true);
  return v8bf16{a[0], a[1], b[0], b[1], d[0], d[1], e[0], e[1]};
}

__device__ __forceinline__ v8bf16 as_bf16x8(uint4 u) {
  v8bf16 r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// max over the 16 lanes that share lane / 16
__device__ __forceinline__ float max16(float v) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 16));
  return v;
}
__device__ __forceinline__ float sum16(float v) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, 16);
  return v;
}

// One staged chunk of 32 entries.
struct alignas(16) MlaChunkLds {
  uint8_t km[kMlaChunk][kMlaKmPitch];     // codes, token-major (padded rows)
  // codes dim-major, one slab per 4 consecutive tokens: word d of slab q
  // holds dim d of tokens 4q..4q+3 (byte i = token 4q+i); slabs padded so
  // that the two slabs one P.V operand reads fall in different banks
  uint32_t vt[kMlaChunk / 4][kMlaVtPitch];
  uint16_t pe[kMlaChunk][kMlaPePitch];    // RoPE values (bf16), padded rows
  float sct[4][kMlaChunk];                // tile scales, [tile][token]
  int valid[kMlaChunk];
};

struct alignas(16) MlaSmem {
  MlaChunkLds c;
  float part[4][2][64][4];                // per-wave partial scores (C layout)
  uint16_t p[4][kMlaHg][kMlaChunk];       // per-wave P * tile scale (bf16), [head][token]
};

// Registers holding one chunk of gathered entries for one thread:
// codes of tokens 4*(t/32)+0..3 at bytes [16*(t%32), +16), the RoPE piece
// (token t/8, bytes 16*(t%8)) and, for t < 32, the scales of token t.
struct MlaStage {
  uint4 c[4];
  uint4 pe;
  uint4 sc;
  int valid;       // token t < 32: slot valid
  uint32_t vmask;  // bit j: chunk token j valid
};

// Lane l of every wave loads the slot id of chunk token l & 31, without a
// branch (lim > 0 whenever this runs; a position past lim is masked where
// the id is used, one chunk later, so that nothing waits on this load early).
__device__ __forceinline__ int mla_load_id(const int32_t* __restrict__ srow, int base, int lim) {
  return srow[min(base + (int)(threadIdx.x & 31), lim - 1)];
}

// Issues the loads of one chunk's entries.  Each lane turns its token's id
// into an entry offset (one 32-bit division); the loading threads fetch the
// offsets they need by lane shuffle.  An invalid id (padding, outside the
// cache, past the split) points at entry 0, so every load is unconditional
// and in bounds.
__device__ __forceinline__ MlaStage mla_gather(const uint8_t* __restrict__ cache, int id, int base,
                                               int lim, int64_t num_slots, uint32_t block_size,
                                               int64_t block_stride) {
  const int t = threadIdx.x;
  const bool ok = base + (t & 31) < lim && id >= 0 && (int64_t)id < num_slots;
  const uint32_t s = ok ? (uint32_t)id : 0u;
  const uint32_t blk = s / block_size;
  const int64_t off = (int64_t)blk * block_stride + (int64_t)(s - blk * block_size) * kMlaEntry;
  const int lo = (int)(uint32_t)off, hi = (int)(uint32_t)((uint64_t)off >> 32);
  auto off_of = [&](int j) {  // j: lane holding the token's offset
    return (int64_t)(((uint64_t)(uint32_t)__shfl(hi, j) << 32) | (uint32_t)__shfl(lo, j));
  };
  MlaStage st;
  const int tg = t >> 5, dp = t & 31;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    st.c[i] = *reinterpret_cast<const uint4*>(cache + off_of(4 * tg + i) + 16 * dp);
  st.pe = *reinterpret_cast<const uint4*>(cache + off_of(t >> 3) + kMlaRopeOff + 16 * (t & 7));
  st.sc = *reinterpret_cast<const uint4*>(cache + off + kMlaScaleOff);  // token t & 31
  st.valid = ok;
  st.vmask = (uint32_t)__ballot(ok);  // lanes 0..31 hold tokens 0..31
  return st;
}

// 4x4 byte transpose: out[d] byte i = in[i] byte d
__device__ __forceinline__ void tr4x4(uint32_t a, uint32_t b, uint32_t c, uint32_t d, uint32_t (&o)[4]) {
  // pairs first: ab_lo = [a0 b0 a1 b1], ab_hi = [a2 b2 a3 b3], same for cd
  const uint32_t ab_lo = __builtin_amdgcn_perm(b, a, 0x05010400u);
  const uint32_t ab_hi = __builtin_amdgcn_perm(b, a, 0x07030602u);
  const uint32_t cd_lo = __builtin_amdgcn_perm(d, c, 0x05010400u);
  const uint32_t cd_hi = __builtin_amdgcn_perm(d, c, 0x07030602u);
  o[0] = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x05040100u);  // a0 b0 c0 d0
  o[1] = __builtin_amdgcn_perm(cd_lo, ab_lo, 0x07060302u);  // a1 b1 c1 d1
  o[2] = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x05040100u);
  o[3] = __builtin_amdgcn_perm(cd_hi, ab_hi, 0x07060302u);
}

// Invalid tokens (padding, ids outside the cache, past the split) were read
// from entry 0; their codes and scales are staged as zeros, so whatever
// bytes that entry holds cannot reach a product (their weights are 0 and
// 0 * NaN would not be).
__device__ __forceinline__ void mla_stage_to_lds(MlaChunkLds& sm, const MlaStage& st) {
  const int t = threadIdx.x;
  const int tg = t >> 5, dp = t & 31;
  uint4 c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool v = (st.vmask >> (4 * tg + i)) & 1u;
    c[i] = v ? st.c[i] : make_uint4(0u, 0u, 0u, 0u);
    // two 8-byte stores: rows are 8-byte (not 16-byte) aligned
    *reinterpret_cast<uint2*>(&sm.km[4 * tg + i][16 * dp]) = make_uint2(c[i].x, c[i].y);
    *reinterpret_cast<uint2*>(&sm.km[4 * tg + i][16 * dp + 8]) = make_uint2(c[i].z, c[i].w);
  }
  const uint32_t w[4][4] = {{c[0].x, c[0].y, c[0].z, c[0].w},
                            {c[1].x, c[1].y, c[1].z, c[1].w},
                            {c[2].x, c[2].y, c[2].z, c[2].w},
                            {c[3].x, c[3].y, c[3].z, c[3].w}};
  // this thread's 4 tokens x 16 dims, transposed: 64 contiguous bytes of slab tg
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t o[4];
    tr4x4(w[0][q], w[1][q], w[2][q], w[3][q], o);
    *reinterpret_cast<uint4*>(&sm.vt[tg][16 * dp + 4 * q]) = make_uint4(o[0], o[1], o[2], o[3]);
  }
  *reinterpret_cast<uint4*>(&sm.pe[t >> 3][8 * (t & 7)]) = st.pe;
  if (t < kMlaChunk) {
    sm.sct[0][t] = st.valid ? __uint_as_float(st.sc.x) : 0.0f;
    sm.sct[1][t] = st.valid ? __uint_as_float(st.sc.y) : 0.0f;
    sm.sct[2][t] = st.valid ? __uint_as_float(st.sc.z) : 0.0f;
    sm.sct[3][t] = st.valid ? __uint_as_float(st.sc.w) : 0.0f;
    sm.valid[t] = st.valid;
  }
}

// The same chunk staged by 512 threads: thread t loads 8 code bytes of 4
// tokens (tokens 4(t/64)..+3, bytes 8(t%64)..+7) and one 16-byte piece of an
// entry's tail: a RoPE piece for t < 256 (token t/8, piece t%8), the tile
// scales of token t%32 otherwise.
struct MlaStage8 {
  uint2 c[4];
  uint4 tail;
  int valid;       // token t % 32: slot valid
  uint32_t vmask;  // bit j: chunk token j valid
};

__device__ __forceinline__ MlaStage8 mla_gather8(const uint8_t* __restrict__ cache, int id, int base,
                                                 int lim, int64_t num_slots, uint32_t block_size,
                                                 int64_t block_stride) {
  const int t = threadIdx.x;
  const bool ok = base + (t & 31) < lim && id >= 0 && (int64_t)id < num_slots;
  const uint32_t s = ok ? (uint32_t)id : 0u;
  const uint32_t blk = s / block_size;
  const int64_t off = (int64_t)blk * block_stride + (int64_t)(s - blk * block_size) * kMlaEntry;
  const int lo = (int)(uint32_t)off, hi = (int)(uint32_t)((uint64_t)off >> 32);
  auto off_of = [&](int j) {  // j: lane holding the token's offset
    return (int64_t)(((uint64_t)(uint32_t)__shfl(hi, j) << 32) | (uint32_t)__shfl(lo, j));
  };
  MlaStage8 st;
  const int tg = __builtin_amdgcn_readfirstlane(t >> 6), dp = t & 63;
  // the four code tokens of a wave are the same for all its lanes: their
  // offsets come through scalar lane reads, not lane shuffles
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t ol = (uint32_t)__builtin_amdgcn_readlane(lo, 4 * tg + i);
    const uint32_t oh = (uint32_t)__builtin_amdgcn_readlane(hi, 4 * tg + i);
    st.c[i] = *reinterpret_cast<const uint2*>(cache + (int64_t)(((uint64_t)oh << 32) | ol) + 8 * dp);
  }
  const int64_t tail = t < 256 ? off_of((t >> 3) & 31) + kMlaRopeOff + 16 * (t & 7) : off + kMlaScaleOff;
  st.tail = *reinterpret_cast<const uint4*>(cache + tail);
  st.valid = ok;
  st.vmask = (uint32_t)__ballot(ok);  // lanes 0..31 hold tokens 0..31
  return st;
}


__global__ __launch_bounds__(256) void sparse_mla_decode_kernel(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_pe, int heads,
    const uint8_t* __restrict__ cache, int64_t num_slots, int64_t block_size, int64_t block_stride,
    const int32_t* __restrict__ slots, int k, float sm_log2, int nsplit, int split_len, int rows,
    float* __restrict__ out, float* __restrict__ lse, float* __restrict__ ws_o,
    float* __restrict__ ws_ml) {
  __shared__ MlaSmem sm;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int ngroups = heads / kMlaHg;
  const int split = blockIdx.x % nsplit;
  const int hg = (blockIdx.x / nsplit) % ngroups;
  const int row = blockIdx.x / (nsplit * ngroups);
  const int base0 = split * split_len;
  const int lim = min(k, base0 + split_len);
  const int32_t* srow = slots + (int64_t)row * k;

  // A operands: wave w's latent tile (4 steps of 32 dims) and its RoPE step
  const int head = hg * kMlaHg + n;  // row n of the A operand
  const uint16_t* qn = q_nope + ((int64_t)row * heads + head) * kMlaKv + w * kMlaTile;
  v8bf16 qa[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) qa[s] = as_bf16x8(*reinterpret_cast<const uint4*>(qn + 32 * s + 8 * g));
  const int rope_nb = w >> 1, rope_ks = w & 1;  // this wave's RoPE MFMA: token block, 32-dim step
  const v8bf16 qp = as_bf16x8(*reinterpret_cast<const uint4*>(
      q_pe + ((int64_t)row * heads + head) * kMlaRope + 32 * rope_ks + 8 * g));

  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  float m[4], l[4];  // running max (log2 units) and sum for heads 4g..4g+3
  v4f o[8];          // O for heads 4g..4g+3, dims w*128 + nb*16 + n
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    m[e] = -INFINITY;
    l[e] = 0.0f;
  }
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) o[nb] = zero;

  // Entries are gathered one chunk ahead, slot ids two chunks ahead.
  if (base0 < lim) {  // uniform
    int id = mla_load_id(srow, base0, lim);
    MlaStage st = mla_gather(cache, id, base0, lim, num_slots, (uint32_t)block_size, block_stride);
    id = mla_load_id(srow, base0 + kMlaChunk, lim);
    for (int base = base0; base < lim; base += kMlaChunk) {
      __syncthreads();  // the previous chunk is no longer read
      mla_stage_to_lds(sm.c, st);
      st = mla_gather(cache, id, base + kMlaChunk, lim, num_slots, (uint32_t)block_size, block_stride);
      id = mla_load_id(srow, base + 2 * kMlaChunk, lim);
      __syncthreads();

      // partial scores: this wave's tile (scaled per token) + one RoPE step
      v4f acc[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        v4f a = zero;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint2 c = *reinterpret_cast<const uint2*>(&sm.c.km[16 * nb + n][w * kMlaTile + 32 * s + 8 * g]);
          a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], fp8x8_to_bf16(c), a, 0, 0, 0);
        }
        const float scl = sm.c.sct[w][16 * nb + n];  // token 16nb+n, tile w
        acc[nb] = a * scl;
      }
      {
        const uint4 pe = *reinterpret_cast<const uint4*>(&sm.c.pe[16 * rope_nb + n][32 * rope_ks + 8 * g]);
        const v4f r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qp, as_bf16x8(pe), zero, 0, 0, 0);
        if (rope_nb == 0) acc[0] += r;
        else acc[1] += r;
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) *reinterpret_cast<v4f*>(&sm.part[w][nb][lane][0]) = acc[nb];
      __syncthreads();
      // full scores in log2 units; lane (g, n): heads 4g+e, tokens n and 16+n
      float sc[2][4];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        v4f s = *reinterpret_cast<const v4f*>(&sm.part[0][nb][lane][0]);
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) s += *reinterpret_cast<const v4f*>(&sm.part[ww][nb][lane][0]);
        const bool ok = sm.c.valid[16 * nb + n] != 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[nb][e] = ok ? s[e] * sm_log2 : -INFINITY;
      }
      // online softmax (every wave computes the same), P * tile-w scale to LDS
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float cm = max16(fmaxf(sc[0][e], sc[1][e]));
        const float mn = fmaxf(m[e], cm);
        const float corr = mn == -INFINITY ? 1.0f : exp2f(m[e] - mn);
        float ps = 0.0f;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const float p = mn == -INFINITY ? 0.0f : exp2f(sc[nb][e] - mn);
          ps += p;
          sm.p[w][4 * g + e][16 * nb + n] = (uint16_t)f32_to_bf16_rne(p * sm.c.sct[w][16 * nb + n]);
        }
        l[e] = l[e] * corr + sum16(ps);
        m[e] = mn;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) o[nb][e] *= corr;
      }
      // the P tile was written by other lanes of this wave
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const v8bf16 pa = as_bf16x8(*reinterpret_cast<const uint4*>(&sm.p[w][n][8 * g]));
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const int d = w * kMlaTile + 16 * nb + n;  // tokens 8g..8g+7 of dim d
        const uint2 c = make_uint2(sm.c.vt[2 * g][d], sm.c.vt[2 * g + 1][d]);
        o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, fp8x8_to_bf16(c), o[nb], 0, 0, 0);
      }
    }
  }

  // lane (g, n): heads 4g+e, dims w*128 + nb*16 + n
  const int64_t rh0 = (int64_t)row * heads + hg * kMlaHg;
  if (nsplit == 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float inv = l[e] > 0.0f ? 1.0f / l[e] : 0.0f;
      float* dst = out + (rh0 + 4 * g + e) * kMlaKv + w * kMlaTile + n;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) dst[16 * nb] = o[nb][e] * inv;
      if (lse && w == 0 && n == 0)
        lse[rh0 + 4 * g + e] = l[e] > 0.0f ? (m[e] + __log2f(l[e])) * 0.69314718055994531f : -INFINITY;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t rhs = (rh0 + 4 * g + e) * nsplit + split;
      float* dst = ws_o + rhs * kMlaKv + w * kMlaTile + n;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) dst[16 * nb] = o[nb][e];
      if (w == 0 && n == 0) {
        ws_ml[2 * rhs] = m[e];
        ws_ml[2 * rhs + 1] = l[e];
      }
    }
  }
}

// The wide kernel stages each chunk as bf16, converted once per workgroup
// (every fp8 code is a bf16 value), in one [slot][dim] layout read two ways:
// the Q.K^T operands are 16-byte row reads (8 dims of one slot), and the P.V
// operands come through ds_read_b64_tr_b16, which hands lane n of a 16-lane
// group element n of four rows (4 slots of one dim).  16-byte chunk c of
// slot r sits at c ^ mla_swz(r): eight consecutive slots then put one chunk
// in eight different 16-byte bank groups (the row reads take 8 lanes a
// cycle) and four consecutive slots put a 32-byte chunk pair in four
// different 32-byte groups (the transposing reads take 16 lanes a cycle).
__device__ __forceinline__ int mla_swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

struct alignas(16) MlaChunkBf {
  uint4 kv[kMlaChunk][kMlaKv / 8];    // latent values, bf16, swizzled chunks
  uint4 pe[kMlaChunk][kMlaRope / 8];  // RoPE values, bf16, swizzled chunks
  float sct[4][kMlaChunk];            // tile scales, [tile][token]
  int valid[kMlaChunk];
};

// mla_gather8's registers -> a bf16 chunk (invalid tokens as zero codes and
// scales, see mla_stage_to_lds).
__device__ __forceinline__ void mla_stage8_to_lds_bf(MlaChunkBf& sm, const MlaStage8& st) {
  const int t = threadIdx.x;
  const int tg = t >> 6, dp = t & 63;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * tg + i;
    const bool v = (st.vmask >> r) & 1u;
    const v8bf16 b = fp8x8_to_bf16(v ? st.c[i] : make_uint2(0u, 0u));
    uint4 u;
    __builtin_memcpy(&u, &b, 16);
    sm.kv[r][dp ^ mla_swz(r)] = u;
  }
  if (t < 256) {
    const int r = t >> 3;
    sm.pe[r][(t & 7) ^ mla_swz(r)] = st.tail;
  } else if (t < 256 + kMlaChunk) {
    const int j = t - 256;
    sm.sct[0][j] = st.valid ? __uint_as_float(st.tail.x) : 0.0f;
    sm.sct[1][j] = st.valid ? __uint_as_float(st.tail.y) : 0.0f;
    sm.sct[2][j] = st.valid ? __uint_as_float(st.tail.z) : 0.0f;
    sm.sct[3][j] = st.valid ? __uint_as_float(st.tail.w) : 0.0f;
    sm.valid[j] = st.valid;
  }
}

typedef short v4s16 __attribute__((ext_vector_type(4)));

// 4 bf16 of one dim for four consecutive slots (ds_read_b64_tr_b16), from a
// byte address inside the LDS chunk.
__device__ __forceinline__ v4s16 lds_tr4(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s16*)(const_cast<uint8_t*>(p)));
}

// 64 heads per workgroup in eight waves: wave w takes heads 16(w%4)..+15
// and latent tiles 2(w/4), 2(w/4)+1 (value dims 256(w/4)..+255) plus RoPE
// step w/4.  The two waves of a head block add their partial scores through
// LDS, so each wave holds a quarter of Q and half of O (under 256
// registers: two waves share a SIMD), and the eight waves share the staged
// chunks (three rotating buffers, one barrier per chunk).
// Scores are formed transposed, S^T = K Q^T: lane (g, n) then holds head n
// for tokens 4g..4g+3 and 16+4g..16+4g+3, which are exactly the eight
// tokens it supplies as the A operand of P.V when the B operand (V) is read
// with two transposing reads of slots 4g..4g+3 and 16+4g..16+4g+3.  The
// softmax state of head n is therefore per lane; the running max is shared
// by the four lanes of a head (two shuffles a chunk) and the running sum is
// reduced once at the end.  O is rescaled
// only when a head's max grows by more than 2^8 (until then the weights
// 2^(s - m) stay below 2^8, harmless in bf16 and fp32).
__global__ __launch_bounds__(512) void sparse_mla_decode_wide_kernel(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_pe, int heads,
    const uint8_t* __restrict__ cache, int64_t num_slots, int64_t block_size, int64_t block_stride,
    const int32_t* __restrict__ slots, int k, float sm_log2, int nsplit, int split_len, int rows,
    float* __restrict__ out, float* __restrict__ lse, float* __restrict__ ws_o,
    float* __restrict__ ws_ml) {
  __shared__ MlaChunkBf buf[3];
  __shared__ v4f xs[2][4][2][2][64];  // partial scores [chunk parity][head block][tile half][token half][lane]
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = lane >> 4, n = lane & 15;
  // Workgroup g runs on XCD g % 8.  The head groups of one (row, split) pair
  // take the same g % 8 and neighbouring dispatch slots, so they read the
  // pair's entries through one XCD's L2 at about the same time.
  const int ngroups = heads / kMlaWideHeads;
  const int xcd = blockIdx.x & 7, jx = blockIdx.x >> 3;
  const int hg = jx % ngroups;
  const int pair = (jx / ngroups) * 8 + xcd;
  if (pair >= rows * nsplit) return;  // grid padded to a multiple of 8 pairs
  const int split = pair % nsplit;
  const int row = pair / nsplit;
  const int base0 = split * split_len;
  const int lim = min(k, base0 + split_len);
  const int32_t* srow = slots + (int64_t)row * k;
  const int hw = wv & 3, dh = wv >> 2;  // head block, value-dim half
  const int head0 = hg * kMlaWideHeads + hw * kMlaHg;  // this wave's 16 heads

  // B operands of S^T: lane (g, n) holds head head0+n, dims 256dh + 32s+8g .. +7
  // of the latent part and 32dh+8g .. +7 of the RoPE part
  const int64_t qh = (int64_t)row * heads + head0 + n;
  v8bf16 qa[kMlaKv / 64];
#pragma unroll
  for (int s = 0; s < kMlaKv / 64; ++s)
    qa[s] = as_bf16x8(*reinterpret_cast<const uint4*>(q_nope + qh * kMlaKv + 256 * dh + 32 * s + 8 * g));
  const v8bf16 qp = as_bf16x8(*reinterpret_cast<const uint4*>(q_pe + qh * kMlaRope + 32 * dh + 8 * g));

  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  v4f o[kMlaKv / 32];  // O rows = heads head0+4g+e, column dim 256dh + 16i + n
#pragma unroll
  for (int i = 0; i < kMlaKv / 32; ++i) o[i] = zero;
  float m_run = -INFINITY, l_run = 0.0f;  // head head0+n (l: this lane's tokens only)

  const int nchunks = base0 < lim ? (lim - base0 + kMlaChunk - 1) / kMlaChunk : 0;
  if (nchunks > 0) {  // uniform
    int id = mla_load_id(srow, base0, lim);
    MlaStage8 st = mla_gather8(cache, id, base0, lim, num_slots, (uint32_t)block_size, block_stride);
    id = mla_load_id(srow, base0 + kMlaChunk, lim);
    mla_stage8_to_lds_bf(buf[0], st);
    st = mla_gather8(cache, id, base0 + kMlaChunk, lim, num_slots, (uint32_t)block_size, block_stride);
    id = mla_load_id(srow, base0 + 2 * kMlaChunk, lim);
    __syncthreads();
    // per-lane byte offsets inside a chunk (the rest of each address is a
    // compile-time constant): Q.K^T rows n and 16+n, 16-byte chunks 4s+g
    // (s even: qk0, odd: qk1) of a 32-dim step; P.V rows 4g+r (and 16+4g+r),
    // n = 4r+q reading 8 bytes of dims 16d + 4q of its row, for d % 4 = 0..3
    const int sw = mla_swz(n);
    const uint32_t qk0 = (uint32_t)(n * kMlaKv * 2 + ((g ^ sw) << 4));
    const uint32_t qk1 = (uint32_t)(n * kMlaKv * 2 + (((4 + g) ^ sw) << 4));
    const int pr = n >> 2, pq = n & 3;
    const int psw = (pr << 1) | (g & 1);  // mla_swz(4g + pr) = mla_swz(16 + 4g + pr)
    uint32_t pvo[4];
#pragma unroll
    for (int d4 = 0; d4 < 4; ++d4)
      pvo[d4] = (uint32_t)((4 * g + pr) * kMlaKv * 2 + (((2 * d4 + (pq >> 1)) ^ psw) << 4) + 8 * (pq & 1));
    int cur = 0, nxt = 1;  // buffers of chunks c and c+1 (three rotate)
    for (int c = 0; c < nchunks; ++c) {
      const MlaChunkBf& b = buf[cur];
      const uint8_t* kvb = reinterpret_cast<const uint8_t*>(&b.kv[0][0]);
      v4f s0 = zero, s1 = zero;
      auto qk = [&]() __attribute__((always_inline)) {
        // partial S^T over this wave's two tiles (each scaled) and RoPE step,
        // tokens n (acc 0) and 16+n (acc 1)
#pragma unroll
        for (int w2 = 0; w2 < 2; ++w2) {
          const int w = 2 * dh + w2;
          v4f a0 = zero, a1 = zero;
#pragma unroll
          for (int st4 = 0; st4 < 4; ++st4) {
            // chunk 16w + 4 st4 + g: bits 3+ are constant, bits 0-2 come from the lane
            const uint8_t* rp = kvb + (st4 & 1 ? qk1 : qk0) + ((16 * w + 8 * (st4 >> 1)) << 4);
            const uint4 c0 = *reinterpret_cast<const uint4*>(rp);
            const uint4 c1 = *reinterpret_cast<const uint4*>(rp + 16 * kMlaKv * 2);
            a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(c0), qa[4 * w2 + st4], a0, 0, 0, 0);
            a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(c1), qa[4 * w2 + st4], a1, 0, 0, 0);
          }
          s0 += a0 * *reinterpret_cast<const v4f*>(&b.sct[w][4 * g]);
          s1 += a1 * *reinterpret_cast<const v4f*>(&b.sct[w][16 + 4 * g]);
        }
        {
          const uint4 p0 = b.pe[n][(4 * dh + g) ^ sw];
          const uint4 p1 = b.pe[16 + n][(4 * dh + g) ^ sw];
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(p0), qp, s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(p1), qp, s1, 0, 0, 0);
        }
        // the pair's halves meet in LDS; both waves form the same sum
        // (x + y == y + x), hence the same softmax state
        xs[c & 1][hw][dh][0][lane] = s0;
        xs[c & 1][hw][dh][1][lane] = s1;
      };
      auto stage = [&]() __attribute__((always_inline)) {
        // One barrier a chunk: before it, stage chunk c+1 into the third
        // buffer (its last reader, chunk c-2's P.V, finished before every wave
        // reached the previous barrier) and issue the loads of chunk c+2; after
        // it, the partial scores and chunk c+1 are visible.  The partial
        // scores alternate between two arrays for the same reason.  Past the
        // end these touch only valid addresses and are never read.
        mla_stage8_to_lds_bf(buf[nxt], st);
        st = mla_gather8(cache, id, base0 + (c + 2) * kMlaChunk, lim, num_slots, (uint32_t)block_size,
                        block_stride);
        id = mla_load_id(srow, base0 + (c + 3) * kMlaChunk, lim);
      };
      // Waves are dealt to the four SIMDs in turn, so waves hw and hw+4 (the
      // two halves of one head block) share a SIMD.  They take the two tasks
      // before the barrier in opposite orders, so that one's MFMAs run while
      // the other converts and stores the next chunk.
      if (dh == 0) {
        qk();
        stage();
      } else {
        stage();
        qk();
      }
      __syncthreads();
      s0 += xs[c & 1][hw][dh ^ 1][0][lane];
      s1 += xs[c & 1][hw][dh ^ 1][1][lane];
      // scores in log2 units; token order 4g+e, then 16+4g+e
      const int4 ok0 = *reinterpret_cast<const int4*>(&b.valid[4 * g]);
      const int4 ok1 = *reinterpret_cast<const int4*>(&b.valid[16 + 4 * g]);
      float sv[8] = {ok0.x ? s0[0] * sm_log2 : -INFINITY, ok0.y ? s0[1] * sm_log2 : -INFINITY,
                     ok0.z ? s0[2] * sm_log2 : -INFINITY, ok0.w ? s0[3] * sm_log2 : -INFINITY,
                     ok1.x ? s1[0] * sm_log2 : -INFINITY, ok1.y ? s1[1] * sm_log2 : -INFINITY,
                     ok1.z ? s1[2] * sm_log2 : -INFINITY, ok1.w ? s1[3] * sm_log2 : -INFINITY};
      float mx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                       fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const bool grow = m_new > m_run + 8.0f;  // m_run = -inf and a finite score: true
      if (__any(grow)) {
        const float corr = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
        l_run *= corr;
        m_run = grow ? m_new : m_run;
        float ce[4];  // factors of O's rows, heads 4g+e (held by lanes 4g+e)
#pragma unroll
        for (int e = 0; e < 4; ++e) ce[e] = __shfl(corr, 4 * g + e);
#pragma unroll
        for (int i = 0; i < kMlaKv / 32; ++i) {
#pragma unroll
          for (int e = 0; e < 4; ++e) o[i][e] *= ce[e];
        }
      }
      const float mu = m_run == -INFINITY ? 0.0f : m_run;  // then every score here is -inf
      float pv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pv[i] = __builtin_amdgcn_exp2f(sv[i] - mu);
        l_run += pv[i];
      }
      // P.V over this wave's two latent tiles: weights times the tile's scales, bf16
#pragma unroll
      for (int w2 = 0; w2 < 2; ++w2) {
        const int w = 2 * dh + w2;
        const v4f t0 = *reinterpret_cast<const v4f*>(&b.sct[w][4 * g]);
        const v4f t1 = *reinterpret_cast<const v4f*>(&b.sct[w][16 + 4 * g]);
        const v8bf16 pa = {(__bf16)(pv[0] * t0[0]), (__bf16)(pv[1] * t0[1]), (__bf16)(pv[2] * t0[2]),
                           (__bf16)(pv[3] * t0[3]), (__bf16)(pv[4] * t1[0]), (__bf16)(pv[5] * t1[1]),
                           (__bf16)(pv[6] * t1[2]), (__bf16)(pv[7] * t1[3])};
#pragma unroll
        for (int d = 0; d < kMlaTile / 16; ++d) {
          // dims 128w + 16d .. +15: 16-byte chunks 16w + 2d + (0, 1); the
          // lane's chunk index XOR its row's swizzle is pvo[d % 4] + 8 (d / 4)
          const uint8_t* vp = kvb + pvo[d & 3] + ((16 * w + 8 * (d >> 2)) << 4);
          const v4s16 lo = lds_tr4(vp);                        // slots 4g .. 4g+3
          const v4s16 hi = lds_tr4(vp + 16 * kMlaKv * 2);      // slots 16+4g .. 16+4g+3
          const v8bf16 vb = __builtin_shufflevector(__builtin_bit_cast(v4bf16, lo), __builtin_bit_cast(v4bf16, hi),
                                                    0, 1, 2, 3, 4, 5, 6, 7);
          o[w2 * 8 + d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, o[w2 * 8 + d], 0, 0, 0);
        }
      }
      cur = nxt;
      nxt = nxt == 2 ? 0 : nxt + 1;
    }
  }

  // row sums over the four lanes of a head; O's rows need heads 4g+e
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const int64_t rh0 = (int64_t)row * heads + head0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float me = __shfl(m_run, 4 * g + e), le = __shfl(l_tot, 4 * g + e);
    const int64_t rh = rh0 + 4 * g + e;
    if (nsplit == 1) {
      const float inv = le > 0.0f ? 1.0f / le : 0.0f;
      float* dst = out + rh * kMlaKv + 256 * dh + n;
#pragma unroll
      for (int i = 0; i < kMlaKv / 32; ++i) dst[16 * i] = o[i][e] * inv;
      if (lse && dh == 0 && n == 0) lse[rh] = le > 0.0f ? (me + __log2f(le)) * 0.69314718055994531f : -INFINITY;
    } else {
      const int64_t rhs = rh * nsplit + split;
      float* dst = ws_o + rhs * kMlaKv + 256 * dh + n;
#pragma unroll
      for (int i = 0; i < kMlaKv / 32; ++i) dst[16 * i] = o[i][e];
      if (dh == 0 && n == 0) {
        ws_ml[2 * rhs] = me;
        ws_ml[2 * rhs + 1] = le;
      }
    }
  }
}

// Combines the splits of one (row, head): 128 threads x 4 dims.
__global__ __launch_bounds__(128) void sparse_mla_combine_kernel(const float* __restrict__ ws_o,
                                                                 const float* __restrict__ ws_ml,
                                                                 int nsplit, float* __restrict__ out,
                                                                 float* __restrict__ lse) {
  const int64_t rh = blockIdx.x;
  const float* ml = ws_ml + rh * nsplit * 2;
  float mx = -INFINITY;
  for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, ml[2 * s]);
  float L = 0.0f;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int s = 0; s < nsplit; ++s) {
    const float ms = ml[2 * s], ls = ml[2 * s + 1];
    const float f = (mx == -INFINITY || ls == 0.0f) ? 0.0f : exp2f(ms - mx);
    L += ls * f;
    const float4 v = *reinterpret_cast<const float4*>(ws_o + (rh * nsplit + s) * kMlaKv + 4 * threadIdx.x);
    acc.x += v.x * f;
    acc.y += v.y * f;
    acc.z += v.z * f;
    acc.w += v.w * f;
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  *reinterpret_cast<float4*>(out + rh * kMlaKv + 4 * threadIdx.x) =
      make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (lse && threadIdx.x == 0) lse[rh] = L > 0.0f ? (mx + __log2f(L)) * 0.69314718055994531f : -INFINITY;
}

// Launch plan: the wide kernel when the heads come in groups of 64 (one
// workgroup per CU), else the narrow one (16 heads, about two per CU); the
// slot list is split in 32-slot multiples until the grid fills the chip.
struct MlaPlan {
  bool wide;
  int nsplit;     // splits actually launched
  int split_len;  // slots per split (multiple of 32)
  int64_t grid;
};

MlaPlan mla_plan(int64_t rows, int heads, int k) {
  MlaPlan p;
  p.wide = heads % kMlaWideHeads == 0;
  const int64_t wgs = rows * (heads / (p.wide ? kMlaWideHeads : kMlaHg));
  const int64_t target = p.wide ? 256 : 512;
  const int kk = std::max(k, 1);
  const int max_split = (kk + kMlaChunk - 1) / kMlaChunk;
  int64_t ns = (target + wgs - 1) / std::max<int64_t>(wgs, 1);
  ns = std::min<int64_t>(std::max<int64_t>(ns, 1), std::min(max_split, 16));
  p.split_len = (int)(((kk + ns - 1) / ns + kMlaChunk - 1) / kMlaChunk * kMlaChunk);
  p.nsplit = (kk + p.split_len - 1) / p.split_len;
  // the wide kernel pads its pairs (row, split) to a multiple of 8 (XCD map)
  p.grid = p.wide ? (rows * p.nsplit + 7) / 8 * 8 * (heads / kMlaWideHeads) : wgs * p.nsplit;
  return p;
}

size_t mla_workspace(int64_t rows, int heads, const MlaPlan& p) {
  return p.nsplit > 1 ? (size_t)rows * heads * p.nsplit * (kMlaKv + 2) * sizeof(float) : 0;
}

}  // namespace

extern "C" size_t sparse_mla_workspace_bytes(int32_t rows, int32_t heads, int32_t k) {
  if (rows <= 0 || heads <= 0 || heads % kMlaHg || heads > 128 || k <= 0) return 0;
  return mla_workspace(rows, heads, mla_plan(rows, heads, k));
}

extern "C" int sparse_mla_decode(const void* q_nope, const void* q_pe, int32_t rows, int32_t heads,
                                 const void* cache, int64_t num_blocks, int32_t block_size,
                                 const int32_t* slots, int32_t k, float sm_scale, float* out,
                                 float* lse, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  if (rows < 0 || heads <= 0 || k < 0 || num_blocks < 0 || block_size <= 0) return SAI_EINVAL;
  if (heads % kMlaHg || heads > 128) return SAI_EUNSUPPORTED;
  if (rows == 0) return SAI_OK;
  if (!q_nope || !q_pe || !cache || !out || (k > 0 && !slots) || num_blocks == 0) return SAI_EINVAL;
  if (!aligned16(q_nope) || !aligned16(q_pe) || !aligned16(cache) || !aligned16(out)) return SAI_EINVAL;
  if (!(sm_scale == sm_scale)) return SAI_EINVAL;
  if (num_blocks > INT64_MAX / ((int64_t)block_size * kMlaEntry)) return SAI_EUNSUPPORTED;
  const MlaPlan p = mla_plan(rows, heads, k);
  const size_t need = mla_workspace(rows, heads, p);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return SAI_EWORKSPACE;
  if (p.grid > 0x7FFFFFFF || (p.nsplit > 1 && (int64_t)rows * heads > 0x7FFFFFFF)) return SAI_EUNSUPPORTED;
  float* ws_o = need ? reinterpret_cast<float*>(workspace) : nullptr;
  float* ws_ml = need ? ws_o + (size_t)rows * heads * p.nsplit * kMlaKv : nullptr;
  launch(p.wide ? sparse_mla_decode_wide_kernel : sparse_mla_decode_kernel, dim3((unsigned)p.grid),
         dim3(p.wide ? 512 : 256), 0, stream, (const uint16_t*)q_nope, (const uint16_t*)q_pe, (int)heads,
         (const uint8_t*)cache, num_blocks * (int64_t)block_size, (int64_t)block_size,
         (int64_t)block_size * kMlaEntry, slots, k, sm_scale * 1.4426950408889634f, p.nsplit,
         p.split_len, (int)rows, out, lse, ws_o, ws_ml);
  if (hipGetLastError() != hipSuccess) return SAI_ELAUNCH;
  if (p.nsplit > 1) {
    launch(sparse_mla_combine_kernel, dim3((unsigned)(rows * (int64_t)heads)), dim3(128), 0, stream,
           (const float*)ws_o, (const float*)ws_ml, p.nsplit, out, lse);
    if (hipGetLastError() != hipSuccess) return SAI_ELAUNCH;
  }
  return SAI_OK;
}
