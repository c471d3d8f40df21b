// Prefill indexer logits on gfx950 (mqa_logits, mqa_logits_chunked): every
// query token of a request scored against the request's contiguous fp8 K
// (the output of gather_indexer_k), with the causal limit of its row.
//
// Score (the DeepSeek-V3.2 lightning indexer; vLLM PR #36250 names the op):
//   L[r, s] = k_scale[s] * sum_h w[r, h] * max(q[r, h, :] . k[s, :], 0)
// on v_mfma_f32_16x16x128_f8f6f4 with the operand and accumulator layouts of
// score_mfma.h (A = 16 heads of one query row, B = 16 keys).
//
// Prefill is fp8-MFMA / VALU co-bound: every key is reused by all later
// tokens, and the epilogue costs two VALU instructions (ReLU, weighted add)
// per score, as many VALU cycles as the MFMAs take.  So the kernel keeps the
// loop down to those instructions:
//  * K reaches LDS by DMA (buffer_load ... lds): no staging registers, no
//    per-block address arithmetic beyond one add per load, and the buffer
//    resource's range check reads zero past the request's keys, so the
//    tail needs no clamps;
//  * a workgroup is a tile of kPfWaves consecutive query rows of one request
//    (one row per wave, Q and head weights in registers for the whole row)
//    and walks the row's key blocks from 0 to the tile's causal limit, so
//    the per-workgroup set-up is paid once per tile rather than per chunk;
//  * a two-slot LDS ring with one barrier per block: a step waits for its
//    own DMA of block j, meets the other waves at the barrier, reads the
//    block's operands and scales, and only then starts the DMA of block
//    j+1 into the other slot (the compiler drains every LDS DMA in flight
//    before any later LDS read, as it cannot tell the slots apart, so no
//    LDS read may follow a DMA within a step); the only global stores in
//    the loop are one 256-byte logit store per block and wave (a buffer
//    store whose range check drops the stores of rows that are not
//    written), so the wait for block j's DMA counts one younger operation;
//  * after the loop each wave writes -inf from the end of its last scored
//    block to the end of its row.
// Tiles are dealt to XCDs by tile % 8, each XCD taking its tiles from the
// last (heaviest, most keys) down.
#include "score_mfma.h"

using namespace sai;
using namespace sai::score;

#ifndef SAI_PF_WAVES
#define SAI_PF_WAVES 4
#endif

namespace {

constexpr int kPfWaves = SAI_PF_WAVES;  // query rows per workgroup, one per wave
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kRing = 2;                                 // LDS K slots
constexpr int kSlotBytes = kValueBytes + kBlock * 4;     // 8448: codes (swizzled), then scales
constexpr int kKLoads = 8 / kPfWaves;                    // 16-byte DMA loads per wave and block
constexpr int kScaleLanes = kBlock / kPfWaves;           // scales loaded per wave and block
static_assert(kKLoads * kPfWaves == 8, "the waves share a block's 8 DMA loads");
constexpr uint32_t kOOB = 0xFFFF0000u;                   // buffer offset past every resource
constexpr int64_t kMaxKeys = kOOB / kDim;                // keys a request's K resource can span
constexpr int64_t kPlainStoreMax = 8 << 20;              // logits written with plain stores

typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* LdsPtr;

// Wave-uniform raw buffer resource over [base, base + bytes): loads past the
// end read zero and stores past it are dropped (word 3: untyped buffer with
// a 32-bit data format, gfx9 encoding).
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

template <bool NT>
__device__ __forceinline__ void buf_store(float v, Rsrc r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, NT ? 2 : 0);
}
template <bool NT>
__device__ __forceinline__ void buf_store4(float v, Rsrc r, uint32_t off) {
  const uint32_t b = __float_as_uint(v);
  const v4u x = {b, b, b, b};
  __builtin_amdgcn_raw_buffer_store_b128(x, r, off, 0, NT ? 2 : 0);
}

// Operands of one block in LDS slot `slot`: key tile t's B operand is chunks
// g and 4+g of key tile_key(t) + n, at byte offsets ra / rb
// (+ tile_key(t) * 128) of the slot; the scale of key `lane`.
struct PfOps {
  v8i b[4];
  float s;
};

__device__ __forceinline__ PfOps read_ops(const uint8_t* slot, uint32_t ra, uint32_t rb) {
  PfOps o;
#pragma unroll
  for (int t = 0; t < 4; ++t)
    o.b[t] = make_v8i(*reinterpret_cast<const uint4*>(slot + tile_key(t) * kDim + ra),
                      *reinterpret_cast<const uint4*>(slot + tile_key(t) * kDim + rb));
  o.s = *reinterpret_cast<const float*>(slot + kValueBytes + 4 * (threadIdx.x & 63));
  return o;
}

// One block's scores for this wave's row: the MFMAs of key tile t are issued
// before tile t-1's ReLU-weighted sums, which then never wait on them.  Lane
// l returns the scaled logit of key l.
__device__ __forceinline__ float score_ops(const PfOps& o, const v8i (&qa)[4], const float4 (&wf)[4]) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  float p[4];
  v4f cprev[4];
#pragma unroll
  for (int t = 0; t <= 4; ++t) {
    v4f ccur[4];
    if (t < 4) {
#pragma unroll
      for (int hg = 0; hg < 4; ++hg)
        ccur[hg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[hg], o.b[t], zero, 0, 0, 0, 0, 0, 0);
    }
    if (t > 0) {
      float acc = 0.0f;
#pragma unroll
      for (int hg = 0; hg < 4; ++hg) acc = relu_dot4(wf[hg], cprev[hg], acc);
      p[t - 1] = acc;
    }
    if (t < 4) {
#pragma unroll
      for (int hg = 0; hg < 4; ++hg) cprev[hg] = ccur[hg];
    }
  }
  // keep that order in the schedule: per tile its 4 MFMAs followed by the
  // previous tile's 32 VALU instructions
#pragma unroll
  for (int t = 0; t <= 4; ++t) {
    if (t < 4) __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    if (t > 0) __builtin_amdgcn_sched_group_barrier(0x002, 32, 0);
  }
  return reduce_scatter4(p[0], p[1], p[2], p[3]) * o.s;
}

// Request b's query rows are [cu[b], cu[b+1]) and its keys the K rows
// [cu_k[b], cu_k[b+1]); the queries are the last n_q of the request's n_k
// tokens, so request-local query i sees keys [0, n_k - n_q + i + 1) (plain
// prefill: cu_k = cu).  Rows whose limit exceeds the stride are not written.
template <bool NT>
__global__ __launch_bounds__(kPfThreads) void prefill_logits_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ wts, const uint8_t* __restrict__ k,
    const float* __restrict__ ks, const int32_t* __restrict__ cu, const int32_t* __restrict__ cu_k,
    int32_t batch, int64_t total_q, int64_t total_k, float* __restrict__ logits, int32_t stride,
    int32_t* __restrict__ row_len_out, int32_t* __restrict__ row_req_out, int32_t ntiles_max, bool vec) {
  extern __shared__ int smem[];
  int* s_tile = smem;                  // [batch+1] prefix of query tiles
  int* scratch = smem + (batch + 1);
  __shared__ __align__(16) uint8_t s_ring[kRing * kSlotBytes];
  __shared__ float4 s_w[kPfWaves][16];

  int run = 0;
  for (int base = 0; base < batch; base += kPfThreads) {
    const int b = base + threadIdx.x;
    int nt = 0;
    if (b < batch) nt = cdiv_i(max(cu[b + 1] - cu[b], 0), kPfWaves);
    int tot;
    const int e = block_exclusive_scan<kPfThreads>(nt, scratch, &tot);
    if (b < batch) s_tile[b] = run + e;
    run += tot;
  }
  if (threadIdx.x == 0) s_tile[batch] = run;
  __syncthreads();

  const int xcd = blockIdx.x & 7, jx = blockIdx.x >> 3;
  const int t8 = (ntiles_max + 7) / 8;
  const int tile = (t8 - 1 - jx) * 8 + xcd;
  if (jx >= t8 || tile >= s_tile[batch] || tile >= ntiles_max) return;
  int lo = 0, hi = batch;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_tile[mid] <= tile) lo = mid; else hi = mid;
  }
  // workgroup-uniform request data, made scalar for the buffer resources
  const int b = __builtin_amdgcn_readfirstlane(lo);
  const int i0 = __builtin_amdgcn_readfirstlane((tile - s_tile[b]) * kPfWaves);
  const int cq0 = __builtin_amdgcn_readfirstlane(cu[b]);
  const int cq1 = __builtin_amdgcn_readfirstlane(cu[b + 1]);
  const int ck0 = __builtin_amdgcn_readfirstlane(cu_k[b]);
  const int ck1 = __builtin_amdgcn_readfirstlane(cu_k[b + 1]);
  const int nq = max(cq1 - cq0, 0);
  const int nk = max(ck1 - ck0, 0);
  const int off = nk - nq;  // keys before the first query's own
  const int len = (int)max64(0, min64(nq, (int64_t)stride - off));  // rows written
  if (i0 >= len) return;
  const int tile_rows = min(kPfWaves, len - i0);
  const int tile_lim = off + i0 + tile_rows;  // keys the tile's last row sees
  const int nblk = tile_lim > 0 ? cdiv_i(tile_lim, kBlock) : 0;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int i = i0 + wave;  // this wave's request-local row
  const int64_t tok = (int64_t)cq0 + i;
  const bool row_ok = i < len && tok >= 0 && tok < total_q;  // (a row outside q is never touched)
  const int lim = off + i + 1;  // keys row i sees (<= 0: none)

  if (threadIdx.x < kPfWaves * 16) {
    const int r = threadIdx.x >> 4, h4 = threadIdx.x & 15;
    float4 w = make_float4(0, 0, 0, 0);
    const int64_t t = (int64_t)cq0 + i0 + r;
    if (i0 + r < len && t >= 0 && t < total_q) w = *reinterpret_cast<const float4*>(wts + t * kHeads + 4 * h4);
    s_w[r][h4] = w;
  }
  v8i qa[4];
  if (row_ok && nblk > 0) {
    load_qfrag(qa, q + tok * (kHeads * kDim));
  } else {
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) qa[hg] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  }

  // K resources over the request's keys (none outside [0, total_k))
  const int64_t kvalid = ck0 < 0 ? 0 : max64(0, min64((int64_t)nk, total_k - ck0));
  const Rsrc kr = make_rsrc(k + (int64_t)ck0 * kDim, (uint32_t)(kvalid * kDim));
  const Rsrc sr = make_rsrc(ks + ck0, (uint32_t)(kvalid * 4));
  // the row's logits; an empty resource for a row that is not written
  const Rsrc rr = make_rsrc(logits + tok * stride, row_ok ? (uint32_t)stride * 4u : 0u);

  // DMA lane mapping: load u of this wave is instruction ii = wave*kKLoads+u
  // of the block, which fills slot positions 64ii .. 64ii+63; position p =
  // key*8 + c holds 16-byte chunk c ^ (key & 7) of the key, so lane l fetches
  // key 8ii + l/8, chunk (l % 8) ^ (l / 8).
  uint32_t kofs[kKLoads];
#pragma unroll
  for (int u = 0; u < kKLoads; ++u) {
    const int ii = wave * kKLoads + u;
    kofs[u] = (uint32_t)((8 * ii + (lane >> 3)) * kDim + (((lane & 7) ^ (lane >> 3)) * 16));
  }
  const uint32_t sofs = (uint32_t)(wave * kScaleLanes + lane) * 4u;
  auto dma = [&](int slot, int j) {
    uint8_t* base = s_ring + slot * kSlotBytes;
    const bool real = j < nblk;
    const uint32_t kb = real ? (uint32_t)j * (uint32_t)kValueBytes : kOOB;
    const uint32_t sb = real ? (uint32_t)j * (uint32_t)(kBlock * 4) : kOOB;
#pragma unroll
    for (int u = 0; u < kKLoads; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (LdsPtr)(base + 1024 * (wave * kKLoads + u)), 16,
                                               kb + kofs[u], 0, 0, 0);
    if (lane < kScaleLanes)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (LdsPtr)(base + kValueBytes + 4 * wave * kScaleLanes), 4,
                                               sb + sofs, 0, 0, 0);
  };
  dma(0, 0);
  __syncthreads();  // s_w
  float4 wf[4];
#pragma unroll
  for (int hg = 0; hg < 4; ++hg) wf[hg] = s_w[wave][4 * hg + (lane >> 4)];
  // Q is complete before the loop, so no wait for it lands inside
  asm volatile("" ::"v"(qa[0]), "v"(qa[1]), "v"(qa[2]), "v"(qa[3]));

  const int g = lane >> 4, n = lane & 15;
  const uint32_t ra = (uint32_t)(n * kDim + ((g ^ (n & 7)) * 16));
  const uint32_t rb = (uint32_t)(n * kDim + (((4 + g) ^ (n & 7)) * 16));
  // Step j (slot S = j % 2): wait for this wave's DMA of block j (issued in
  // step j-1 before its logit store, the one younger memory operation),
  // publish the slot, read the operands, start block j+1's DMA into the
  // other slot, score, store.  The compiler does not order LDS reads after
  // an LDS DMA the way this needs, hence the explicit wait, with a memory
  // clobber so nothing moves across it.
#define SAI_PF_STEP(S, J)                                                          \
  {                                                                                \
    const int j_ = (J);                                                            \
    if (j_ > 0) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");                   \
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");                          \
    __syncthreads();                                                               \
    const PfOps o = read_ops(s_ring + (S) * kSlotBytes, ra, rb);                   \
    dma((S) ^ 1, j_ + 1);                                                          \
    const float v = score_ops(o, qa, wf);                                          \
    const int col = j_ * kBlock + lane;                                            \
    buf_store<NT>(select_f(col < lim, v, kNegInfBits), rr, (uint32_t)col * 4u);    \
  }
  for (int j = 0; j < nblk; j += kRing) {
    SAI_PF_STEP(0, j)
    if (j + 1 < nblk) SAI_PF_STEP(1, j + 1)
  }
#undef SAI_PF_STEP

  // -inf from the end of the scored blocks to the end of the row
  const float ninf = __uint_as_float(kNegInfBits);
  if (vec) {
    for (int x = nblk * kBlock + 4 * lane; x < stride; x += 256) buf_store4<NT>(ninf, rr, (uint32_t)x * 4u);
  } else {
    for (int x = nblk * kBlock + lane; x < stride; x += 64) buf_store<NT>(ninf, rr, (uint32_t)x * 4u);
  }
  if (lane == 0 && row_ok) {
    if (row_len_out) row_len_out[tok] = max(lim, 0);
    if (row_req_out) row_req_out[tok] = b;
  }
}

int launch_prefill(const void* q_fp8, const float* weights, const void* k_fp8, const float* k_scale,
                   const int32_t* cu_q, const int32_t* cu_k, int32_t batch, int64_t total_q,
                   int64_t total_k, float* logits, int64_t logits_stride, int32_t* row_len_out,
                   int32_t* row_req_out, hipStream_t stream) {
  if (batch < 0 || total_q < 0 || total_k < 0 || logits_stride < 0) return SAI_EINVAL;
  if (batch == 0 || total_q == 0) return SAI_OK;
  if (!q_fp8 || !weights || !cu_q || !cu_k || !logits || logits_stride == 0) return SAI_EINVAL;
  if (total_k > 0 && (!k_fp8 || !k_scale)) return SAI_EINVAL;
  if (!aligned16(q_fp8) || !aligned16(weights) || (total_k > 0 && !aligned16(k_fp8))) return SAI_EINVAL;
  // buffer offsets are 32-bit: a row's logits and a request's K must fit
  if (batch > 4096 || logits_stride >= (int64_t)1 << 30 || total_k > kMaxKeys) return SAI_EUNSUPPORTED;
  const int64_t ntiles = (total_q + kPfWaves - 1) / kPfWaves + batch;
  const int64_t G = 8 * ((ntiles + 7) / 8);
  if (G > 0x7FFFFFFF) return SAI_EUNSUPPORTED;
  // prefix of query tiles [batch+1] + the block scan's scratch [waves+1]
  const size_t lds = (size_t)((batch + 1) + kPfWaves + 1) * sizeof(int);
  const bool vec = logits_stride % 4 == 0 && aligned16(logits);
  if (total_q * logits_stride * (int64_t)sizeof(float) <= kPlainStoreMax)
    launch(prefill_logits_kernel<false>, dim3((unsigned)G), dim3(kPfThreads), lds, stream,
           (const uint8_t*)q_fp8, weights, (const uint8_t*)k_fp8, k_scale, cu_q, cu_k, batch, total_q,
           total_k, logits, (int32_t)logits_stride, row_len_out, row_req_out, (int32_t)ntiles, vec);
  else
    launch(prefill_logits_kernel<true>, dim3((unsigned)G), dim3(kPfThreads), lds, stream,
           (const uint8_t*)q_fp8, weights, (const uint8_t*)k_fp8, k_scale, cu_q, cu_k, batch, total_q,
           total_k, logits, (int32_t)logits_stride, row_len_out, row_req_out, (int32_t)ntiles, vec);
  return hipGetLastError() == hipSuccess ? SAI_OK : SAI_ELAUNCH;
}

}  // namespace

extern "C" int mqa_logits(const void* q_fp8, const float* weights, const void* k_fp8,
                          const float* k_scale, const int32_t* cu_seq_lens, int32_t batch,
                          int64_t total_tokens, float* logits, int64_t logits_stride,
                          int32_t* row_len_out, int32_t* row_req_out, hipStream_t stream) {
  if (total_tokens > 0 && batch > 0 && (!k_fp8 || !k_scale)) return SAI_EINVAL;
  return launch_prefill(q_fp8, weights, k_fp8, k_scale, cu_seq_lens, cu_seq_lens, batch, total_tokens,
                        total_tokens, logits, logits_stride, row_len_out, row_req_out, stream);
}

extern "C" int mqa_logits_chunked(const void* q_fp8, const float* weights, const void* k_fp8,
                                  const float* k_scale, const int32_t* cu_seq_lens_q,
                                  const int32_t* cu_seq_lens_k, int32_t batch, int64_t total_q,
                                  int64_t total_k, float* logits, int64_t logits_stride,
                                  int32_t* row_len_out, int32_t* row_req_out, hipStream_t stream) {
  return launch_prefill(q_fp8, weights, k_fp8, k_scale, cu_seq_lens_q, cu_seq_lens_k, batch, total_q,
                        total_k, logits, logits_stride, row_len_out, row_req_out, stream);
}
