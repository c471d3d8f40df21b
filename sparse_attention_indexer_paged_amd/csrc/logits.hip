// Indexer logits on gfx950: fp8 MFMA contraction + fused ReLU / head-weight /
// scale epilogue.
//
// Score (the DeepSeek-V3.2 lightning indexer; vLLM PR #36250 names the op
// fp8_paged_mqa_logits):
//   L[r, s] = k_scale[s] * sum_h w[r, h] * max(q[r, h, :] . k[s, :], 0)
//
// Mapping onto v_mfma_f32_16x16x128_f8f6f4 (fp8 e4m3 x fp8 e4m3 -> fp32):
//   A (16 x 128) = 16 heads of one query row, B (128 x 16) = 16 keys,
//   so one MFMA gives 16 heads x 16 keys of dot products, and a 64-key cache
//   block of one row takes 4 head groups x 4 key tiles = 16 MFMAs.
// Operand layout: lane l = 16*g + n holds row/column n and 32 bytes of the
// 128-long contraction.  The contraction order only has to agree between A
// and B, so lane (g, n) takes bytes [16g, 16g+16) and [64+16g, 64+16g+16) of
// its head or key row: each dwordx4 load instruction then reads a contiguous
// 64-byte half of every key row it touches, straight from HBM into VGPRs in
// operand order (no LDS round trip; each K byte is used by one wave only).
// Accumulator layout: lane (g, n), register i = head 4g + i of the group, key n.
// Epilogue: each lane folds its 16 heads of one key (4 groups x 4 registers)
// with fp32 max + fma; two cross-lane swaps (v_permlane32_swap,
// v_permlane16_swap) then sum the four lanes that share a key and at the same
// time scatter the 4 key tiles so that lane l ends with key l of the block:
// one coalesced 256-byte store per row.
#include <algorithm>

#include "sai_device.h"

using namespace sai;

#ifndef SAI_DECODE_WAVES
#define SAI_DECODE_WAVES 2048
#endif
#ifndef SAI_DECODE_DEPTH
#define SAI_DECODE_DEPTH 1
#endif
#ifndef SAI_DECODE_CAP
#define SAI_DECODE_CAP 4
#endif
#ifndef SAI_DECODE_STAGE
#define SAI_DECODE_STAGE 2048
#endif

namespace {

// Decode launch shape: waves of the persistent grid (8 per CU), blocks in
// the per-wave register ring (DEPTH-1 blocks in flight while one is scored;
// at 1 each wave loads a block and scores it, and the eight waves of a CU
// keep more K in flight than its miss queue takes, with fewer registers),
// the most units scored per straight-line group, and the floats of each
// wave's LDS result stage.
constexpr int kDecodeWaves = SAI_DECODE_WAVES;
constexpr int kDecodeDepth = SAI_DECODE_DEPTH;
constexpr int kDecodeCap = SAI_DECODE_CAP;
constexpr int kStageFloats = SAI_DECODE_STAGE;
constexpr int kFillCols = 256;  // -inf fill piece: one float4 per lane
constexpr int64_t kPlainStoreMaxBytes = 8 << 20;  // decode logits written with plain stores

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

static inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Key tile t of a 64-key block covers keys tile_key(t) .. tile_key(t)+15.
// After the reduce-scatter, tiles 0,2,1,3 land in lanes 0-15, 16-31, 32-47,
// 48-63; with this assignment lane l holds key l.
__device__ __forceinline__ int tile_key(int t) { return ((t & 1) << 5) | ((t & 2) << 3); }

// The per-lane share of one 64-key block: 4 key tiles x 32 operand bytes,
// plus the scale of key `lane`.
struct KFrag {
  uint4 v[8];
  float s;
};

__device__ __forceinline__ v8i make_v8i(uint4 a, uint4 b) {
  v8i r;
  r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
  r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
  return r;
}

// Loads of one paged block (values, then scales at blk + 8192) in operand
// order: lane (g, n) of key tile t takes bytes [16g, 16g+16) and
// [64+16g, 64+16g+16) of key tile_key(t)+n.  When !real, the same number of
// loads all aim at the first 16 bytes of `dummy`, so every path issues an
// identical instruction stream (the data is then ignored).
__device__ __forceinline__ void load_kfrag_or_dummy(KFrag& f, const uint8_t* __restrict__ blk,
                                                    const uint8_t* __restrict__ dummy, bool real) {
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const uint8_t* base = real ? blk : dummy;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int off = real ? (tile_key(t) + n) * kDim + 16 * g : 0;
    f.v[2 * t] = *reinterpret_cast<const uint4*>(base + off);
    f.v[2 * t + 1] = *reinterpret_cast<const uint4*>(base + off + (real ? 64 : 0));
  }
  f.s = *reinterpret_cast<const float*>(base + (real ? kValueBytes + 4 * lane : 0));
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

// Unscaled head-reduced scores of one 64-key block for one query row; lane l
// returns key l.
__device__ __forceinline__ float score_row(const KFrag& kf, const v8i (&qa)[4], const float4 (&wv)[4]) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  float p[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const v8i b = make_v8i(kf.v[2 * t], kf.v[2 * t + 1]);
    float acc = 0.0f;
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) {
      const v4f c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[hg], b, zero, 0, 0, 0, 0, 0, 0);
      acc = relu_dot4(wv[hg], c, acc);
    }
    p[t] = acc;
  }
  return reduce_scatter4(p[0], p[1], p[2], p[3]);
}

__device__ __forceinline__ int cdiv_i(int a, int b) { return (a + b - 1) / b; }

// ------------------------------------------------------------------ decode
// Scores NS consecutive key blocks of one request (block ids in lanes
// 0..NS-1 of myblk) for its NN query rows and writes the masked logits of
// block i, row r to st[(r * slots + i) * 64 + lane] in LDS.  NS is a
// compile-time count, so the ring below is straight-line code: every slot
// issues the same loads on every path (an invalid block id re-reads one
// 16-byte word of q instead), which lets the in-order vmcnt accounting
// leave the DEPTH-1 prefetched blocks in flight while one is scored.  No
// global store sits in the loop, so no K load ever queues behind one.
template <int NN, int DEPTH, int NS>
__device__ __forceinline__ void score_group(const uint8_t* __restrict__ cache, int64_t num_blocks,
                                            const uint8_t* __restrict__ dummy, int myblk,
                                            const v8i (&qa)[NN][4], const float4 (&wf)[NN][4], int c0,
                                            int ctx, float* st, int slots) {
  const int lane = threadIdx.x & 63;
  KFrag buf[DEPTH];
  bool okb[DEPTH];
  auto issue = [&](int i) {
    const int32_t blk = __builtin_amdgcn_readlane(myblk, i);
    const bool ok = blk >= 0 && blk < num_blocks;
    okb[i % DEPTH] = ok;
    load_kfrag_or_dummy(buf[i % DEPTH], cache + (int64_t)(ok ? blk : 0) * kBlockBytes, dummy, ok);
    // keep the prefetch where it is: the scheduler would otherwise sink
    // these loads down to their use
    __builtin_amdgcn_sched_barrier(0);
  };
#pragma unroll
  for (int i = 0; i < DEPTH - 1 && i < NS; ++i) issue(i);
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    if (i + DEPTH - 1 < NS) issue(i + DEPTH - 1);
    const KFrag& cur = buf[i % DEPTH];
    const int col = (c0 + i) * kBlock + lane;
#pragma unroll
    for (int r = 0; r < NN; ++r) {
      const float sc = score_row(cur, qa[r], wf[r]);
      const float v = select_f(okb[i % DEPTH], sc * cur.s, kNaNBits);
      st[(r * slots + i) * kBlock + lane] = select_f(col < ctx - NN + r + 1, v, kNegInfBits);
    }
  }
}

// Calls score_group with NS == n (1 <= n <= NS; n is wave-uniform).
template <int NN, int DEPTH, int NS>
__device__ __forceinline__ void dispatch_group(int n, const uint8_t* __restrict__ cache, int64_t num_blocks,
                                               const uint8_t* __restrict__ dummy, int myblk,
                                               const v8i (&qa)[NN][4], const float4 (&wf)[NN][4], int c0,
                                               int ctx, float* st, int slots) {
  if (n == NS || NS == 1) {
    score_group<NN, DEPTH, NS>(cache, num_blocks, dummy, myblk, qa, wf, c0, ctx, st, slots);
  } else if constexpr (NS > 1) {
    dispatch_group<NN, DEPTH, NS - 1>(n, cache, num_blocks, dummy, myblk, qa, wf, c0, ctx, st, slots);
  }
}

// Grid of persistent waves, each with an equal share of the work: units
// (b, c) = key block c of request b are flattened in (b, c) order and wave w
// of NW scores units [w*U/NW, (w+1)*U/NW); the -inf fill of the columns past
// each request's last key block is cut into pieces of kFillCols columns,
// flattened and split the same way.  Each workgroup builds the two prefix
// sums over the requests in LDS from the device-side context lengths (no
// host sync).  A wave walks its units in groups of at most CAP blocks of one
// request, stages the logits in its LDS slice and writes them out as
// contiguous row runs (float4 per lane when rows are 16-byte aligned) once
// its units are done or the slice is full.
template <int NN, int DEPTH, int CAP, bool NT>
__global__ __launch_bounds__(256) void paged_logits_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ wts, const uint8_t* __restrict__ cache,
    int64_t num_blocks, const int32_t* __restrict__ bt, int64_t bt_stride,
    const int32_t* __restrict__ ctx_lens, int32_t batch, float* __restrict__ logits,
    int64_t stride, int32_t* __restrict__ row_len_out, int32_t* __restrict__ row_req_out, bool vec,
    bool clean) {
  constexpr int kSlots = kStageFloats / (kBlock * NN);  // staged units per wave
  constexpr int kCap = CAP < kSlots ? CAP : kSlots;      // a group fits the stage
  static_assert(kCap >= 1, "stage too small");
  extern __shared__ float4 smem4[];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  float* stage = reinterpret_cast<float*>(smem4) + wid * kStageFloats;
  int* s_unit = reinterpret_cast<int*>(reinterpret_cast<float*>(smem4) + 4 * kStageFloats);
  int* s_fill = s_unit + (batch + 1);     // [batch+1] prefix of fill pieces
  int* s_ctx = s_unit + 2 * (batch + 1);  // [batch] clamped context
  int* s_tot = s_unit + 3 * (batch + 1);  // [8] per-wave totals

  const int maxc = (int)min64(stride, bt_stride * kBlock);

  int run_u = 0, run_f = 0;
  for (int base = 0; base < batch; base += 256) {
    const int bb = base + threadIdx.x;
    int nu = 0, nf = 0;
    if (bb < batch) {
      const int c = min(max(ctx_lens[bb], 0), maxc);
      s_ctx[bb] = c;
      nu = cdiv_i(c, kBlock);
      // no fill pieces when only the request's own blocks are to be written
      nf = clean ? (int)((max(stride - (int64_t)nu * kBlock, (int64_t)0) + kFillCols - 1) / kFillCols) : 0;
    }
    const int iu = wave_inclusive_scan(nu), jf = wave_inclusive_scan(nf);
    if (lane == 63) {
      s_tot[wid] = iu;
      s_tot[4 + wid] = jf;
    }
    __syncthreads();
    int pu = run_u, pf = run_f;
    for (int k = 0; k < wid; ++k) {
      pu += s_tot[k];
      pf += s_tot[4 + k];
    }
    if (bb < batch) {
      s_unit[bb] = pu + iu - nu;
      s_fill[bb] = pf + jf - nf;
    }
    run_u += s_tot[0] + s_tot[1] + s_tot[2] + s_tot[3];
    run_f += s_tot[4] + s_tot[5] + s_tot[6] + s_tot[7];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    s_unit[batch] = run_u;
    s_fill[batch] = run_f;
  }
  __syncthreads();

  const int G = gridDim.x;
  const int lg = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int w = __builtin_amdgcn_readfirstlane(lg * 4 + wid);
  const int nw = G * 4;

  for (int r = w * 64 + lane; r < batch * NN; r += nw * 64) {
    const int b = r / NN, j = r - b * NN;
    if (row_len_out) row_len_out[r] = max(s_ctx[b] - NN + j + 1, 0);
    if (row_req_out) row_req_out[r] = b;
  }

  // last b in [0, batch) with pre[b] <= u (pre non-decreasing, pre[0] = 0
  // <= u; called wave-uniformly): a coarse ballot over every cs-th entry,
  // then a fine one inside the chosen stretch of cs <= 64 entries
  auto find = [&](const int* pre, int u) {
    const int cs = (batch + 63) >> 6;
    const uint64_t mc = __ballot(pre[min(lane * cs, batch - 1)] <= u);
    const int c = min(63 - (int)__builtin_clzll(mc), (batch - 1) / cs);
    const int j = c * cs + lane;
    const uint64_t mf = __ballot(lane < cs && j < batch && pre[min(j, batch - 1)] <= u);
    return c * cs + (63 - (int)__builtin_clzll(mf));
  };

  // Writes the staged units [sa, sb) (stage slots 0 .. sb-sa-1; unit sa
  // belongs to request bs) to their rows: per request, each row's run of
  // columns is contiguous in LDS and in the logits.
  auto flush = [&](int sa, int sb, int bs) {
    // the stage was written by other lanes of this wave
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int u = sa; u < sb;) {
      while (s_unit[bs + 1] <= u) ++bs;
      const int e = min(sb, s_unit[bs + 1]);
      const int64_t col0 = (int64_t)(u - s_unit[bs]) * kBlock;
      const int ncol = (int)min64((int64_t)(e - u) * kBlock, stride - col0);
#pragma unroll
      for (int r = 0; r < NN; ++r) {
        const float* src = stage + (r * kSlots + (u - sa)) * kBlock;
        float* dst = logits + ((int64_t)bs * NN + r) * stride + col0;
        if (vec) {
          for (int x = 4 * lane; x < ncol; x += 256)
            store_logit4<NT>(dst + x, *reinterpret_cast<const float4*>(src + x));
        } else {
          for (int x = lane; x < ncol; x += 64) store_logit<NT>(dst + x, src[x]);
        }
      }
      u = e;
    }
  };

  // The -inf fill needs only the context lengths, so its stores go out
  // before the K stream starts and complete while the first loads wait.
  const int F = s_fill[batch];
  int f = (int)((int64_t)F * w / nw);
  const int f1 = (int)((int64_t)F * (w + 1) / nw);
  if (f < f1) {
    int b = find(s_fill, f);
    const float ninf = __uint_as_float(kNegInfBits);
    const float4 ninf4 = make_float4(ninf, ninf, ninf, ninf);
    for (; f < f1; ++f) {
      while (s_fill[b + 1] <= f) ++b;
      const int64_t col = (int64_t)(s_unit[b + 1] - s_unit[b]) * kBlock + (int64_t)(f - s_fill[b]) * kFillCols;
#pragma unroll
      for (int r = 0; r < NN; ++r) {
        float* row = logits + ((int64_t)b * NN + r) * stride;
        if (vec) {
          if (col + 4 * lane < stride) store_logit4<NT>(row + col + 4 * lane, ninf4);
        } else {
#pragma unroll
          for (int k = 0; k < kFillCols / 64; ++k)
            if (col + 64 * k + lane < stride) store_logit<NT>(row + col + 64 * k + lane, ninf);
        }
      }
    }
  }
  const int U = s_unit[batch];
  const int u0 = (int)((int64_t)U * w / nw);
  const int u1 = (int)((int64_t)U * (w + 1) / nw);
  // Per group: the block ids come in with one vector load (lane i holds
  // unit i), the query rows are (re)loaded only when the request changes,
  // then a ring of exactly n slots scores the group into the stage.
  int u = u0;
  int b = u0 < u1 ? find(s_unit, u0) : 0;
  int sa = u0, bs = b;  // first staged unit and its request
  int qb = -1;
  v8i qa[NN][4];
  float4 wf[NN][4];
  while (u < u1) {
    while (s_unit[b + 1] <= u) ++b;
    const int n = min(kCap, min(u1, s_unit[b + 1]) - u);  // 1..kCap units of request b
    if (u + n - sa > kSlots) {
      flush(sa, u, bs);
      sa = u;
      bs = b;
    }
    const int c0 = u - s_unit[b];
    const int myblk = lane < n ? bt[(int64_t)b * bt_stride + c0 + lane] : -1;
    if (b != qb) {
      qb = b;
#pragma unroll
      for (int r = 0; r < NN; ++r) {
        load_qfrag(qa[r], q + ((int64_t)qb * NN + r) * (kHeads * kDim));
        load_wfrag(wf[r], wts + ((int64_t)qb * NN + r) * kHeads);
      }
    }
    dispatch_group<NN, DEPTH, kCap>(n, cache, num_blocks, q, myblk, qa, wf, c0, s_ctx[b],
                                    stage + (u - sa) * kBlock, kSlots);
    u += n;
  }
  if (sa < u1) flush(sa, u1, bs);
}

// ------------------------------------------------------------------ prefill
// Prefill is fp8-MFMA / VALU co-bound (every key is reused by all later
// tokens), so K is staged once per workgroup in LDS and shared by its waves.
// Workgroup = kPfTileRows consecutive tokens of one request (kPfWaves waves
// x kPfRowsPerWave query rows, Q in VGPRs, head weights read from LDS) x a
// key chunk of 16 blocks (1024 columns).  The chunk's K blocks stream
// through a double-buffered LDS image: all threads fetch a later block with
// coalesced 16-byte loads while the current one is scored, then write it to
// LDS with the 16-byte chunk c of key n at position c ^ (n & 7) of the key's
// row, so the MFMA operand reads (lanes n = 0..15 of one key tile at a
// 128-byte stride) spread over all LDS banks.  Every column of the chunk is
// written for the tile's rows (-inf past each row's causal limit).  Tiles
// are dealt to XCDs by tile % 8, heaviest first.
#ifndef SAI_PF_ROWS
#define SAI_PF_ROWS 1
#endif
#ifndef SAI_PF_WAVES
#define SAI_PF_WAVES 4
#endif
#ifndef SAI_PF_WF_LDS
#define SAI_PF_WF_LDS 0
#endif
#ifndef SAI_PF_DEPTH
#define SAI_PF_DEPTH 2
#endif
#ifndef SAI_PF_WAVES_PER_EU
#define SAI_PF_WAVES_PER_EU 0
#endif
constexpr int kPfRowsPerWave = SAI_PF_ROWS;
constexpr int kPfWaves = SAI_PF_WAVES;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kPfTileRows = kPfWaves * kPfRowsPerWave;
constexpr int kPfChunksPerThread = 512 / kPfThreads;  // 16-byte chunks of a K block per thread
static_assert(kPfChunksPerThread * kPfThreads == 512, "a K block is 512 chunks of 16 bytes");
constexpr int kPfChunkBlocks = 16;
constexpr int kChunk = kPfChunkBlocks * kBlock;

struct PfBlock {
  uint4 code[kBlock * 8];  // 64 keys x 8 chunks of 16 bytes, swizzled
  float scale[kBlock];
};

__device__ __forceinline__ int pf_swz(int n, int c) { return n * 8 + (c ^ (n & 7)); }

// Global -> registers: thread t fetches chunks t and t+256 of the block
// (key = chunk / 8, 16-byte column = chunk % 8; chunk t+256 is key
// 32 + t/8) and key (t % 64)'s scale.
// Every load is issued unconditionally from a token index clamped into
// [0, total) so that all of them are in flight together; keys past the
// request are zeroed when the block is written to LDS.
struct PfStage {
  uint4 c[kPfChunksPerThread];  // chunks t + kPfThreads * e
  float s;                      // scale of key t % 64
};

__device__ __forceinline__ PfStage pf_fetch(const uint8_t* __restrict__ k, const float* __restrict__ ks,
                                            int64_t key0, int64_t total) {
  const int t = threadIdx.x;
  PfStage st;
  if (key0 + kBlock <= total) {  // wave-uniform: the block lies inside the buffer, no clamp
    const uint8_t* kb = k + key0 * kDim;
#pragma unroll
    for (int e = 0; e < kPfChunksPerThread; ++e)
      st.c[e] = *reinterpret_cast<const uint4*>(kb + (t + kPfThreads * e) * 16);
    st.s = ks[key0 + (t & 63)];
  } else {
#pragma unroll
    for (int e = 0; e < kPfChunksPerThread; ++e) {
      const int chunk = t + kPfThreads * e;
      st.c[e] = *reinterpret_cast<const uint4*>(k + min64(key0 + (chunk >> 3), total - 1) * kDim + (chunk & 7) * 16);
    }
    st.s = ks[min64(key0 + (t & 63), total - 1)];
  }
  return st;
}

// Registers -> LDS image (swizzled), keys at or past nvalid as zero.
// (Masks rather than selects of whole values: a select between a stage
// member and a zero constant can become a select of addresses, which puts
// the stages in scratch memory.)
__device__ __forceinline__ uint4 and4(uint4 v, uint32_t m) { return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m); }

__device__ __forceinline__ void pf_store(PfBlock& blk, const PfStage& st, int nvalid) {
  const int t = threadIdx.x;
  if (nvalid >= kBlock) {  // wave-uniform: every key of the block belongs to the request
#pragma unroll
    for (int e = 0; e < kPfChunksPerThread; ++e) {
      const int chunk = t + kPfThreads * e;
      blk.code[pf_swz(chunk >> 3, chunk & 7)] = st.c[e];
    }
    if (t < kBlock) blk.scale[t] = st.s;
  } else {
#pragma unroll
    for (int e = 0; e < kPfChunksPerThread; ++e) {
      const int chunk = t + kPfThreads * e;
      blk.code[pf_swz(chunk >> 3, chunk & 7)] = and4(st.c[e], (chunk >> 3) < nvalid ? ~0u : 0u);
    }
    if (t < kBlock) blk.scale[t] = __uint_as_float(__float_as_uint(st.s) & (t < nvalid ? ~0u : 0u));
  }
}

// B operand of key tile t: lane (g, n) takes 16-byte columns g and 4+g of key
// tile_key(t)+n, the same contraction order as the paged decode loads.
__device__ __forceinline__ v8i pf_operand(const PfBlock& blk, int t) {
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int key = tile_key(t) + n;
  return make_v8i(blk.code[pf_swz(key, g)], blk.code[pf_swz(key, 4 + g)]);
}

#if SAI_PF_WAVES_PER_EU
#define SAI_PF_ATTR __attribute__((amdgpu_waves_per_eu(SAI_PF_WAVES_PER_EU)))
#else
#define SAI_PF_ATTR
#endif
// Request b's query rows are [cu[b], cu[b+1]) and its keys the K rows
// [cu_k[b], cu_k[b+1]); the queries are the last n_q of the request's n_k
// tokens, so request-local query i sees keys [0, n_k - n_q + i + 1) (plain
// prefill: cu_k = cu).  Rows whose limit exceeds the stride are not written.
__global__ __launch_bounds__(kPfThreads) SAI_PF_ATTR void prefill_logits_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ wts, const uint8_t* __restrict__ k,
    const float* __restrict__ ks, const int32_t* __restrict__ cu, const int32_t* __restrict__ cu_k,
    int32_t batch, int64_t total, float* __restrict__ logits, int64_t stride,
    int32_t* __restrict__ row_len_out, int32_t* __restrict__ row_req_out, int32_t nchunks,
    int32_t ntiles_max, bool vec) {
  extern __shared__ int smem[];
  int* s_tile = smem;                  // [batch+1] prefix of query tiles
  int* scratch = smem + (batch + 1);
  __shared__ PfBlock s_k[2];
  __shared__ float4 s_w[kPfTileRows][16];
  __shared__ __align__(16) float s_res[kPfTileRows][kChunk];  // the chunk's logits per row

  int run = 0;
  for (int base = 0; base < batch; base += kPfThreads) {
    const int b = base + threadIdx.x;
    int nt = 0;
    if (b < batch) {
      const int len = max(cu[b + 1] - cu[b], 0);
      nt = cdiv_i(len, kPfTileRows);
    }
    int tot;
    const int e = block_exclusive_scan<kPfThreads>(nt, scratch, &tot);
    if (b < batch) s_tile[b] = run + e;
    run += tot;
  }
  if (threadIdx.x == 0) s_tile[batch] = run;
  __syncthreads();

  // Workgroup g runs on XCD g % 8.  Tiles are dealt to XCDs by tile % 8, so
  // the causal work (later tiles see more keys) is spread evenly over the
  // XCDs, and each XCD takes its tiles from the last (heaviest) down; the
  // chunks of one tile are consecutive on one XCD and share its Q in L2.
  const int xcd = blockIdx.x & 7, jx = blockIdx.x >> 3;
  const int t8 = (ntiles_max + 7) / 8;
  const int tj = jx / nchunks, chunk = jx - tj * nchunks;
  const int tile = (t8 - 1 - tj) * 8 + xcd;
  if (tj >= t8 || tile >= s_tile[batch] || tile >= ntiles_max) return;
  int lo = 0, hi = batch;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_tile[mid] <= tile) lo = mid; else hi = mid;
  }
  const int b = lo;
  const int64_t base_tok = cu[b];   // first query row
  const int64_t kb0 = cu_k[b];      // first key row
  const int nq = max(cu[b + 1] - cu[b], 0);
  const int nk = max(cu_k[b + 1] - kb0, 0);
  const int off = nk - nq;          // keys before the first query's own
  // rows written: i with off + i + 1 <= stride; keys in play: the first nk
  const int len = (int)max64(0, min64(nq, stride - off));
  const int i0 = (tile - s_tile[b]) * kPfTileRows;
  if (i0 >= len) return;  // the whole tile lies past a clamped request

  if (threadIdx.x < kPfTileRows * 16) {
    const int r = threadIdx.x >> 4, h4 = threadIdx.x & 15;
    float4 w = make_float4(0, 0, 0, 0);
    if (i0 + r < len) w = *reinterpret_cast<const float4*>(wts + (base_tok + i0 + r) * kHeads + 4 * h4);
    s_w[r][h4] = w;
  }

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ir0 = i0 + wave * kPfRowsPerWave;            // first request-local row of this wave
  const int nrows = max(0, min(kPfRowsPerWave, len - ir0));
  const int wlim = off + ir0 + nrows;                    // keys visible to the wave's last row

  if (chunk == 0 && lane < nrows) {
    if (row_len_out) row_len_out[base_tok + ir0 + lane] = max(off + ir0 + lane + 1, 0);
    if (row_req_out) row_req_out[base_tok + ir0 + lane] = b;
  }

  const int col0 = chunk * kChunk;
  const int col_end = (int)min64((int64_t)col0 + kChunk, stride);
  const int kend = min(col_end, off + min(i0 + kPfTileRows, len));  // keys any row of the tile sees
  const int nblk = kend > col0 ? cdiv_i(kend - col0, kBlock) : 0;
  const float ninf = __uint_as_float(kNegInfBits);

  v8i qa[kPfRowsPerWave][4];
#pragma unroll
  for (int r = 0; r < kPfRowsPerWave; ++r) {
    if (r < nrows && nblk > 0) {
      load_qfrag(qa[r], q + (base_tok + ir0 + r) * (kHeads * kDim));
    } else {
#pragma unroll
      for (int hg = 0; hg < 4; ++hg) qa[r][hg] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }

  __syncthreads();  // s_w
  // head weights of lane (g, n): heads 16hg + 4g .. +3, read from LDS in
  // the loop (SAI_PF_WF_LDS, saves 16 VGPRs per row) or kept in registers
#if SAI_PF_WF_LDS
  auto wfr = [&](int r, int hg) { return s_w[wave * kPfRowsPerWave + r][4 * hg + (lane >> 4)]; };
#else
  float4 wf[kPfRowsPerWave][4];
#pragma unroll
  for (int r = 0; r < kPfRowsPerWave; ++r)
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) wf[r][hg] = s_w[wave * kPfRowsPerWave + r][4 * hg + (lane >> 4)];
  auto wfr = [&](int r, int hg) { return wf[r][hg]; };
#endif

  // Software pipeline over the chunk's blocks: block j is scored from LDS
  // buffer j%2 while block j+DEPTH is fetched into registers and block j+1
  // (fetched DEPTH-1 steps earlier) is written to the other buffer.  The
  // loop is unrolled by DEPTH so the register stages rotate statically, and
  // no global store sits in it (results go to s_res), so the in-order vmcnt
  // accounting only ever waits for the oldest fetch.
  const int64_t kbase = kb0 + col0;
  PfStage sa, sb, sc;
  if (nblk > 0) {
    sc = pf_fetch(k, ks, kbase, total);
    pf_store(s_k[0], sc, nk - col0);  // waits for Q and w as well
    sa = pf_fetch(k, ks, kbase + kBlock, total);
    if (SAI_PF_DEPTH > 2) sb = pf_fetch(k, ks, kbase + 2 * kBlock, total);
  }
  __syncthreads();
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  float* res = s_res[wave * kPfRowsPerWave];
  // Scores block J (from LDS) while CUR (block J+1) is written to the other
  // buffer and NXT receives block J+2; a macro rather than a lambda so the
  // two register stages stay plain locals (by-reference stages end up in
  // scratch memory).
#define SAI_PF_STEP(J, CUR, NXT)                                                              \
  {                                                                                           \
    const int j_ = (J);                                                                       \
    NXT = pf_fetch(k, ks, kbase + (int64_t)(j_ + SAI_PF_DEPTH) * kBlock, total);              \
    const int key0 = col0 + j_ * kBlock;                                                      \
    const int col = key0 + lane;                                                              \
    if (j_ < nblk && key0 < wlim) {                                                           \
      const PfBlock& blk = s_k[j_ & 1];                                                       \
      float p[kPfRowsPerWave][4];                                                             \
      /* software pipeline over the 4 key tiles: tile t's MFMAs are issued  */                \
      /* before tile t-1's ReLU-weighted sums, which never wait on them     */                \
      v4f cprev[kPfRowsPerWave][4];                                                           \
      v8i bops[4]; /* all 4 key tiles' operands are read up front */                          \
      _Pragma("unroll") for (int t = 0; t < 4; ++t) bops[t] = pf_operand(blk, t);             \
      _Pragma("unroll") for (int t = 0; t <= 4; ++t) {                                        \
        v4f ccur[kPfRowsPerWave][4];                                                          \
        if (t < 4) {                                                                          \
          const v8i bop = bops[t];                                                            \
          _Pragma("unroll") for (int r = 0; r < kPfRowsPerWave; ++r)                          \
            _Pragma("unroll") for (int hg = 0; hg < 4; ++hg)                                  \
              ccur[r][hg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(                 \
                  qa[r][hg], bop, zero, 0, 0, 0, 0, 0, 0);                                    \
        }                                                                                     \
        if (t > 0) {                                                                          \
          _Pragma("unroll") for (int r = 0; r < kPfRowsPerWave; ++r) {                        \
            float acc = 0.0f;                                                                 \
            _Pragma("unroll") for (int hg = 0; hg < 4; ++hg)                                  \
              acc = relu_dot4(wfr(r, hg), cprev[r][hg], acc);                                 \
            p[r][t - 1] = acc;                                                                \
          }                                                                                   \
        }                                                                                     \
        if (t < 4)                                                                            \
          _Pragma("unroll") for (int r = 0; r < kPfRowsPerWave; ++r)                          \
            _Pragma("unroll") for (int hg = 0; hg < 4; ++hg) cprev[r][hg] = ccur[r][hg];      \
      }                                                                                       \
      /* keep that order in the schedule: the 8 operand reads, then per tile */               \
      /* its MFMAs followed by the previous tile's 32 VALU ops per row      */               \
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);                                      \
      _Pragma("unroll") for (int t = 0; t <= 4; ++t) {                                        \
        if (t < 4) __builtin_amdgcn_sched_group_barrier(0x008, 4 * kPfRowsPerWave, 0);        \
        if (t > 0) __builtin_amdgcn_sched_group_barrier(0x002, 32 * kPfRowsPerWave, 0);       \
      }                                                                                       \
      const float sc = blk.scale[lane];                                                       \
      _Pragma("unroll") for (int r = 0; r < kPfRowsPerWave; ++r) {                            \
        const float v = reduce_scatter4(p[r][0], p[r][1], p[r][2], p[r][3]) * sc;             \
        res[r * kChunk + j_ * kBlock + lane] = select_f(col < off + ir0 + r + 1, v, kNegInfBits); \
      }                                                                                       \
    } else if (j_ < nblk) { /* steps past the last block write nothing */                   \
      _Pragma("unroll") for (int r = 0; r < kPfRowsPerWave; ++r)                              \
        res[r * kChunk + j_ * kBlock + lane] = ninf;                                          \
    }                                                                                         \
    pf_store(s_k[(j_ + 1) & 1], CUR, nk - (key0 + kBlock));                                    \
    __syncthreads();                                                                          \
  }
#if SAI_PF_DEPTH > 2
  // stages rotate: CUR holds block j+1 (fetched two steps ago), NXT gets j+3
  for (int j = 0; j < nblk; j += 3) {
    SAI_PF_STEP(j, sa, sc)
    SAI_PF_STEP(j + 1, sb, sa)
    SAI_PF_STEP(j + 2, sc, sb)
  }
#else
  for (int j = 0; j < nblk; j += 2) {
    SAI_PF_STEP(j, sa, sb)
    SAI_PF_STEP(j + 1, sb, sa)
  }
#endif
#undef SAI_PF_STEP

  // write the wave's rows for the whole chunk: staged blocks, then -inf
  const int nstaged = min(nblk * kBlock, col_end - col0);
  for (int r = 0; r < nrows; ++r) {
    float* dst = logits + (base_tok + ir0 + r) * stride + col0;
    const float* src = res + r * kChunk;
    if (vec) {
      for (int x = 4 * lane; x < col_end - col0; x += 256) {
        const float4 v = x < nstaged ? *reinterpret_cast<const float4*>(src + x)
                                     : make_float4(ninf, ninf, ninf, ninf);
        store_logit4(dst + x, v);
      }
    } else {
      for (int x = lane; x < col_end - col0; x += 64) store_logit(dst + x, x < nstaged ? src[x] : ninf);
    }
  }
}

template <int NN>
int launch_paged(const void* q, const float* w, const void* cache, int64_t num_blocks,
                 const int32_t* bt, int64_t bt_stride, const int32_t* ctx, int32_t batch,
                 float* logits, int64_t stride, int32_t* rl, int32_t* rr, bool clean, hipStream_t s) {
  if (batch > 4096) return SAI_EUNSUPPORTED;  // LDS prefix arrays
  const int64_t wblocks = (stride + kBlock - 1) / kBlock;
  const int64_t units_max = (int64_t)batch * wblocks;
  const int64_t waves = std::min<int64_t>(kDecodeWaves, std::max<int64_t>(units_max, 1));
  int64_t G = (waves + 3) / 4;
  G = (G + 7) / 8 * 8;
  const size_t lds = 4 * kStageFloats * sizeof(float) + (size_t)(3 * (batch + 1) + 8) * sizeof(int);
  if (lds > 65536) {  // large batches need the device's full per-workgroup LDS
    int dev = 0, max_lds = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
      return SAI_ELAUNCH;
    if (lds > (size_t)max_lds) return SAI_EUNSUPPORTED;
  }
  const bool vec = stride % 4 == 0 && aligned16(logits);
  // A logits buffer of at most kPlainStoreMaxBytes is written with plain
  // stores, so the top-k reading it next finds it in the caches (64 rows x
  // 16384 columns: step 35.1 -> 34.3 us); larger ones are streamed past the
  // caches (32 x 131072: plain stores cost 1.2 % of the step; 256 x 65536:
  // even).
  if ((int64_t)batch * NN * stride * (int64_t)sizeof(float) <= kPlainStoreMaxBytes)
    launch((paged_logits_kernel<NN, kDecodeDepth, kDecodeCap, false>), dim3((unsigned)G), dim3(256), lds, s,
           (const uint8_t*)q, w, (const uint8_t*)cache, num_blocks, bt, bt_stride, ctx, batch, logits,
           stride, rl, rr, vec, clean);
  else
    launch((paged_logits_kernel<NN, kDecodeDepth, kDecodeCap, true>), dim3((unsigned)G), dim3(256), lds, s,
           (const uint8_t*)q, w, (const uint8_t*)cache, num_blocks, bt, bt_stride, ctx, batch, logits,
           stride, rl, rr, vec, clean);
  return hipGetLastError() == hipSuccess ? SAI_OK : SAI_ELAUNCH;
}

}  // namespace

namespace {
int paged_entry(const void* q_fp8, const float* weights, const void* kv_cache, int64_t num_blocks,
                const int32_t* block_table, int64_t bt_stride, const int32_t* context_lens,
                int32_t batch, int32_t next_n, float* logits, int64_t logits_stride,
                int32_t* row_len_out, int32_t* row_req_out, bool clean, hipStream_t stream) {
  if (batch < 0 || num_blocks < 0 || bt_stride < 0 || logits_stride < 0) return SAI_EINVAL;
  if (next_n < 1 || next_n > SAI_NEXT_N_MAX) return SAI_EUNSUPPORTED;
  if (batch == 0) return SAI_OK;
  if (!q_fp8 || !weights || !kv_cache || !block_table || !context_lens || !logits) return SAI_EINVAL;
  if (!aligned16(q_fp8) || !aligned16(weights) || !aligned16(kv_cache)) return SAI_EINVAL;
  if (logits_stride == 0) return SAI_EINVAL;
  const int64_t wblocks = (logits_stride + kBlock - 1) / kBlock;
  if ((int64_t)batch * wblocks > 0x7FFFFFFF / 2 || logits_stride > 0x7FFFFFFF - kBlock)
    return SAI_EUNSUPPORTED;
  switch (next_n) {
    case 1: return launch_paged<1>(q_fp8, weights, kv_cache, num_blocks, block_table, bt_stride, context_lens, batch, logits, logits_stride, row_len_out, row_req_out, clean, stream);
    case 2: return launch_paged<2>(q_fp8, weights, kv_cache, num_blocks, block_table, bt_stride, context_lens, batch, logits, logits_stride, row_len_out, row_req_out, clean, stream);
    case 3: return launch_paged<3>(q_fp8, weights, kv_cache, num_blocks, block_table, bt_stride, context_lens, batch, logits, logits_stride, row_len_out, row_req_out, clean, stream);
    default: return launch_paged<4>(q_fp8, weights, kv_cache, num_blocks, block_table, bt_stride, context_lens, batch, logits, logits_stride, row_len_out, row_req_out, clean, stream);
  }
}
}  // namespace

extern "C" int paged_mqa_logits(const void* q_fp8, const float* weights, const void* kv_cache,
                                int64_t num_blocks, const int32_t* block_table, int64_t bt_stride,
                                const int32_t* context_lens, int32_t batch, int32_t next_n,
                                float* logits, int64_t logits_stride, int32_t* row_len_out,
                                int32_t* row_req_out, hipStream_t stream) {
  return paged_entry(q_fp8, weights, kv_cache, num_blocks, block_table, bt_stride, context_lens, batch,
                     next_n, logits, logits_stride, row_len_out, row_req_out, true, stream);
}

extern "C" int paged_mqa_logits_visible(const void* q_fp8, const float* weights, const void* kv_cache,
                                        int64_t num_blocks, const int32_t* block_table,
                                        int64_t bt_stride, const int32_t* context_lens, int32_t batch,
                                        int32_t next_n, float* logits, int64_t logits_stride,
                                        int32_t* row_len_out, int32_t* row_req_out, hipStream_t stream) {
  return paged_entry(q_fp8, weights, kv_cache, num_blocks, block_table, bt_stride, context_lens, batch,
                     next_n, logits, logits_stride, row_len_out, row_req_out, false, stream);
}

namespace {
int launch_prefill(const void* q_fp8, const float* weights, const void* k_fp8, const float* k_scale,
                   const int32_t* cu_q, const int32_t* cu_k, int32_t batch, int64_t total_q,
                   int64_t total_k, float* logits, int64_t logits_stride, int32_t* row_len_out,
                   int32_t* row_req_out, hipStream_t stream) {
  if (batch < 0 || total_q < 0 || total_k < 0 || logits_stride < 0) return SAI_EINVAL;
  if (batch == 0 || total_q == 0) return SAI_OK;
  if (!q_fp8 || !weights || !cu_q || !cu_k || !logits || logits_stride == 0) return SAI_EINVAL;
  if (total_k > 0 && (!k_fp8 || !k_scale)) return SAI_EINVAL;
  if (!aligned16(q_fp8) || !aligned16(weights) || (total_k > 0 && !aligned16(k_fp8))) return SAI_EINVAL;
  if (batch > 4096 || logits_stride > 0x7FFFFFFF - kChunk) return SAI_EUNSUPPORTED;
  const int64_t nchunks = (logits_stride + kChunk - 1) / kChunk;
  const int64_t ntiles = (total_q + kPfTileRows - 1) / kPfTileRows + batch;
  const int64_t G = 8 * ((ntiles + 7) / 8) * nchunks;
  if (G > 0x7FFFFFFF) return SAI_EUNSUPPORTED;
  // prefix of query tiles [batch+1] + the block scan's scratch [waves+1]
  const size_t lds = (size_t)((batch + 1) + kPfWaves + 1) * sizeof(int);
  launch(prefill_logits_kernel, dim3((unsigned)G), dim3(kPfThreads), lds, stream,
         (const uint8_t*)q_fp8, weights, (const uint8_t*)k_fp8, k_scale, cu_q, cu_k, batch,
         total_k, logits, logits_stride, row_len_out, row_req_out, (int32_t)nchunks,
         (int32_t)ntiles, logits_stride % 4 == 0 && aligned16(logits));
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
