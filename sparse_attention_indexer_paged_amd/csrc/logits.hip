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

#include "indexer_internal.h"
#include "score_mfma.h"

using namespace sai;
using namespace sai::score;

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


// The per-lane share of one 64-key block: 4 key tiles x 32 operand bytes,
// plus the scale of key `lane`.
struct KFrag {
  uint4 v[8];
  float s;
};

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

// ------------------------------------------------------------------ decode
// Scores NS consecutive key blocks of one request (block ids in lanes
// 0..NS-1 of myblk) for its NN query rows and writes the masked logits of
// block i, row r to st[(r * slots + i) * 64 + lane] in LDS.  NS is a
// compile-time count, so the ring below is straight-line code: every slot
// issues the same loads on every path (an invalid block id re-reads one
// 16-byte word of q instead), which lets the in-order vmcnt accounting
// leave the DEPTH-1 prefetched blocks in flight while one is scored.  No
// global store sits in the loop, so no K load ever queues behind one.
// With HIST every visible logit of row r also counts into bin (order key >>
// 22) of the wave's LDS histogram hist[r * kHistBins ..] (an LDS atomic).
template <int NN, int DEPTH, int NS, bool HIST>
__device__ __forceinline__ void score_group(const uint8_t* __restrict__ cache, int64_t num_blocks,
                                            const uint8_t* __restrict__ dummy, int myblk,
                                            const v8i (&qa)[NN][4], const float4 (&wf)[NN][4], int c0,
                                            int ctx, float* st, int slots, int* hist) {
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
      const bool vis = col < ctx - NN + r + 1;
      st[(r * slots + i) * kBlock + lane] = select_f(vis, v, kNegInfBits);
      if constexpr (HIST) {
        if (vis) atomicAdd(&hist[r * kHistBins + (f32_order_key(v) >> (32 - kHistBits))], 1);
      }
    }
  }
}

// Calls score_group with NS == n (1 <= n <= NS; n is wave-uniform).
template <int NN, int DEPTH, int NS, bool HIST>
__device__ __forceinline__ void dispatch_group(int n, const uint8_t* __restrict__ cache, int64_t num_blocks,
                                               const uint8_t* __restrict__ dummy, int myblk,
                                               const v8i (&qa)[NN][4], const float4 (&wf)[NN][4], int c0,
                                               int ctx, float* st, int slots, int* hist) {
  if (n == NS || NS == 1) {
    score_group<NN, DEPTH, NS, HIST>(cache, num_blocks, dummy, myblk, qa, wf, c0, ctx, st, slots, hist);
  } else if constexpr (NS > 1) {
    dispatch_group<NN, DEPTH, NS - 1, HIST>(n, cache, num_blocks, dummy, myblk, qa, wf, c0, ctx, st, slots,
                                            hist);
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
//
// With HIST each wave also counts its visible logits per row into an LDS
// histogram of the top kHistBits order-key bits and adds it to the row's
// histogram in `hist` ([rows][kHistBins], device atomics) when it moves to
// another request and at its end: the counts the top-k's first phase needs,
// with no global operation inside the K loop.
template <int NN, int DEPTH, int CAP, bool NT, bool HIST>
__global__ __launch_bounds__(256) void paged_logits_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ wts, const uint8_t* __restrict__ cache,
    int64_t num_blocks, const int32_t* __restrict__ bt, int64_t bt_stride,
    const int32_t* __restrict__ ctx_lens, int32_t batch, float* __restrict__ logits,
    int64_t stride, int32_t* __restrict__ row_len_out, int32_t* __restrict__ row_req_out, bool vec,
    bool clean, int32_t* __restrict__ hist) {
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
  int* s_hist = s_tot + 8 + wid * NN * kHistBins;  // [NN][kHistBins] this wave's histograms (HIST)
  if constexpr (HIST) {
#pragma unroll
    for (int i = 0; i < NN * kHistBins / 256; ++i)
      reinterpret_cast<int4*>(s_hist)[i * 64 + lane] = make_int4(0, 0, 0, 0);
  }
  // adds this wave's histograms of request hb to `hist` and clears them
  auto flush_hist = [&](int hb) {
#pragma unroll
    for (int r = 0; r < NN; ++r) {
      int* gh = hist + ((int64_t)hb * NN + r) * kHistBins;
#pragma unroll
      for (int i = 0; i < kHistBins / 256; ++i) {
        const int j = (i * 64 + lane) * 4;
        const int4 h = *reinterpret_cast<const int4*>(s_hist + r * kHistBins + j);
        if (h.x) __hip_atomic_fetch_add(gh + j, h.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (h.y) __hip_atomic_fetch_add(gh + j + 1, h.y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (h.z) __hip_atomic_fetch_add(gh + j + 2, h.z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (h.w) __hip_atomic_fetch_add(gh + j + 3, h.w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *reinterpret_cast<int4*>(s_hist + r * kHistBins + j) = make_int4(0, 0, 0, 0);
      }
    }
  };

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
      if constexpr (HIST) {
        if (qb >= 0) flush_hist(qb);
      }
      qb = b;
#pragma unroll
      for (int r = 0; r < NN; ++r) {
        load_qfrag(qa[r], q + ((int64_t)qb * NN + r) * (kHeads * kDim));
        load_wfrag(wf[r], wts + ((int64_t)qb * NN + r) * kHeads);
      }
    }
    dispatch_group<NN, DEPTH, kCap, HIST>(n, cache, num_blocks, q, myblk, qa, wf, c0, s_ctx[b],
                                          stage + (u - sa) * kBlock, kSlots, s_hist);
    u += n;
  }
  if (sa < u1) flush(sa, u1, bs);
  if constexpr (HIST) {
    if (qb >= 0) flush_hist(qb);
  }
}

template <int NN>
int launch_paged(const void* q, const float* w, const void* cache, int64_t num_blocks,
                 const int32_t* bt, int64_t bt_stride, const int32_t* ctx, int32_t batch,
                 float* logits, int64_t stride, int32_t* rl, int32_t* rr, bool clean, int32_t* hist,
                 hipStream_t s) {
  if (batch > 4096) return SAI_EUNSUPPORTED;  // LDS prefix arrays
  const int64_t wblocks = (stride + kBlock - 1) / kBlock;
  const int64_t units_max = (int64_t)batch * wblocks;
  const int64_t waves = std::min<int64_t>(kDecodeWaves, std::max<int64_t>(units_max, 1));
  int64_t G = (waves + 3) / 4;
  G = (G + 7) / 8 * 8;
  const size_t lds = 4 * kStageFloats * sizeof(float) + (size_t)(3 * (batch + 1) + 8) * sizeof(int) +
                     (hist ? (size_t)4 * NN * kHistBins * sizeof(int) : 0);
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
  const bool plain = (int64_t)batch * NN * stride * (int64_t)sizeof(float) <= kPlainStoreMaxBytes;
#define SAI_PAGED_LAUNCH(NT_, HIST_)                                                                  \
  launch((paged_logits_kernel<NN, kDecodeDepth, kDecodeCap, NT_, HIST_>), dim3((unsigned)G), dim3(256), lds, \
         s, (const uint8_t*)q, w, (const uint8_t*)cache, num_blocks, bt, bt_stride, ctx, batch, logits,   \
         stride, rl, rr, vec, clean, hist)
  if (hist) {
    if (plain) SAI_PAGED_LAUNCH(false, true); else SAI_PAGED_LAUNCH(true, true);
  } else {
    if (plain) SAI_PAGED_LAUNCH(false, false); else SAI_PAGED_LAUNCH(true, false);
  }
#undef SAI_PAGED_LAUNCH
  return hipGetLastError() == hipSuccess ? SAI_OK : SAI_ELAUNCH;
}

}  // namespace


// The paged logits call behind paged_mqa_logits, paged_mqa_logits_visible
// and the fused top-k entry (hist: the per-row histograms, or null).
int sai_paged_logits(const void* q_fp8, const float* weights, const void* kv_cache, int64_t num_blocks,
                     const int32_t* block_table, int64_t bt_stride, const int32_t* context_lens,
                     int32_t batch, int32_t next_n, float* logits, int64_t logits_stride,
                     int32_t* row_len_out, int32_t* row_req_out, bool clean, int32_t* hist,
                     hipStream_t stream) {
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
    case 1: return launch_paged<1>(q_fp8, weights, kv_cache, num_blocks, block_table, bt_stride, context_lens, batch, logits, logits_stride, row_len_out, row_req_out, clean, hist, stream);
    case 2: return launch_paged<2>(q_fp8, weights, kv_cache, num_blocks, block_table, bt_stride, context_lens, batch, logits, logits_stride, row_len_out, row_req_out, clean, hist, stream);
    case 3: return launch_paged<3>(q_fp8, weights, kv_cache, num_blocks, block_table, bt_stride, context_lens, batch, logits, logits_stride, row_len_out, row_req_out, clean, hist, stream);
    default: return launch_paged<4>(q_fp8, weights, kv_cache, num_blocks, block_table, bt_stride, context_lens, batch, logits, logits_stride, row_len_out, row_req_out, clean, hist, stream);
  }
}

extern "C" int paged_mqa_logits(const void* q_fp8, const float* weights, const void* kv_cache,
                                int64_t num_blocks, const int32_t* block_table, int64_t bt_stride,
                                const int32_t* context_lens, int32_t batch, int32_t next_n,
                                float* logits, int64_t logits_stride, int32_t* row_len_out,
                                int32_t* row_req_out, hipStream_t stream) {
  return sai_paged_logits(q_fp8, weights, kv_cache, num_blocks, block_table, bt_stride, context_lens, batch,
                          next_n, logits, logits_stride, row_len_out, row_req_out, true, nullptr, stream);
}

extern "C" int paged_mqa_logits_visible(const void* q_fp8, const float* weights, const void* kv_cache,
                                        int64_t num_blocks, const int32_t* block_table,
                                        int64_t bt_stride, const int32_t* context_lens, int32_t batch,
                                        int32_t next_n, float* logits, int64_t logits_stride,
                                        int32_t* row_len_out, int32_t* row_req_out, hipStream_t stream) {
  return sai_paged_logits(q_fp8, weights, kv_cache, num_blocks, block_table, bt_stride, context_lens, batch,
                          next_n, logits, logits_stride, row_len_out, row_req_out, false, nullptr, stream);
}
