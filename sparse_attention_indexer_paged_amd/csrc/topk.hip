// Per-row top-k of the indexer logits (ROCm/ATOM PR #1094, Technical
// Details: the sparse top-k over each query's request-local keys, handed on
// in a 2-D [rows, k] index buffer).
//
// Selection is exact, on 32-bit order-preserving keys (f32_order_key:
// larger logit -> larger key, -0.0 folded onto +0.0): find the k-th largest
// key T, the count of keys above it, and need = k - that count of the keys
// equal to T to take, lowest indices first.  The output pass walks the row
// in ascending index order; a workgroup scan of per-thread (above-T,
// equal-to-T) counts gives every winner its output slot, so indices come
// out sorted with no sort.  Rows whose visible length is at most k skip all
// of this and emit 0..n-1.
//
// topk_select_kernel (rows up to 16384 columns, and the segments and merge
// of wider rows) keeps each thread's keys in registers from the single read
// to the output and finds T from a sample, a histogram over the sampled
// value range and a brute-force rank of the few keys in the threshold bin,
// with an exact radix select as the fallback.  On the 1024-thread shapes
// the keys at or above the sample's bound (about 1.3 k of the row) are
// first compacted into LDS in position order, so the later phases handle 4
// keys per thread instead of 8-16.  topk_wide_kernel takes rows of up to
// 65536 columns whole when the launch has few rows (one workgroup per row,
// no candidate round trip).  Rows too wide for the segment-and-merge plan
// take topk_row_kernel, which streams the row from L2 for each of three
// radix rounds (11, 11, 10 key bits).
#include <atomic>
#include <type_traits>

#include "indexer_internal.h"

using namespace sai;

namespace {

constexpr int kThreads = 1024;
constexpr int kBins = 2048;

template <bool VEC>
__device__ __forceinline__ void load4(const float* __restrict__ x, int i, int n, float (&v)[4]) {
  if (VEC && i + 3 < n) {
    const float4 f = *reinterpret_cast<const float4*>(x + i);
    v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (i + e < n) ? x[i + e] : 0.0f;
  }
}

// Exact top-k of one row of n > k columns read from memory, by NT
// threads: three radix rounds over the row (11, 11, 10 key bits), each
// re-reading it, then an ordered output pass that hands every winner's
// output slot and column to emit(j, i).  LDS: hist holds kBins ints, scan
// NT/64 + 1, sel 6.  VEC: rows are 16-byte aligned, so 4 consecutive
// columns load as one float4.
template <int NT, bool VEC, class Emit>
__device__ __forceinline__ void stream_select(const float* __restrict__ x, int n, int k, int* hist,
                                              int* scan, uint32_t (*sel)[2], Emit emit) {
  static_assert(2 * NT >= kBins, "two bins per thread cover the histogram");
  const int tid = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  int need = k;  // winners still to place among keys matching the prefix
  const int shifts[3] = {21, 10, 0};
  const uint32_t dmask[3] = {0x7FFu, 0x7FFu, 0x3FFu};
  for (int round = 0; round < 3; ++round) {
    const int sh = shifts[round];
    const uint32_t dm = dmask[round];
    const int nb = (int)dm + 1;
    for (int i = tid; i < kBins; i += NT) hist[i] = 0;
    if (tid == 0) sel[round][0] = sel[round][1] = 0;
    __syncthreads();
    for (int i = tid * 4; i < n; i += NT * 4) {
      float v[4];
      load4<VEC>(x, i, n, v);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (i + e < n) {
          const uint32_t key = f32_order_key(v[e]);
          if ((key & pmask) == prefix) atomicAdd(&hist[(key >> sh) & dm], 1);
        }
      }
    }
    __syncthreads();
    // thread t owns bins nb-1-2t and nb-2-2t (descending), scanned in thread order
    const int bhi = nb - 1 - 2 * tid, blo = nb - 2 - 2 * tid;
    const int hhi = bhi >= 0 ? hist[bhi] : 0;
    const int hlo = blo >= 0 ? hist[blo] : 0;
    int total;
    const int before = block_exclusive_scan<NT>(hhi + hlo, scan, &total);
    if (bhi >= 0 && before < need && need <= before + hhi) {
      sel[round][0] = (uint32_t)bhi;
      sel[round][1] = (uint32_t)before;
    } else if (blo >= 0 && before + hhi < need && need <= before + hhi + hlo) {
      sel[round][0] = (uint32_t)blo;
      sel[round][1] = (uint32_t)(before + hhi);
    }
    __syncthreads();
    prefix |= sel[round][0] << sh;
    pmask |= dm << sh;
    need -= (int)sel[round][1];
  }
  const uint32_t T = prefix;

  // ordered output: tiles of NT*4 columns, thread t owns 4 consecutive
  int gt_run = 0, eq_run = 0;
  for (int base = 0; base < n; base += NT * 4) {
    const int i = base + tid * 4;
    float v[4];
    load4<VEC>(x, i, n, v);
    uint32_t key[4];
    int ngt = 0, neq = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      key[e] = f32_order_key(v[e]);
      const bool in = i + e < n;
      ngt += (in && key[e] > T);
      neq += (in && key[e] == T);
    }
    int tot;
    const int ex = block_exclusive_scan<NT>(ngt | (neq << 16), scan, &tot);
    int gt_b = gt_run + (ex & 0xFFFF), eq_b = eq_run + (ex >> 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (i + e >= n) break;
      if (key[e] > T) {
        const int pos = gt_b + min(eq_b, need);
        if ((unsigned)pos < (unsigned)k) emit(pos, i + e);
        ++gt_b;
      } else if (key[e] == T) {
        const int pos = gt_b + eq_b;
        if (eq_b < need && (unsigned)pos < (unsigned)k) emit(pos, i + e);
        ++eq_b;
      }
    }
    gt_run += tot & 0xFFFF;
    eq_run += tot >> 16;
  }
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void topk_row_kernel(
    const float* __restrict__ logits, int64_t stride, const int32_t* __restrict__ row_len,
    int32_t k, int32_t* __restrict__ out) {
  __shared__ int s_hist[kBins];
  __shared__ int s_scan[kThreads / 64 + 1];
  __shared__ uint32_t s_sel[3][2];  // per round: chosen bin, count above it

  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  int32_t* o = out + (int64_t)r * k;
  const int n = (int)min((int64_t)max(row_len[r], 0), stride);
  if (n <= k) {
    for (int j = tid; j < k; j += kThreads) o[j] = j < n ? j : -1;
    return;
  }
  stream_select<kThreads, VEC>(logits + (int64_t)r * stride, n, k, s_hist, s_scan, s_sel,
                               [&](int j, int32_t i) { o[j] = i; });
}

// Inclusive wave64 prefix sum on DPP: shifts of 1, 2, 4, 8 within each row of
// 16 lanes, then row 0/2 totals broadcast into rows 1/3 (row_bcast:15) and
// the row-1 total into rows 2/3 (row_bcast:31).  Lanes without a source keep
// the 0 passed as `old`.
__device__ __forceinline__ int wave_scan_dpp(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Wave64 maximum of unsigned values, in lane 63 (same DPP pattern as
// wave_scan_dpp, with 0 as the identity).
__device__ __forceinline__ uint32_t wave_max_dpp(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));
  return v;
}

#ifndef SAI_TOPK_MANY_WGS
#define SAI_TOPK_MANY_WGS 512
#endif
constexpr int kSegCols = 16384;              // columns per segment of a wide row
constexpr int kWideCols = 65536;             // widest row one workgroup takes whole
constexpr int kManyWgs = SAI_TOPK_MANY_WGS;  // from this many workgroups on, use small ones
constexpr int kCandMax = 64;               // threshold-bin keys resolved by brute force
constexpr int kCompCap = 4096;             // keys at or above the sampled bound kept in LDS
// Launches of at most this many workgroups are latency-bound: their rows'
// loads go out before the row lengths are known (a few wasted reads of rows
// that need no selection are cheaper than the extra round trip).
constexpr unsigned kEarlyLoadWgs = 1024;

struct BinPick {
  int bin, above;
  bool found;
};

// Every lane of the calling wave gets the bin of hist[0..NB) that holds the
// need-th largest element when bins are taken from the top down, and the
// count above that bin; found is false if the histogram holds fewer than
// need (with clamp_to_total, need is first lowered to the total).  Lane l
// owns the PER = NB/64 bins [NB-PER(l+1), NB-PER*l), read with 16-byte LDS
// loads; a DPP scan of the lane sums in lane order (descending bins) finds
// the lane holding the need-th element, which walks its bins downwards; the
// result is broadcast from that lane.
// ROLLED: the walk is a loop over groups of 4 bins (fewer registers, for
// callers that hold many values in registers across the pick).
template <int NB, bool ROLLED = false>
__device__ __forceinline__ BinPick pick_bin(const int* hist, int need, bool clamp_to_total = false) {
  constexpr int PER = NB / 64;
  const int lane = threadIdx.x & 63;
  const int lo = NB - PER * (lane + 1);
  // two passes over the lane's bins, 4 at a time, so the bins never occupy
  // PER registers at once: the sum, then the walk
  int sum = 0;
#pragma unroll
  for (int j = 0; j < PER; j += 4) {
    const int4 v = *reinterpret_cast<const int4*>(hist + lo + j);
    sum += v.x + v.y + v.z + v.w;
  }
  const int inc = wave_scan_dpp(sum);
  if (clamp_to_total) need = min(need, __builtin_amdgcn_readlane(inc, 63));
  const int acc = inc - sum;
  const bool hit = acc < need && need <= inc;
  // branch-free walk from the lane's top bin down: the bins whose running
  // total stays below need are the ones above the chosen bin
  int run = 0, nbelow = 0, sum_above = 0;
#pragma unroll(ROLLED ? 1 : PER / 4)
  for (int j = PER - 4; j >= 0; j -= 4) {
    const int4 v = *reinterpret_cast<const int4*>(hist + lo + j);
    const int h4[4] = {v.w, v.z, v.y, v.x};  // bins lo+j+3 .. lo+j
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      run += h4[q];
      const bool short_of = acc + run < need;
      nbelow += short_of;
      sum_above += short_of ? h4[q] : 0;
    }
  }
  const int bin = lo + PER - 1 - nbelow, above = acc + sum_above;
  const uint64_t m = __ballot(hit);
  if (m == 0) return {0, 0, false};
  const int src = (int)__builtin_ctzll(m);
  return {__builtin_amdgcn_readlane(bin, src), __builtin_amdgcn_readlane(above, src), true};
}

// The float whose order key is k (the inverse of f32_order_key; -0 comes
// back as +0).
__device__ __forceinline__ float order_key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Selection key: the order key of the logit, never 0 (0 marks a position
// that is not part of the row: past its length, or an unused candidate
// slot).
__device__ __forceinline__ uint32_t sel_key(float v) {
  const uint32_t k = f32_order_key(v);
  return k ? k : 1u;
}

// Optional fused slot map: with out != nullptr every final index i of row r
// is also written as its global paged-cache slot,
// bt[row_req[r] * bt_stride + i / 64] * 64 + i % 64, or -1 (for i = -1, a
// request outside [0, batch), a block past bt_stride or a negative entry).
struct SlotMap {
  const int32_t* row_req;
  const int32_t* bt;
  int64_t bt_stride;
  int32_t batch;
  int32_t* out;
};

// Block-table rows of up to kBtLds entries are staged in LDS (dynamic
// shared memory) at the start of the kernel, so the slot of every output
// index is one LDS read instead of a dependent global load at the end.
constexpr int kBtLds = 4096;

__device__ __forceinline__ int32_t slot_of(const SlotMap& sm, int32_t b, int32_t i) {
  if (i < 0 || b < 0 || b >= sm.batch || (int64_t)(i / 64) >= sm.bt_stride) return -1;
  const int32_t blk = sm.bt[(int64_t)b * sm.bt_stride + i / 64];
  return blk >= 0 ? blk * 64 + i % 64 : -1;
}

// Register-resident exact top-k of one row (or one segment of a row, or
// one row's candidate list): thread t keeps the keys of positions
// [t*VPT, (t+1)*VPT) in registers from the single read to the output.
//
//   CIN  = false: positions are the columns of a logits row (segment);
//          true:  positions are a candidate list (key, column) of nseg*k
//                 slots per row, written by the segment pass.
//   COUT = false: write the winners' columns, ascending, to out_idx[r, k];
//          true:  write the segment's winners (key, column), ascending, to
//                 its k-slot candidate list; unused slots get (0, -1).
//
// Finding the k-th largest key T:
//  1. A sample of one key per thread gives, through a 2048-bin histogram of
//     the top 11 key bits, a lower bound key_lo on T with a 30% margin, and
//     the largest sampled key key_hi.
//  2. Keys >= key_lo are counted in 2048 bins (1024 in many-row launches)
//     spread linearly over [key_lo, key_hi] (keys above key_hi go to the
//     top bin); the bin holding the k-th largest key typically holds a
//     few keys.
//     (With kComp the keys >= key_lo are compacted into LDS first and this
//     and the following phases run on them.)
//  3. Those keys (at most kCandMax) are copied to LDS and every wave ranks
//     them by brute force in registers, which gives T exactly.
// If the bound was too high or the bin too full (heavy ties, odd
// distributions), an exact 3-round radix select over all keys (11, 11, 10
// bits) runs instead, so the result is exact either way.
//
// Output: a workgroup scan of per-thread (above T, equal to T) counts gives
// every winner its slot (the `need` lowest-index keys equal to T win), so
// the winners come out in ascending position order; they are staged in LDS
// and written with coalesced stores.
//
// HIST (one-pass rows with early loads only): the row's histogram of the top
// kHistBits order-key bits over its visible columns, counted by the paged
// logits kernel, is in hist[r * kHistBins ..].  It replaces the sample: the
// bin holding the k-th largest key gives key_lo exactly (with the count
// above it) and the linear bins of step 2 span that bin's value range.  The
// row's histogram is read once and set back to zero for the next call.  A
// wrong histogram costs speed, never exactness (the bound is checked like a
// sampled one).
//
// Launches of many workgroups (without EARLY) are throughput-bound: they ask
// the compiler for 8 waves per SIMD (at most 64 registers, so 2-8
// workgroups share a CU instead of 1-2), and their bin picks walk the bins
// in a loop, which needs far fewer registers than the unrolled walk.
template <int NT, int VPT, bool VEC, bool CIN, bool COUT, bool EARLY, bool HIST = false>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(EARLY ? 1 : 8))) void topk_select_kernel(
    const float* __restrict__ logits, int64_t stride, const int32_t* __restrict__ row_len,
    int32_t k, int32_t nseg, const uint32_t* __restrict__ c_key, const int32_t* __restrict__ c_col,
    int32_t* __restrict__ out_idx, uint32_t* __restrict__ o_key, int32_t* __restrict__ o_col,
    SlotMap sm, int32_t* __restrict__ hist) {
  constexpr int kWaves = NT / 64, SEG = VPT * NT;
  static_assert(!COUT || SEG == kSegCols, "a segment pass covers exactly one segment");
  static_assert(!HIST || (EARLY && !CIN && !COUT && NT >= kHistBins), "histograms: one-pass early rows");
  // Compaction (see below) on the 1024-thread shapes with at least 8 keys
  // per thread: CPER = 4 compacted keys per thread, kCompCap in all.  (On
  // the many-workgroup 512-thread shapes it measured even or slower: 8192
  // rows of <= 8192 even, segment passes of 256 rows x 4 segments 52 -> 64
  // us, its extra registers costing a wave per SIMD.)
  constexpr int CPER = kCompCap / NT;
  constexpr bool kComp = !CIN && NT == 1024 && VPT >= 2 * CPER;
  __shared__ __align__(16) int s_h0[kBins];
  __shared__ __align__(16) int s_h1[kBins];
  __shared__ uint32_t s_ck[kComp ? kCompCap : 1];  // compacted keys
  uint16_t* const s_cp = reinterpret_cast<uint16_t*>(s_h0);  // their positions (s_h0 is free then)
  static_assert(kCompCap * 2 <= kBins * 4, "positions fit the first histogram");
  __shared__ uint32_t s_cand[kCandMax];
  __shared__ int s_wsum[kWaves];
  __shared__ uint32_t s_misc[2];  // [0] threshold-bin keys, [1] largest sampled key
  __shared__ int s_pick[3];       // wave 0's pick_bin result: bin, above, found

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int r = COUT ? (int)(blockIdx.x / nseg) : (int)blockIdx.x;
  const int base = tid * VPT;
  // column of position 0 (rows and segments)
  const int64_t cbase = COUT ? (int64_t)(blockIdx.x - (unsigned)r * nseg) * SEG : 0;
  uint32_t key[VPT];
  int32_t col[CIN ? VPT : 1];
  float v[CIN ? 1 : VPT];
  // Every load is issued unconditionally from an address clamped into the
  // row (or, for the merge, into the row's candidate block), so all of a
  // thread's loads are in flight together and positions past the length are
  // masked afterwards.  With EARLY (few workgroups, so latency-bound) they
  // go out before the row length has arrived and are clamped to the stride;
  // otherwise after it, clamped to the length rounded up to 4 columns (a
  // causal prefill row then reads only its visible part: positions past it
  // re-read the row's last 16 bytes, a line already on its way), and rows
  // which need no selection (length <= k) skip them.  (A runtime choice
  // would join the two orders, and the wait-count pass drains all loads at
  // such a join.)  `lim` is the number of columns that may be read, >= 1,
  // a multiple of 4 for VEC.
  auto load_row = [&](int64_t lim) {
    if (CIN) {
      const int nc = nseg * k;
      const uint32_t* kp = c_key + (int64_t)r * nc;
      const int32_t* cp = c_col + (int64_t)r * nc;
  #pragma unroll
      for (int e = 0; e < VPT; e += 4) {
        if (VEC) {  // nc is a multiple of 4
          const int p = min(base + e, nc - 4);
          const uint4 kv = *reinterpret_cast<const uint4*>(kp + p);
          const int4 cv = *reinterpret_cast<const int4*>(cp + p);
          key[e] = kv.x; key[e + 1] = kv.y; key[e + 2] = kv.z; key[e + 3] = kv.w;
          col[e] = cv.x; col[e + 1] = cv.y; col[e + 2] = cv.z; col[e + 3] = cv.w;
        } else {
  #pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int p = min(base + e + i, nc - 1);
            key[e + i] = kp[p];
            col[e + i] = cp[p];
          }
        }
      }
    } else {
      const float* x0 = logits + (int64_t)r * stride;  // stride floats
  #pragma unroll
      for (int e = 0; e < VPT; e += 4) {
        if (VEC) {  // stride is a multiple of 4
          const int64_t p = min(cbase + base + e, lim - 4);
          const float4 f = *reinterpret_cast<const float4*>(x0 + p);
          v[e] = f.x; v[e + 1] = f.y; v[e + 2] = f.z; v[e + 3] = f.w;
        } else {
  #pragma unroll
          for (int i = 0; i < 4; ++i) v[e + i] = x0[min(cbase + base + e + i, lim - 1)];
        }
      }
    }
  };
  // the row's histogram goes out first: waiting for it then waits for no
  // other load (the wait counter retires loads in order)
  int32_t hval = 0;
  if constexpr (HIST) {
    if (tid < kHistBins) hval = hist[(int64_t)r * kHistBins + tid];
  }
  if constexpr (EARLY) load_row(stride);
  // read after the row's loads are issued: a scalar load ahead of them
  // would make their address computation wait for it
  const int len = (int)min((int64_t)max(row_len[r], 0), stride);
  const int32_t req = sm.out ? sm.row_req[r] : 0;
  extern __shared__ int32_t s_bt[];  // [bt_stride] when bt_lds
  const bool bt_lds = sm.out && sm.bt_stride <= kBtLds;
  // whether this workgroup writes final indices (see the early returns below)
  const bool emits = COUT ? (len > k && len <= kSegCols && blockIdx.x == (unsigned)r * nseg)
                          : (!CIN || len <= k || len > kSegCols);
  // The request's block-table row goes to LDS for the slot ids.  With EARLY
  // it is loaded into registers while the row's loads (above) are in flight
  // and stored just before the barrier ahead of the output, which publishes
  // it; otherwise it is staged right after the row's loads are issued.
  constexpr int kBtPer = EARLY ? (kBtLds + NT - 1) / NT : 1;
  int32_t btv[kBtPer];
  auto load_bt = [&]() {
    if (bt_lds && emits) {
      const bool okr = req >= 0 && req < sm.batch;
      const int32_t* rowp = sm.bt + (int64_t)(okr ? req : 0) * sm.bt_stride;
#pragma unroll
      for (int i = 0; i < kBtPer; ++i) {
        const int c = tid + i * NT;
        btv[i] = okr && c < (int)sm.bt_stride ? rowp[c] : -1;
      }
    }
  };
  auto store_bt = [&]() {
    if (bt_lds && emits) {
#pragma unroll
      for (int i = 0; i < kBtPer; ++i)
        if (tid + i * NT < (int)sm.bt_stride) s_bt[tid + i * NT] = btv[i];
    }
  };
  // without EARLY: load and store in one pass, right after the row's loads
  auto stage_bt = [&]() {
    if constexpr (EARLY) {
      load_bt();
      store_bt();
    } else if (bt_lds && emits) {
      const bool okr = req >= 0 && req < sm.batch;
      for (int c = tid; c < (int)sm.bt_stride; c += NT)
        s_bt[c] = okr ? sm.bt[(int64_t)req * sm.bt_stride + c] : -1;
    }
  };
  // Clears the histograms; done while the row's loads are in flight, so
  // this barrier overlaps their latency.
  auto clear_hist = [&]() {
    if constexpr (HIST) {  // the row's histogram to LDS (loaded first thing), zero for the next call
      if (tid < kHistBins) {
        s_h0[tid] = hval;
        hist[(int64_t)r * kHistBins + tid] = 0;
      }
      for (int i = tid; i < kBins; i += NT) s_h1[i] = 0;
    } else {
      for (int i = tid; i < kBins; i += NT) {
        s_h0[i] = 0;
        s_h1[i] = 0;
      }
    }
    if (tid < 2) s_misc[tid] = 0u;
    __syncthreads();
  };
  auto emit = [&](int j, int32_t i) {  // final index j of row r
    out_idx[(int64_t)r * k + j] = i;
    if (sm.out) {
      int32_t slot = -1;
      if (bt_lds) {
        if (i >= 0 && i / 64 < (int)sm.bt_stride) {
          const int32_t blk = s_bt[i / 64];
          slot = blk >= 0 ? blk * 64 + i % 64 : -1;
        }
      } else {
        slot = slot_of(sm, req, i);
      }
      sm.out[(int64_t)r * k + j] = slot;
    }
  };
  // A workgroup with no selection to do stops here: rows of at most k
  // columns (all win), and in the split plan the segments and merge of a
  // row that fits one segment (segment 0 finishes it).
  auto done_early = [&]() {
    if (len <= k) {
      if (!COUT) {
        stage_bt();
        __syncthreads();  // publishes s_bt
        for (int j = tid; j < k; j += NT) emit(j, j < len ? j : -1);
      }
      return true;
    }
    return (CIN && len <= kSegCols) || (COUT && len <= kSegCols && blockIdx.x != (unsigned)r * nseg);
  };
  if constexpr (!EARLY) {
    if (done_early()) return;
    // len > k >= 1 here; for VEC the stride is a multiple of 4
    load_row(VEC ? min(stride, ((int64_t)len + 3) & ~(int64_t)3) : (int64_t)len);
  }
  int n;  // positions of this workgroup
  if (CIN) {
    n = nseg * k;
  } else if (COUT) {
    n = (int)max(min((int64_t)len - cbase, (int64_t)SEG), (int64_t)0);
  } else {
    n = len;
  }
  // With early loads nothing that depends on the row length branches before
  // the keys are converted: a branch there would let the compiler sink the
  // loads below it, i.e. wait for the length before issuing them.
  if constexpr (EARLY) load_bt(); else stage_bt();
  clear_hist();
  if (CIN) {
#pragma unroll
    for (int e = 0; e < VPT; ++e)
      if (base + e >= n) {
        key[e] = 0u;
        col[e] = -1;
      }
  } else {
#pragma unroll
    for (int e = 0; e < VPT; ++e) key[e] = base + e < n ? sel_key(v[e]) : 0u;
  }
  if constexpr (EARLY) {
    if (done_early()) return;
  }
  const bool final_out = !COUT || len <= kSegCols;
  auto column = [&](int e) -> int32_t {
    if constexpr (CIN) return col[e];
    else return (int32_t)(cbase + base + e);
  };

  // pick_bin by wave 0, broadcast to the workgroup through LDS
  auto pick = [&](const int* h, int nd, auto nb_tag, bool clamp = false) {
    constexpr int NB = decltype(nb_tag)::value;
    if (wid == 0) {
      const BinPick p = pick_bin<NB, !EARLY>(h, nd, clamp);
      if (lane == 0) {
        s_pick[0] = p.bin;
        s_pick[1] = p.above;
        s_pick[2] = p.found;
      }
    }
    __syncthreads();
    return BinPick{s_pick[0], s_pick[1], s_pick[2] != 0};
  };
  using B11 = std::integral_constant<int, 2048>;
  using B10 = std::integral_constant<int, 1024>;

  if (COUT && !final_out && n <= k) {  // at most k columns: all are candidates
    uint32_t* ok = o_key + (int64_t)blockIdx.x * k;
    int32_t* oc = o_col + (int64_t)blockIdx.x * k;
#pragma unroll
    for (int e = 0; e < VPT; ++e)
      if (base + e < n) {
        ok[base + e] = key[e];
        oc[base + e] = column(e);
      }
    for (int j = n + tid; j < k; j += NT) {
      ok[j] = 0u;
      oc[j] = -1;
    }
    return;
  }

  // 1. the lower bound key_lo and the top of the value range of step 2:
  // from the row's histogram (HIST), else from a sample (the histograms
  // were cleared while the row was loading)
  uint32_t lo_digit, key_lo, key_top;  // lo_digit: key_lo's top 11 bits
  if constexpr (HIST) {
    const BinPick ph = pick(s_h0, k, std::integral_constant<int, kHistBins>{});
    // no bin holds the k-th key (a wrong histogram): key_lo above every key,
    // so the bound fails and the radix select runs unpruned
    lo_digit = ph.found ? (uint32_t)ph.bin << (kHistBits == 10 ? 1 : 0) : 0u;
    key_lo = ph.found ? (uint32_t)ph.bin << (32 - kHistBits) : 0xFFFFFFFFu;
    key_top = ph.found ? key_lo + ((1u << (32 - kHistBits)) - 1u) : 0xFFFFFFFFu;
  } else {
    if (key[0] != 0u) atomicAdd(&s_h0[key[0] >> 21], 1);
    const uint32_t wmax = wave_max_dpp(key[0]);
    if (lane == 63) atomicMax(&s_misc[1], wmax);
    __syncthreads();
    const int S = (n + VPT - 1) / VPT;
    // k*S*13 < 2^25 and n*10 < 2^19: 32-bit arithmetic
    const int m = min(S, (int)(((uint32_t)k * S * 13u + (uint32_t)n * 10u - 1u) / ((uint32_t)n * 10u)) + 8);
    const BinPick ps = pick(s_h0, m, B11{}, true);
    lo_digit = (uint32_t)ps.bin;
    key_lo = lo_digit << 21;
    key_top = max(s_misc[1], key_lo);
  }
  const float v_lo = order_key_value(key_lo);
  const float range = order_key_value(key_top) - v_lo;
  // linear bins: 2048 in few-row launches, 1024 in many-row ones (a
  // shorter pick; 8192-token prefill top-k 91.4 -> 89.8 us, chunked
  // prefill 176.9 -> 173.9 us; on the long-context merges fewer bins were
  // slower)
  constexpr int kLin = EARLY ? kBins : kBins / 2;
  const float scale = (float)kLin / range;
  auto fbin = [&](uint32_t kk) {
    return (int)fminf((order_key_value(kk) - v_lo) * scale, (float)(kLin - 1));
  };

  // 2. linear bins over the logit values [v_lo, v_hi] (a finite, non-empty
  // range: anything else goes straight to the radix select)
  bool fast = isfinite(v_lo) && isfinite(range) && range > 0.0f && isfinite(scale);

  // 2a. Only keys >= key_lo can win while the bound holds, about 1.3 k of the
  // row.  With kComp they are compacted, in ascending position order, into
  // LDS (keys in s_ck, positions in s_cp), and the histogram, candidate and
  // output phases run on each thread's CPER compacted keys instead of its
  // VPT register keys.  The register keys stay live for the radix
  // fallback, which then also writes the output.
  bool comp = false;
  uint32_t ckey[kComp ? CPER : 1];
  int32_t ccol[kComp ? CPER : 1];
  if constexpr (kComp) {
    if (fast) {
      int cnt = 0;
#pragma unroll
      for (int e = 0; e < VPT; ++e) cnt += (key[e] != 0u && key[e] >= key_lo);
      const int incl = wave_scan_dpp(cnt);
      if (lane == 63) s_wsum[wid] = incl;
      __syncthreads();
      int off = incl - cnt, total = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const int sw = s_wsum[w];
        off += w < wid ? sw : 0;
        total += sw;
      }
      comp = total >= k && total <= kCompCap;
      if (comp) {
#pragma unroll
        for (int e = 0; e < VPT; ++e) {
          if (key[e] != 0u && key[e] >= key_lo) {
            s_ck[off] = key[e];
            s_cp[off] = (uint16_t)(base + e);
            ++off;
          }
        }
      }
      __syncthreads();  // the compacted list; every wave has read s_wsum
      if (comp) {
#pragma unroll
        for (int j = 0; j < CPER; ++j) {
          const int i = tid * CPER + j;
          ckey[j] = i < total ? s_ck[i] : 0u;
          ccol[j] = i < total ? (int32_t)(cbase + s_cp[i]) : -1;
        }
      }
    }
  }
  BinPick p1 = {0, 0, false};
  if (fast) {
    if (comp) {
#pragma unroll
      for (int j = 0; j < (kComp ? CPER : 1); ++j)
        if (ckey[j] != 0u) atomicAdd(&s_h1[fbin(ckey[j])], 1);
    } else {
#pragma unroll
      for (int e = 0; e < VPT; ++e)
        if (key[e] != 0u && key[e] >= key_lo) atomicAdd(&s_h1[fbin(key[e])], 1);
    }
    __syncthreads();
    p1 = pick(s_h1, k, std::integral_constant<int, kLin>{});
    fast = p1.found;
  }
  if (fast) {
    if (comp) {
#pragma unroll
      for (int j = 0; j < (kComp ? CPER : 1); ++j) {
        if (ckey[j] != 0u && fbin(ckey[j]) == p1.bin) {
          const uint32_t sl = atomicAdd(&s_misc[0], 1u);
          if (sl < (uint32_t)kCandMax) s_cand[sl] = ckey[j];
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < VPT; ++e) {
        if (key[e] != 0u && key[e] >= key_lo && fbin(key[e]) == p1.bin) {
          const uint32_t sl = atomicAdd(&s_misc[0], 1u);
          if (sl < (uint32_t)kCandMax) s_cand[sl] = key[e];
        }
      }
    }
    __syncthreads();
    fast = s_misc[0] <= (uint32_t)kCandMax;
  }

  uint32_t T = 0;
  int need = 0;  // keys equal to T that win (lowest positions first)
  if (fast) {
    // 3. rank the threshold bin's keys: T is the need1-th largest of them
    // (every wave computes the same from the same LDS contents)
    const int nc = (int)s_misc[0];
    const int need1 = k - p1.above;
    const uint32_t c = lane < nc ? s_cand[lane] : 0u;
    int gt = 0, ge = 0;
    for (int j = 0; j < nc; ++j) {
      const uint32_t cj = __builtin_amdgcn_readlane(c, j);
      gt += cj > c;
      ge += cj >= c;
    }
    const uint64_t hm = __ballot(lane < nc && gt < need1 && need1 <= ge);
    if (hm != 0) {
      const int src = (int)__builtin_ctzll(hm);
      T = __builtin_amdgcn_readlane(c, src);
      need = need1 - __builtin_amdgcn_readlane(gt, src);
    } else {
      fast = false;
    }
  }
  if (!fast) {
    // exact radix select; the first digit counts only digits >= lo_digit
    // unless that holds fewer than k keys
    uint32_t prefix = 0, pmask = 0;
    int nd = k;
    auto round = [&](int* h, int shift, uint32_t dm, uint32_t min_digit, auto nb_tag) {
      for (int i = tid; i < kBins; i += NT) h[i] = 0;
      __syncthreads();
#pragma unroll
      for (int e = 0; e < VPT; ++e) {
        const uint32_t d = (key[e] >> shift) & dm;
        if (key[e] != 0u && (key[e] & pmask) == prefix && d >= min_digit) atomicAdd(&h[d], 1);
      }
      __syncthreads();
      const BinPick p = pick(h, nd, nb_tag);
      if (p.found) {
        prefix |= (uint32_t)p.bin << shift;
        pmask |= dm << shift;
        nd -= p.above;
      }
      return p.found;
    };
    // every wave is done reading both histograms; from here consecutive
    // rounds alternate buffers, so a clear never overlaps a slower wave's
    // pick of the round before
    __syncthreads();
    int* hb = s_h0;
    auto flip = [&]() { hb = hb == s_h0 ? s_h1 : s_h0; };
    const bool pruned = round(hb, 21, 0x7FFu, lo_digit, B11{});
    flip();
    if (!pruned) {
      round(hb, 21, 0x7FFu, 0u, B11{});
      flip();
    }
    round(hb, 10, 0x7FFu, 0u, B11{});
    flip();
    round(hb, 0, 0x3FFu, 0u, B10{});
    T = prefix;
    need = nd;
    comp = false;  // the output comes from the register keys
  }

  // ordered output; counts packed as (equal << 12) | above (above-T totals
  // stay below k <= 2048, equal totals below 2^19).  The keys are the
  // register keys (thread t holds positions [t*VPT, (t+1)*VPT)) or, with
  // comp, the compacted list (thread t holds its ascending slice): either
  // way thread order is position order.
  int ngt = 0, neq = 0;
  if (comp) {
#pragma unroll
    for (int j = 0; j < (kComp ? CPER : 1); ++j) {
      const bool in = ckey[j] != 0u;
      ngt += (in && ckey[j] > T);
      neq += (in && ckey[j] == T);
    }
  } else {
#pragma unroll
    for (int e = 0; e < VPT; ++e) {
      const bool in = key[e] != 0u;
      ngt += (in && key[e] > T);
      neq += (in && key[e] == T);
    }
  }
  const int packed = ngt | (neq << 12);
  const int inc = wave_scan_dpp(packed);
  if (lane == 63) s_wsum[wid] = inc;
  // One-pass rows of the few-row launches write each winner's index and slot
  // id from the thread that holds it (its output position is known once the
  // counts are scanned), so the block-table row goes out with the counts.
  // Many-row launches (whose outputs are large: scattered writes cost more
  // than the barrier) and segment and merge passes stage their output in
  // LDS and write it coalesced.
  constexpr bool kDirect = EARLY && !CIN && !COUT;
  if constexpr (kDirect) store_bt();
  __syncthreads();
  int ex = inc - packed;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) ex += w < wid ? s_wsum[w] : 0;
  int gt_b = ex & 0xFFF, eq_b = ex >> 12;
  int tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) tot += s_wsum[w];
  const int nwin = min(k, (tot & 0xFFF) + min(tot >> 12, need));  // k unless the row is short
  if (comp) {
#pragma unroll
    for (int j = 0; j < (kComp ? CPER : 1); ++j) {
      if (ckey[j] != 0u) {
        int pos = -1;
        if (ckey[j] > T) {
          pos = gt_b + min(eq_b, need);
          ++gt_b;
        } else if (ckey[j] == T) {
          if (eq_b < need) pos = gt_b + eq_b;
          ++eq_b;
        }
        if ((unsigned)pos < (unsigned)k) {
          if constexpr (kDirect) {
            emit(pos, ccol[j]);
          } else {
            s_h0[pos] = ccol[j];
            if (COUT) s_h1[pos] = (int)ckey[j];
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < VPT; ++e) {
      if (key[e] != 0u) {
        int pos = -1;
        if (key[e] > T) {
          pos = gt_b + min(eq_b, need);
          ++gt_b;
        } else if (key[e] == T) {
          if (eq_b < need) pos = gt_b + eq_b;
          ++eq_b;
        }
        if ((unsigned)pos < (unsigned)k) {
          if constexpr (kDirect) {
            emit(pos, column(e));
          } else {
            s_h0[pos] = column(e);
            if (COUT) s_h1[pos] = (int)key[e];
          }
        }
      }
    }
  }
  if constexpr (kDirect) {
    // past nwin (a row with fewer than k keys) the indices are -1
    for (int j = nwin + tid; j < k; j += NT) emit(j, -1);
    return;
  }
  if constexpr (EARLY) store_bt();
  __syncthreads();
  if (COUT && !final_out) {
    uint32_t* ok = o_key + (int64_t)blockIdx.x * k;
    int32_t* oc = o_col + (int64_t)blockIdx.x * k;
    for (int j = tid; j < k; j += NT) {
      ok[j] = j < nwin ? (uint32_t)s_h1[j] : 0u;
      oc[j] = j < nwin ? s_h0[j] : -1;
    }
  } else {
    for (int j = tid; j < k; j += NT) emit(j, j < nwin ? s_h0[j] : -1);
  }
}

// One-pass selection of rows wider than one segment (up to kWideCols
// columns) in launches of few rows: one 1024-thread workgroup per row, the
// row held in registers once, with no candidate round trip through memory.
//
// Thread t holds the float4 groups t, t + 1024, ... of the row (coalesced
// loads, and rows of any length spread over all threads).  2048 evenly
// spaced columns, loaded beside the row, are the sample: the 11-bit digit
// histogram of their keys, then the next 11 bits of the samples in the
// chosen digit, give key_lo, the sampled bound on the k-th largest key with
// the same 30 % rank margin, to 22 key bits.  The columns of the logits at
// or above it (about 1.3 k) are compacted into LDS in any order (each
// thread marks its qualifying registers in a bit mask and writes only
// those columns; a wave reserves its slots with one atomic), and the
// linear histogram, the threshold-bin rank and the output run on 4
// compacted keys per thread, read back from the row.  The output marks the
// winners in two column bitmaps (above T, equal to T); each thread then owns
// 16, 32 or 64 consecutive columns of them (as the row's length needs, so
// the winners spread over all threads), and a scan of the per-thread counts
// puts every winner at its ascending-column slot.  A row the compacted keys
// cannot settle (more than kCompCap keys at or above the bound, fewer than
// k, an unusable value range or threshold bin) takes the exact radix select
// over the row in memory instead.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void topk_wide_kernel(
    const float* __restrict__ logits, int64_t stride, const int32_t* __restrict__ row_len,
    int32_t k, int32_t* __restrict__ out_idx, SlotMap sm) {
  constexpr int NT = kThreads, kWaves = NT / 64, G = kWideCols / 4 / NT, CPER = kCompCap / NT;
  constexpr int S = 2048;  // sampled columns
  constexpr int kMapWords = kWideCols / 32;
  __shared__ __align__(16) int s_h0[kBins];  // sample digits
  __shared__ __align__(16) int s_h1[kBins];  // linear bins
  __shared__ __align__(16) int s_h2[kBins];  // next 11 bits of the samples in the chosen digit
  __shared__ __align__(16) uint32_t s_map[2 * kMapWords];  // the winner bitmaps
  __shared__ uint16_t s_cp[kCompCap + 1];  // compacted columns (slot kCompCap: past the capacity)
  uint32_t* const s_bgt = s_map;              // bit c: column c is above T
  uint32_t* const s_beq = s_map + kMapWords;  // bit c: column c equals T
  __shared__ uint32_t s_cand[kCandMax];
  __shared__ int s_wsum[kWaves + 1];
  __shared__ uint32_t s_misc[3];  // [0] threshold-bin keys, [1] largest sampled key, [2] compacted
  __shared__ int s_pick[3];
  extern __shared__ int32_t s_bt[];  // [bt_stride] when bt_lds

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int r = blockIdx.x;
  const int n = (int)min((int64_t)max(row_len[r], 0), stride);
  // Partner row r ^ 8 runs on the same XCD (workgroup g on XCD g mod 8):
  // this workgroup loads one word of each 128-byte line of the upper half
  // of a partner longer than kSegCols, so that half reaches the shared L2
  // through this CU's miss queue while the partner's own queue works on its
  // lower half (a long row arrives at about 32 GB/s through one CU).  The
  // word is folded into a value nothing reads.
  const int pr = min(r ^ 8, (int)gridDim.x - 1);
  const int np = (int)min((int64_t)max(row_len[pr], 0), stride);
  const int pline = (np >> 6) + tid;  // line of this thread's word: upper half, one line per thread
  const float* pfa =
      np > kSegCols && 32 * pline < np ? logits + (int64_t)pr * stride + 32 * pline : logits;
  const int32_t req = sm.out ? sm.row_req[r] : 0;
  const bool bt_lds = sm.out && sm.bt_stride <= kBtLds;
  if (bt_lds) {  // published by the first barrier below
    const bool okr = req >= 0 && req < sm.batch;
    for (int c = tid; c < (int)sm.bt_stride; c += NT)
      s_bt[c] = okr ? sm.bt[(int64_t)req * sm.bt_stride + c] : -1;
  }
  auto emit = [&](int j, int32_t i) {  // final index j of row r
    out_idx[(int64_t)r * k + j] = i;
    if (sm.out) {
      int32_t slot = -1;
      if (bt_lds) {
        if (i >= 0 && i / 64 < (int)sm.bt_stride) {
          const int32_t blk = s_bt[i / 64];
          slot = blk >= 0 ? blk * 64 + i % 64 : -1;
        }
      } else {
        slot = slot_of(sm, req, i);
      }
      sm.out[(int64_t)r * k + j] = slot;
    }
  };
  if (n <= k) {  // every column wins
    __syncthreads();
    for (int j = tid; j < k; j += NT) emit(j, j < n ? j : -1);
    return;
  }
  const float* x = logits + (int64_t)r * stride;

  // the row: group g = tid + j*NT holds columns 4g..4g+3; groups past the
  // row are not loaded, and columns past n read as NaN (never selected)
  const int ng = (n + 3) >> 2;
  float v[4 * G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    if (j * NT < ng) {
      const int g = min(tid + j * NT, ng - 1);
      if (VEC) {  // 4g + 3 < stride: the stride is a multiple of 4 and >= n
        const float4 f = *reinterpret_cast<const float4*>(x + 4 * g);
        v[4 * j] = f.x; v[4 * j + 1] = f.y; v[4 * j + 2] = f.z; v[4 * j + 3] = f.w;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[4 * j + i] = x[min(4 * g + i, n - 1)];
      }
    }
  }
  // the sample: columns floor(s*n/S), s < S, two per thread
  const float sv0 = x[(int)(((uint32_t)tid * (uint32_t)n) / S)];
  const float sv1 = x[(int)(((uint32_t)(tid + NT) * (uint32_t)n) / S)];
  const float pfv = *pfa;         // the partner's word, issued after this row's loads
  asm volatile("" ::: "memory");  // keeps it here: its value is used only at the end
  for (int i = tid; i < kBins; i += NT) {
    s_h0[i] = 0;
    s_h1[i] = 0;
    s_h2[i] = 0;
  }
  if (tid < 3) s_misc[tid] = 0u;
  const float qnan = __uint_as_float(0x7FC00000u);
#pragma unroll
  for (int j = 0; j < G; ++j) {
    if (j * NT >= ng) {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[4 * j + i] = qnan;
    } else if ((j + 1) * NT * 4 > n) {  // the groups that hold column n - 1
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * (tid + j * NT) + i >= n) v[4 * j + i] = qnan;
    }
  }
  __syncthreads();  // histograms clear; s_bt published

  auto pick = [&](const int* h, int nd, bool clamp = false) {
    if (wid == 0) {
      const BinPick p = pick_bin<kBins, true>(h, nd, clamp);
      if (lane == 0) {
        s_pick[0] = p.bin;
        s_pick[1] = p.above;
        s_pick[2] = p.found;
      }
    }
    __syncthreads();
    return BinPick{s_pick[0], s_pick[1], s_pick[2] != 0};
  };
  auto fallback = [&]() {
    __syncthreads();  // every wave is past its reads of the histograms and candidates
    stream_select<NT, VEC>(x, n, k, s_h1, s_wsum, reinterpret_cast<uint32_t(*)[2]>(s_cand), emit);
  };

  // 1. key_lo: the m-th largest sampled key to 22 bits (all S samples are
  // columns of the row; NaNs have key 1)
  const uint32_t sk0 = sel_key(sv0), sk1 = sel_key(sv1);
  atomicAdd(&s_h0[sk0 >> 21], 1);
  atomicAdd(&s_h0[sk1 >> 21], 1);
  const uint32_t wmax = wave_max_dpp(max(sk0, sk1));
  if (lane == 63) atomicMax(&s_misc[1], wmax);
  __syncthreads();
  // k*S*13 < 2^26 and n*10 < 2^20: 32-bit arithmetic
  const int m = min(S, (int)(((uint32_t)k * S * 13u + (uint32_t)n * 10u - 1u) / ((uint32_t)n * 10u)) + 8);
  const BinPick pc = pick(s_h0, m);
  if ((sk0 >> 21) == (uint32_t)pc.bin) atomicAdd(&s_h2[(sk0 >> 10) & 0x7FFu], 1);
  if ((sk1 >> 21) == (uint32_t)pc.bin) atomicAdd(&s_h2[(sk1 >> 10) & 0x7FFu], 1);
  __syncthreads();
  const BinPick pf = pick(s_h2, m - pc.above);
  const uint32_t key_lo = ((uint32_t)pc.bin << 21) | (pf.found ? (uint32_t)pf.bin << 10 : 0u);
  const uint32_t key_top = max(s_misc[1], key_lo);
  const float v_lo = order_key_value(key_lo);
  const float range = order_key_value(key_top) - v_lo;
  const float scale = 2048.0f / range;
  auto fbin = [&](uint32_t kk) {
    return (int)fminf((order_key_value(kk) - v_lo) * scale, (float)(kBins - 1));
  };
  // a finite, non-empty range (anything else: the radix select)
  if (!(pc.found && isfinite(v_lo) && isfinite(range) && range > 0.0f && isfinite(scale))) {
    fallback();
    return;
  }

  // 2. compaction of the logits >= v_lo, i.e. the keys >= key_lo (v_lo is
  // the finite float whose key is key_lo; NaN compares false)
  // Each thread marks its qualifying positions in a 64-bit mask and writes
  // only their columns (a loop over the set bits, about 3 per thread); the
  // few compacted logits are read back from the row (in L2) as keys.
  {
    uint64_t qm = 0;
#pragma unroll
    for (int e = 0; e < 4 * G; ++e) qm |= (uint64_t)(v[e] >= v_lo) << e;
    const int cnt = __popcll(qm);
    const int incl = wave_scan_dpp(cnt);
    int wbase = 0;
    if (lane == 63) wbase = (int)atomicAdd(&s_misc[2], (uint32_t)incl);
    int off = __builtin_amdgcn_readlane(wbase, 63) + incl - cnt;
    while (qm != 0) {
      const int e = (int)__builtin_ctzll(qm);
      qm &= qm - 1;
      s_cp[min(off, kCompCap)] = (uint16_t)(4 * (tid + (e >> 2) * NT) + (e & 3));
      ++off;
    }
  }
  __syncthreads();
  const int total = (int)s_misc[2];
  if (total < k || total > kCompCap) {
    fallback();
    return;
  }
  uint32_t ckey[CPER];
  int32_t ccol[CPER];
#pragma unroll
  for (int j = 0; j < CPER; ++j) {
    const int i = tid + j * NT;
    ccol[j] = i < total ? (int32_t)s_cp[i] : -1;
  }
#pragma unroll
  for (int j = 0; j < CPER; ++j) ckey[j] = ccol[j] >= 0 ? sel_key(x[ccol[j]]) : 0u;

  // 3. linear bins over [v_lo, v_top]; the threshold bin's keys ranked by
  // brute force give T
#pragma unroll
  for (int j = 0; j < CPER; ++j)
    if (ckey[j] != 0u) atomicAdd(&s_h1[fbin(ckey[j])], 1);
  __syncthreads();
  // the bitmaps are cleared here and published by the pick's barrier
  for (int i = tid; i < 2 * kMapWords; i += NT) s_map[i] = 0u;
  const BinPick p1 = pick(s_h1, k);
  if (p1.found) {
#pragma unroll
    for (int j = 0; j < CPER; ++j) {
      if (ckey[j] != 0u && fbin(ckey[j]) == p1.bin) {
        const uint32_t sl = atomicAdd(&s_misc[0], 1u);
        if (sl < (uint32_t)kCandMax) s_cand[sl] = ckey[j];
      }
    }
  }
  __syncthreads();
  uint32_t T = 0;
  int need = 0;  // keys equal to T that win (lowest columns first)
  bool ok = p1.found && s_misc[0] <= (uint32_t)kCandMax;
  if (ok) {  // every wave computes the same from the same LDS contents
    const int nc = (int)s_misc[0];
    const int need1 = k - p1.above;
    const uint32_t c = lane < nc ? s_cand[lane] : 0u;
    int gt = 0, ge = 0;
    for (int j = 0; j < nc; ++j) {
      const uint32_t cj = __builtin_amdgcn_readlane(c, j);
      gt += cj > c;
      ge += cj >= c;
    }
    const uint64_t hm = __ballot(lane < nc && gt < need1 && need1 <= ge);
    if (hm != 0) {
      const int src = (int)__builtin_ctzll(hm);
      T = __builtin_amdgcn_readlane(c, src);
      need = need1 - __builtin_amdgcn_readlane(gt, src);
    } else {
      ok = false;
    }
  }
  if (!ok) {
    fallback();
    return;
  }

  // 4. ordered output through the bitmaps: thread t owns columns
  // [Ct, Ct + C), C = 16, 32 or 64 as the row needs (so the winners of a
  // shorter row spread over all threads too); counts packed as
  // (equal << 12) | above (above-T totals stay below k <= 2048, equal
  // totals at most kCompCap)
#pragma unroll
  for (int j = 0; j < CPER; ++j) {
    if (ckey[j] > T) atomicOr(&s_bgt[ccol[j] >> 5], 1u << (ccol[j] & 31));
    else if (ckey[j] == T && ckey[j] != 0u) atomicOr(&s_beq[ccol[j] >> 5], 1u << (ccol[j] & 31));
  }
  __syncthreads();
  const int cs = n <= 16 * NT ? 4 : n <= 32 * NT ? 5 : 6;  // log2 C, uniform
  uint64_t gm, em;
  if (cs == 6) {
    const uint2 g2 = reinterpret_cast<const uint2*>(s_bgt)[tid];
    const uint2 e2 = reinterpret_cast<const uint2*>(s_beq)[tid];
    gm = (uint64_t)g2.x | ((uint64_t)g2.y << 32);
    em = (uint64_t)e2.x | ((uint64_t)e2.y << 32);
  } else if (cs == 5) {
    gm = s_bgt[tid];
    em = s_beq[tid];
  } else {
    gm = (s_bgt[tid >> 1] >> (16 * (tid & 1))) & 0xFFFFu;
    em = (s_beq[tid >> 1] >> (16 * (tid & 1))) & 0xFFFFu;
  }
  const int packed = __popcll(gm) | (__popcll(em) << 12);
  const int inc = wave_scan_dpp(packed);
  if (lane == 63) s_wsum[wid] = inc;
  __syncthreads();
  int ex = inc - packed;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) ex += w < wid ? s_wsum[w] : 0;
  int gt_b = ex & 0xFFF, eq_b = ex >> 12;
  uint64_t all = gm | em;
  while (all != 0) {
    const int b = (int)__builtin_ctzll(all);
    all &= all - 1;
    int pos = -1;
    if ((gm >> b) & 1u) {
      pos = gt_b + min(eq_b, need);
      ++gt_b;
    } else {
      if (eq_b < need) pos = gt_b + eq_b;
      ++eq_b;
    }
    if ((unsigned)pos < (unsigned)k) emit(pos, (tid << cs) + b);
  }
  if (__float_as_uint(pfv) == 0x7FC00001u && k < 0) out_idx[0] = 0;  // never true (k >= 1)
}

// How topk_rows handles a row pitch: rows up to kSegCols columns are
// selected in one pass; in launches of fewer than kManyWgs rows, rows up to
// kWideCols columns too (topk_wide_kernel); other wider rows are cut into
// kSegCols-column segments whose winners are merged by a second pass, as
// long as a row's candidate lists fit one workgroup (16384 slots); wider
// still take the streaming kernel.  Workgroup shape: with at least kManyWgs
// workgroups the smallest of 256 or 512 threads x 4..32 positions that
// holds the work, so several workgroups share a CU; with fewer, 1024
// threads x 4..16 positions, which shortens each workgroup's chain.
struct Shape {
  int nt, vpt;  // nt == 0: no register-resident shape holds the work
};

// max_vpt: one-pass launches of many rows stop at 16 positions per thread
// (then 1024 threads): 32-position shapes were slower there (16384-column
// rows: 404 -> 286 us, 8192-column rows: 150 -> 140 us); segment passes keep
// 32 (256 rows x 4 segments: 50.6 us with 512 x 32, 56.1 with 1024 x 16).
Shape shape_for(int64_t n, int64_t wgs, int max_vpt = 32) {
  if (wgs >= kManyWgs) {
    for (int nt : {256, 512})
      for (int vpt : {4, 8, 16, 32})
        if (vpt <= max_vpt && n <= (int64_t)nt * vpt) return {nt, vpt};
  }
  for (int vpt : {4, 8, 16})
    if (n <= 1024LL * vpt) return {1024, vpt};
  return {0, 0};
}

struct TopkPlan {
  Shape one;    // one-pass shape (nt == 0: not one-pass)
  int nseg;     // segments per row (split plan)
  Shape seg;    // segment pass
  Shape merge;  // merge pass
  bool stream;  // neither: the streaming kernel
  bool wide;    // one pass of topk_wide_kernel
};

TopkPlan plan_for(int64_t stride, int k, int64_t rows) {
  if (stride <= kSegCols) return {shape_for(stride, rows, 16), 0, {0, 0}, {0, 0}, false, false};
  if (stride <= kWideCols && rows < kManyWgs) return {{0, 0}, 0, {0, 0}, {0, 0}, false, true};
  const int64_t nseg = (stride + kSegCols - 1) / kSegCols;
  const Shape merge = shape_for(nseg * k, rows);
  if (merge.nt == 0) return {{0, 0}, 0, {0, 0}, {0, 0}, true, false};
  return {{0, 0}, (int)nseg, shape_for(kSegCols, rows * nseg), merge, false, false};
}

template <int NT, int VPT, bool CIN, bool COUT>
void launch_sel(bool vec, unsigned grid, const float* logits, int64_t stride, const int32_t* row_len,
                int32_t k, int32_t nseg, const uint32_t* c_key, const int32_t* c_col, int32_t* out,
                uint32_t* o_key, int32_t* o_col, const SlotMap& sm, hipStream_t s) {
  const size_t dyn = sm.out && sm.bt_stride <= kBtLds ? (size_t)sm.bt_stride * sizeof(int32_t) : 0;
  // early loads only for the 1024-thread shapes, which serve launches of
  // fewer than kManyWgs workgroups
  if constexpr (NT == 1024) {
    if (grid <= kEarlyLoadWgs) {
      if (vec)
        launch((topk_select_kernel<NT, VPT, true, CIN, COUT, true>), dim3(grid), dim3(NT), dyn, s,
               logits, stride, row_len, k, nseg, c_key, c_col, out, o_key, o_col, sm, nullptr);
      else
        launch((topk_select_kernel<NT, VPT, false, CIN, COUT, true>), dim3(grid), dim3(NT), dyn, s,
               logits, stride, row_len, k, nseg, c_key, c_col, out, o_key, o_col, sm, nullptr);
      return;
    }
  }
  if (vec)
    launch((topk_select_kernel<NT, VPT, true, CIN, COUT, false>), dim3(grid), dim3(NT), dyn, s,
           logits, stride, row_len, k, nseg, c_key, c_col, out, o_key, o_col, sm, nullptr);
  else
    launch((topk_select_kernel<NT, VPT, false, CIN, COUT, false>), dim3(grid), dim3(NT), dyn, s,
           logits, stride, row_len, k, nseg, c_key, c_col, out, o_key, o_col, sm, nullptr);
}

// Launches the shape's instantiation (segment passes exist only for the
// shapes that cover exactly one segment).
template <bool CIN, bool COUT>
void launch_shape(Shape sh, bool vec, unsigned grid, const float* logits, int64_t stride,
                  const int32_t* row_len, int32_t k, int32_t nseg, const uint32_t* c_key,
                  const int32_t* c_col, int32_t* out, uint32_t* o_key, int32_t* o_col,
                  const SlotMap& sm, hipStream_t s) {
#define SAI_SEL_CASE(NT_, VPT_)                                                                  \
  if constexpr (!COUT || NT_ * VPT_ == kSegCols) {                                              \
    if (sh.nt == NT_ && sh.vpt == VPT_) {                                                       \
      launch_sel<NT_, VPT_, CIN, COUT>(vec, grid, logits, stride, row_len, k, nseg, c_key, c_col, \
                                       out, o_key, o_col, sm, s);                               \
      return;                                                                                   \
    }                                                                                           \
  }
  SAI_SEL_CASE(256, 4)
  SAI_SEL_CASE(256, 8)
  SAI_SEL_CASE(256, 16)
  SAI_SEL_CASE(256, 32)
  SAI_SEL_CASE(512, 4)
  SAI_SEL_CASE(512, 8)
  SAI_SEL_CASE(512, 16)
  SAI_SEL_CASE(512, 32)
  SAI_SEL_CASE(1024, 4)
  SAI_SEL_CASE(1024, 8)
  SAI_SEL_CASE(1024, 16)
#undef SAI_SEL_CASE
}

bool aligned16p(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" size_t topk_workspace_bytes(int32_t rows, int64_t logits_stride, int32_t k) {
  if (rows <= 0 || logits_stride <= 0 || k < 1 || k > SAI_TOPK_MAX) return 0;
  const TopkPlan p = plan_for(logits_stride, k, rows);
  if (p.nseg == 0) return 0;
  // candidate keys then candidate columns, [rows][nseg][k] each
  return (size_t)rows * (size_t)p.nseg * (size_t)k * 8u;
}

namespace {

int topk_impl(const float* logits, int64_t logits_stride, const int32_t* row_len, int32_t rows,
              int32_t k, int32_t* out_idx, void* workspace, size_t workspace_bytes,
              const SlotMap& sm, bool* streamed, hipStream_t stream) {
  *streamed = false;
  if (rows < 0 || logits_stride < 0) return SAI_EINVAL;
  if (k < 1 || k > SAI_TOPK_MAX) return SAI_EUNSUPPORTED;
  if (rows == 0) return SAI_OK;
  if (!logits || !row_len || !out_idx || logits_stride == 0) return SAI_EINVAL;
  if (logits_stride > 0x7FFFFFFF - 4 * kThreads) return SAI_EUNSUPPORTED;
  const bool vec = (logits_stride % 4 == 0) && aligned16p(logits);
  const TopkPlan p = plan_for(logits_stride, k, rows);
  const unsigned ur = (unsigned)rows;
  if (p.nseg > 0) {  // checked before anything is launched
    const size_t need = topk_workspace_bytes(rows, logits_stride, k);
    if (!workspace || workspace_bytes < need) return SAI_EWORKSPACE;
    if ((int64_t)rows * p.nseg > 0x7FFFFFFF) return SAI_EUNSUPPORTED;
  }
  if (p.wide) {
    const size_t dyn = sm.out && sm.bt_stride <= kBtLds ? (size_t)sm.bt_stride * sizeof(int32_t) : 0;
    if (vec)
      launch(topk_wide_kernel<true>, dim3(ur), dim3(kThreads), dyn, stream, logits, logits_stride,
             row_len, k, out_idx, sm);
    else
      launch(topk_wide_kernel<false>, dim3(ur), dim3(kThreads), dyn, stream, logits, logits_stride,
             row_len, k, out_idx, sm);
  } else if (p.one.nt) {
    launch_shape<false, false>(p.one, vec, ur, logits, logits_stride, row_len, k, 1, nullptr, nullptr,
                               out_idx, nullptr, nullptr, sm, stream);
  } else if (p.nseg > 0) {
    uint32_t* ck = static_cast<uint32_t*>(workspace);
    int32_t* cc = reinterpret_cast<int32_t*>(ck + (size_t)rows * p.nseg * k);
    const bool cvec = (k % 4 == 0) && aligned16p(workspace);
    // the segment pass also writes the final output of rows that fit one segment
    launch_shape<false, true>(p.seg, vec, ur * (unsigned)p.nseg, logits, logits_stride, row_len, k,
                              p.nseg, nullptr, nullptr, out_idx, ck, cc, sm, stream);
    launch_shape<true, false>(p.merge, cvec, ur, logits, logits_stride, row_len, k, p.nseg, ck, cc,
                              out_idx, nullptr, nullptr, sm, stream);
  } else {
    *streamed = true;
    if (vec)
      launch(topk_row_kernel<true>, dim3(rows), dim3(kThreads), 0, stream, logits,
                         logits_stride, row_len, k, out_idx);
    else
      launch(topk_row_kernel<false>, dim3(rows), dim3(kThreads), 0, stream, logits,
                         logits_stride, row_len, k, out_idx);
  }
  return hipGetLastError() == hipSuccess ? SAI_OK : SAI_ELAUNCH;
}

}  // namespace

extern "C" int topk_rows(const float* logits, int64_t logits_stride, const int32_t* row_len,
                         int32_t rows, int32_t k, int32_t* out_idx, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  bool streamed;
  return topk_impl(logits, logits_stride, row_len, rows, k, out_idx, workspace, workspace_bytes,
                   SlotMap{nullptr, nullptr, 0, 0, nullptr}, &streamed, stream);
}

extern "C" int topk_rows_slots(const float* logits, int64_t logits_stride, const int32_t* row_len,
                               const int32_t* row_req, const int32_t* block_table, int64_t bt_stride,
                               int32_t batch, int32_t rows, int32_t k, int32_t* out_idx,
                               int32_t* out_slots, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  if (rows < 0 || batch < 0 || bt_stride < 0) return SAI_EINVAL;
  if (rows > 0 && (!row_req || !block_table || !out_slots)) return SAI_EINVAL;
  bool streamed;
  const int st = topk_impl(logits, logits_stride, row_len, rows, k, out_idx, workspace,
                           workspace_bytes, SlotMap{row_req, block_table, bt_stride, batch, out_slots},
                           &streamed, stream);
  if (st != SAI_OK || !streamed) return st;
  // rows too wide for the fused kernels: map the indices afterwards
  return topk_to_global_slots(out_idx, row_req, block_table, bt_stride, batch, rows, k, out_slots,
                              stream);
}

// ------------------------------------------------- allocation-free variant
// topk_rows_slots_noalloc keeps the segment candidates of wide rows in this
// file-scope device array instead of a caller workspace.  In host code the
// name `scratch` is a host-side stand-in, not a device address: the address
// is resolved per device with hipGetSymbolAddress (with that device
// current) and only the resolved pointer is passed to kernels.  Each device
// holds its own copy until the process ends; every call on a device shares
// it, so calls that overlap on one device race.  The passes overwrite every
// candidate slot they later read, so nothing needs clearing between calls.
static __device__ __align__(256) uint8_t scratch[SAI_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device that owns `stream`, resolved on
// the first call for that device (two threads racing here store the same
// address).
int scratch_for_stream(hipStream_t stream, void** out) {
  int dev = -1, cur = -1;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess || hipGetDevice(&cur) != hipSuccess)
    return SAI_ELAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return SAI_EUNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return SAI_ELAUNCH;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return SAI_ELAUNCH;
    if (e != hipSuccess || p == nullptr) return SAI_ELAUNCH;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return SAI_OK;
}

}  // namespace

extern "C" int topk_rows_slots_noalloc(const float* logits, int64_t logits_stride,
                                       const int32_t* row_len, const int32_t* row_req,
                                       const int32_t* block_table, int64_t bt_stride, int32_t batch,
                                       int32_t rows, int32_t k, int32_t* out_idx, int32_t* out_slots,
                                       hipStream_t stream) {
  if (rows < 0 || batch < 0 || bt_stride < 0 || logits_stride < 0) return SAI_EINVAL;
  if (k < 1 || k > SAI_TOPK_MAX) return SAI_EUNSUPPORTED;
  if (rows == 0) return SAI_OK;
  const size_t need = topk_workspace_bytes(rows, logits_stride, k);
  if (need > (size_t)SAI_NOALLOC_SCRATCH_BYTES) return SAI_ESCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    const int st = scratch_for_stream(stream, &ws);
    if (st != SAI_OK) return st;
  }
  return topk_rows_slots(logits, logits_stride, row_len, row_req, block_table, bt_stride, batch, rows,
                         k, out_idx, out_slots, ws, need, stream);
}

// ------------------------------------------------------------ fused decode
namespace {

// The histogram-seeded one-pass selection (1024 threads, early loads).
void launch_hist_sel(int vpt, bool vec, unsigned rows, const float* logits, int64_t stride,
                     const int32_t* row_len, int32_t k, int32_t* out, const SlotMap& sm, int32_t* hist,
                     hipStream_t s) {
  const size_t dyn = sm.out && sm.bt_stride <= kBtLds ? (size_t)sm.bt_stride * sizeof(int32_t) : 0;
#define SAI_HIST_CASE(VPT_)                                                                             \
  if (vpt == VPT_) {                                                                                    \
    if (vec)                                                                                            \
      launch((topk_select_kernel<1024, VPT_, true, false, false, true, true>), dim3(rows), dim3(1024), dyn, s, \
             logits, stride, row_len, k, 1, nullptr, nullptr, out, nullptr, nullptr, sm, hist);         \
    else                                                                                                \
      launch((topk_select_kernel<1024, VPT_, false, false, false, true, true>), dim3(rows), dim3(1024), dyn, \
             s, logits, stride, row_len, k, 1, nullptr, nullptr, out, nullptr, nullptr, sm, hist);      \
    return;                                                                                             \
  }
  SAI_HIST_CASE(4)
  SAI_HIST_CASE(8)
  SAI_HIST_CASE(16)
#undef SAI_HIST_CASE
}

// Whether a decode step of `rows` rows of width `stride` takes the
// histogram-seeded selection (and the shape it runs in).
bool hist_shape(int64_t rows, int64_t stride, Shape* sh) {
  if (stride > kSegCols || rows >= kManyWgs) return false;
  *sh = shape_for(stride, rows, 16);
  return sh->nt == 1024;
}

}  // namespace

extern "C" size_t paged_mqa_topk_hist_bytes(int32_t rows, int64_t logits_stride) {
  Shape sh;
  if (rows <= 0 || logits_stride <= 0 || !hist_shape(rows, logits_stride, &sh)) return 0;
  return (size_t)rows * kHistBins * sizeof(int32_t);
}

extern "C" int paged_mqa_topk_slots(const void* q_fp8, const float* weights, const void* kv_cache,
                                    int64_t num_blocks, const int32_t* block_table, int64_t bt_stride,
                                    const int32_t* context_lens, int32_t batch, int32_t next_n,
                                    float* logits, int64_t logits_stride, int32_t* row_len_out,
                                    int32_t* row_req_out, int32_t k, int32_t* out_idx, int32_t* out_slots,
                                    int32_t* hist, size_t hist_bytes, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  // everything the selection needs is checked before the logits launch
  if (batch < 0 || logits_stride < 0 || bt_stride < 0 || num_blocks < 0) return SAI_EINVAL;
  if (next_n < 1 || next_n > SAI_NEXT_N_MAX || k < 1 || k > SAI_TOPK_MAX) return SAI_EUNSUPPORTED;
  if (batch == 0) return SAI_OK;
  const int64_t rows = (int64_t)batch * next_n;
  if (!logits || !row_len_out || !row_req_out || !out_idx || !out_slots || !block_table) return SAI_EINVAL;
  if (logits_stride == 0) return SAI_EINVAL;
  if (logits_stride > 0x7FFFFFFF - 4 * kThreads) return SAI_EUNSUPPORTED;
  Shape sh;
  const size_t need_hist = paged_mqa_topk_hist_bytes((int32_t)rows, logits_stride);
  const bool use_hist = hist != nullptr && need_hist > 0 && hist_shape(rows, logits_stride, &sh);
  if (use_hist && hist_bytes < need_hist) return SAI_EWORKSPACE;
  if (!use_hist) {
    const TopkPlan p = plan_for(logits_stride, k, rows);
    if (p.nseg > 0 && (!workspace || workspace_bytes < topk_workspace_bytes((int32_t)rows, logits_stride, k)))
      return SAI_EWORKSPACE;
  }
  const int st = sai_paged_logits(q_fp8, weights, kv_cache, num_blocks, block_table, bt_stride, context_lens,
                                  batch, next_n, logits, logits_stride, row_len_out, row_req_out, true,
                                  use_hist ? hist : nullptr, stream);
  if (st != SAI_OK) return st;
  if (!use_hist)
    return topk_rows_slots(logits, logits_stride, row_len_out, row_req_out, block_table, bt_stride, batch,
                           (int32_t)rows, k, out_idx, out_slots, workspace, workspace_bytes, stream);
  const bool vec = (logits_stride % 4 == 0) && aligned16p(logits);
  launch_hist_sel(sh.vpt, vec, (unsigned)rows, logits, logits_stride, row_len_out, k, out_idx,
                  SlotMap{row_req_out, block_table, bt_stride, batch, out_slots}, hist, stream);
  return hipGetLastError() == hipSuccess ? SAI_OK : SAI_ELAUNCH;
}
