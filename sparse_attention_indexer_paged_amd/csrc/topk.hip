// Per-row top-k of the indexer logits (ROCm/ATOM PR #1094, Technical
// Details: the sparse top-k over each query's request-local keys, handed on
// in a 2-D [rows, k] index buffer).
//
// Selection is exact radix select on 32-bit order-preserving keys
// (f32_order_key: larger logit -> larger key, -0.0 folded onto +0.0):
//   digit 1 = key bits 31..21 (2048 bins), digit 2 = bits 20..10 (2048),
//   digit 3 = bits 9..0 (1024).
// Each round histograms, in LDS, the keys whose higher digits equal the
// prefix fixed so far, then one pass over the bins (a workgroup scan from
// the top bin down) picks the bin holding the k-th largest key.  After three
// rounds the k-th largest key T is known exactly, with `gt` keys above it and
// need = k - gt of the keys equal to T to be taken, lowest indices first.
// The output pass walks the row in ascending index order; a workgroup scan
// of per-thread (above-T, equal-to-T) counts gives every winner its output
// slot, so indices come out sorted with no sort.
// Rows whose visible length is at most k skip all of this and emit 0..n-1.
//
// Rows of up to 16384 columns are read from memory once: thread t of a
// 1024-thread workgroup keeps the keys of columns [t*VPT, (t+1)*VPT) in
// registers through all three rounds and the output pass
// (topk_reg_kernel).  Wider rows take the streaming kernel, which re-reads
// the row from L2 for every pass.
#include "sai_device.h"

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

// VEC: rows are 16-byte aligned, so 4 consecutive columns load as one float4.
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
  const float* x = logits + (int64_t)r * stride;

  uint32_t prefix = 0, pmask = 0;
  int need = k;  // winners still to place among keys matching the prefix
  const int shifts[3] = {21, 10, 0};
  const uint32_t dmask[3] = {0x7FFu, 0x7FFu, 0x3FFu};
  for (int round = 0; round < 3; ++round) {
    const int sh = shifts[round];
    const uint32_t dm = dmask[round];
    const int nb = (int)dm + 1;
    for (int i = tid; i < kBins; i += kThreads) s_hist[i] = 0;
    if (tid == 0) s_sel[round][0] = s_sel[round][1] = 0;
    __syncthreads();
    for (int i = tid * 4; i < n; i += kThreads * 4) {
      float v[4];
      load4<VEC>(x, i, n, v);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (i + e < n) {
          const uint32_t key = f32_order_key(v[e]);
          if ((key & pmask) == prefix) atomicAdd(&s_hist[(key >> sh) & dm], 1);
        }
      }
    }
    __syncthreads();
    // thread t owns bins nb-1-2t and nb-2-2t (descending), scanned in thread order
    const int bhi = nb - 1 - 2 * tid, blo = nb - 2 - 2 * tid;
    const int hhi = bhi >= 0 ? s_hist[bhi] : 0;
    const int hlo = blo >= 0 ? s_hist[blo] : 0;
    int total;
    const int before = block_exclusive_scan<kThreads>(hhi + hlo, s_scan, &total);
    if (bhi >= 0 && before < need && need <= before + hhi) {
      s_sel[round][0] = (uint32_t)bhi;
      s_sel[round][1] = (uint32_t)before;
    } else if (blo >= 0 && before + hhi < need && need <= before + hhi + hlo) {
      s_sel[round][0] = (uint32_t)blo;
      s_sel[round][1] = (uint32_t)(before + hhi);
    }
    __syncthreads();
    prefix |= s_sel[round][0] << sh;
    pmask |= dm << sh;
    need -= (int)s_sel[round][1];
  }
  const uint32_t T = prefix;

  // ordered output: tiles of kThreads*4 columns, thread t owns 4 consecutive
  int gt_run = 0, eq_run = 0;
  for (int base = 0; base < n; base += kThreads * 4) {
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
    const int ex = block_exclusive_scan<kThreads>(ngt | (neq << 16), s_scan, &tot);
    int gt_b = gt_run + (ex & 0xFFFF), eq_b = eq_run + (ex >> 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (i + e >= n) break;
      if (key[e] > T) {
        const int pos = gt_b + min(eq_b, need);
        if ((unsigned)pos < (unsigned)k) o[pos] = i + e;
        ++gt_b;
      } else if (key[e] == T) {
        const int pos = gt_b + eq_b;
        if (eq_b < need && (unsigned)pos < (unsigned)k) o[pos] = i + e;
        ++eq_b;
      }
    }
    gt_run += tot & 0xFFFF;
    eq_run += tot >> 16;
  }
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

#ifndef SAI_TOPK_THREADS
#define SAI_TOPK_THREADS 1024
#endif
constexpr int kRegThreads = SAI_TOPK_THREADS;

// Wave 0 of the workgroup finds the bin holding the need-th largest count
// of hist[0..NB): lane l owns the PER = NB/64 bins [NB-PER(l+1), NB-PER*l),
// read with 16-byte LDS loads into registers; a DPP scan of the lane sums in
// lane order (= descending bins) finds the lane that holds the need-th
// element, and that lane walks its registers downwards.  It writes
// {bin, count above the bin, 1} to sel, or leaves sel untouched if the
// histogram holds fewer than need elements.
template <int NB>
__device__ __forceinline__ void select_bin(const int* hist, int need, int* sel) {
  constexpr int PER = NB / 64;
  const int lane = threadIdx.x & 63;
  const int lo = NB - PER * (lane + 1);
  int h[PER];
#pragma unroll
  for (int j = 0; j < PER; j += 4) {
    const int4 v = *reinterpret_cast<const int4*>(hist + lo + j);
    h[j] = v.x; h[j + 1] = v.y; h[j + 2] = v.z; h[j + 3] = v.w;
  }
  int sum = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) sum += h[j];
  const int inc = wave_scan_dpp(sum);
  int acc = inc - sum;
  if (acc < need && need <= inc) {
    int bin = lo, above = acc;
    bool done = false;
#pragma unroll
    for (int j = PER - 1; j >= 0; --j) {
      if (!done) {
        if (acc + h[j] >= need) {
          bin = lo + j;
          above = acc;
          done = true;
        } else {
          acc += h[j];
        }
      }
    }
    sel[0] = bin;
    sel[1] = above;
    sel[2] = 1;
  }
}

// Register-resident radix select: thread t owns the VPT consecutive
// columns [t*VPT, (t+1)*VPT) of the row (rows up to kRegThreads*VPT columns).
// Before the first round, a sample of one key per thread (every VPT-th
// column) locates a lower bound on the first digit of the k-th largest key,
// with a 30% margin; the first round then counts only keys at or above it,
// which cuts its LDS atomics several-fold.  If the pruned count holds fewer
// than k keys, the first round is redone over every key, so the result is
// exact either way.  Every output write is bounds-guarded by k.
template <int VPT, bool VEC>
__global__ __launch_bounds__(kRegThreads) void topk_reg_kernel(
    const float* __restrict__ logits, int64_t stride, const int32_t* __restrict__ row_len,
    int32_t k, int32_t* __restrict__ out) {
  __shared__ __align__(16) int s_hist[kBins];
  __shared__ int s_wsum[kRegThreads / 64];
  __shared__ int s_sel[5][3];  // sample, round 1, round 1 again, round 2, round 3

  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  constexpr int kWaves = kRegThreads / 64;
  int32_t* o = out + (int64_t)r * k;
  const int n = (int)min((int64_t)max(row_len[r], 0), stride);
  if (n <= k) {
    for (int j = tid; j < k; j += kRegThreads) o[j] = j < n ? j : -1;
    return;
  }
  const float* x = logits + (int64_t)r * stride;
  const int base = tid * VPT;
  uint32_t key[VPT];
#pragma unroll
  for (int e = 0; e < VPT; e += 4) {
    float v[4];
    load4<VEC>(x, base + e, n, v);
#pragma unroll
    for (int i = 0; i < 4; ++i) key[e + i] = f32_order_key(v[i]);
  }

  auto clear = [&](int slot) {
    for (int i = tid; i < kBins; i += kRegThreads) s_hist[i] = 0;
    if (tid < 3) s_sel[slot][tid] = 0;
    __syncthreads();
  };

  // sample: one key per thread that owns any column
  clear(0);
  if (base < n) atomicAdd(&s_hist[key[0] >> 21], 1);
  __syncthreads();
  const int S = (n + VPT - 1) / VPT;
  const int m = min(S, (int)(((int64_t)k * S * 13 + (int64_t)n * 10 - 1) / ((int64_t)n * 10)) + 8);
  if (wid == 0) select_bin<kBins>(s_hist, m, s_sel[0]);
  __syncthreads();
  const uint32_t lo_digit = (uint32_t)s_sel[0][0];

  // round 1 on keys whose first digit is at least lo_digit
  clear(1);
#pragma unroll
  for (int e = 0; e < VPT; ++e)
    if (base + e < n && (key[e] >> 21) >= lo_digit) atomicAdd(&s_hist[key[e] >> 21], 1);
  __syncthreads();
  if (wid == 0) select_bin<kBins>(s_hist, k, s_sel[1]);
  __syncthreads();
  int slot = 1;
  if (!s_sel[1][2]) {  // pruned too much: count every key
    clear(2);
#pragma unroll
    for (int e = 0; e < VPT; ++e)
      if (base + e < n) atomicAdd(&s_hist[key[e] >> 21], 1);
    __syncthreads();
    if (wid == 0) select_bin<kBins>(s_hist, k, s_sel[2]);
    __syncthreads();
    slot = 2;
  }
  uint32_t prefix = (uint32_t)s_sel[slot][0] << 21;
  uint32_t pmask = 0x7FFu << 21;
  int need = k - s_sel[slot][1];

  // round 2: bits 20..10 of keys matching the first digit
  clear(3);
#pragma unroll
  for (int e = 0; e < VPT; ++e)
    if (base + e < n && (key[e] & pmask) == prefix) atomicAdd(&s_hist[(key[e] >> 10) & 0x7FF], 1);
  __syncthreads();
  if (wid == 0) select_bin<kBins>(s_hist, need, s_sel[3]);
  __syncthreads();
  prefix |= (uint32_t)s_sel[3][0] << 10;
  pmask |= 0x7FFu << 10;
  need -= s_sel[3][1];

  // round 3: bits 9..0
  clear(4);
#pragma unroll
  for (int e = 0; e < VPT; ++e)
    if (base + e < n && (key[e] & pmask) == prefix) atomicAdd(&s_hist[key[e] & 0x3FF], 1);
  __syncthreads();
  if (wid == 0) select_bin<1024>(s_hist, need, s_sel[4]);
  __syncthreads();
  prefix |= (uint32_t)s_sel[4][0];
  need -= s_sel[4][1];
  const uint32_t T = prefix;

  // ordered output over the whole row: counts packed as (equal << 12) | above
  // (above-T totals stay below k <= 2048; equal totals below 2^20)
  int ngt = 0, neq = 0;
#pragma unroll
  for (int e = 0; e < VPT; ++e) {
    const bool in = base + e < n;
    ngt += (in && key[e] > T);
    neq += (in && key[e] == T);
  }
  const int packed = ngt | (neq << 12);
  const int inc = wave_scan_dpp(packed);
  if (lane == 63) s_wsum[wid] = inc;
  __syncthreads();
  int ex = inc - packed;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) ex += w < wid ? s_wsum[w] : 0;
  int gt_b = ex & 0xFFF, eq_b = ex >> 12;
#pragma unroll
  for (int e = 0; e < VPT; ++e) {
    if (base + e < n) {
      if (key[e] > T) {
        const int pos = gt_b + min(eq_b, need);
        if ((unsigned)pos < (unsigned)k) o[pos] = base + e;
        ++gt_b;
      } else if (key[e] == T) {
        const int pos = gt_b + eq_b;
        if (eq_b < need && (unsigned)pos < (unsigned)k) o[pos] = base + e;
        ++eq_b;
      }
    }
  }
}

template <int VPT>
void launch_reg(bool vec, const float* logits, int64_t stride, const int32_t* row_len, int32_t rows,
                int32_t k, int32_t* out, hipStream_t s) {
  if (vec)
    hipLaunchKernelGGL((topk_reg_kernel<VPT, true>), dim3(rows), dim3(kRegThreads), 0, s, logits,
                       stride, row_len, k, out);
  else
    hipLaunchKernelGGL((topk_reg_kernel<VPT, false>), dim3(rows), dim3(kRegThreads), 0, s, logits,
                       stride, row_len, k, out);
}

}  // namespace

extern "C" size_t topk_workspace_bytes(int32_t rows, int64_t logits_stride, int32_t k) {
  (void)rows;
  (void)logits_stride;
  (void)k;
  return 0;
}

extern "C" int topk_rows(const float* logits, int64_t logits_stride, const int32_t* row_len,
                         int32_t rows, int32_t k, int32_t* out_idx, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (rows < 0 || logits_stride < 0) return SAI_EINVAL;
  if (k < 1 || k > SAI_TOPK_MAX) return SAI_EUNSUPPORTED;
  if (rows == 0) return SAI_OK;
  if (!logits || !row_len || !out_idx || logits_stride == 0) return SAI_EINVAL;
  if (logits_stride > 0x7FFFFFFF - 4 * kThreads) return SAI_EUNSUPPORTED;
  const bool vec = (logits_stride % 4 == 0) && ((reinterpret_cast<uintptr_t>(logits) & 15u) == 0);
  if (logits_stride <= 4 * kRegThreads)
    launch_reg<4>(vec, logits, logits_stride, row_len, rows, k, out_idx, stream);
  else if (logits_stride <= 8 * kRegThreads)
    launch_reg<8>(vec, logits, logits_stride, row_len, rows, k, out_idx, stream);
  else if (logits_stride <= 16 * kRegThreads)
    launch_reg<16>(vec, logits, logits_stride, row_len, rows, k, out_idx, stream);
  else if (vec)
    hipLaunchKernelGGL(topk_row_kernel<true>, dim3(rows), dim3(kThreads), 0, stream, logits,
                       logits_stride, row_len, k, out_idx);
  else
    hipLaunchKernelGGL(topk_row_kernel<false>, dim3(rows), dim3(kThreads), 0, stream, logits,
                       logits_stride, row_len, k, out_idx);
  return hipGetLastError() == hipSuccess ? SAI_OK : SAI_ELAUNCH;
}
