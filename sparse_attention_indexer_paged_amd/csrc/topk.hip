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
// The output pass walks the row in ascending index order in tiles; a
// workgroup scan of per-thread (above-T, equal-to-T) counts gives every
// winner its output slot, so indices come out sorted with no sort.
// Rows whose visible length is at most k skip all of this and emit 0..n-1.
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
  __shared__ uint32_t s_sel[2];  // chosen bin, count above it

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
      s_sel[0] = (uint32_t)bhi;
      s_sel[1] = (uint32_t)before;
    } else if (blo >= 0 && before + hhi < need && need <= before + hhi + hlo) {
      s_sel[0] = (uint32_t)blo;
      s_sel[1] = (uint32_t)(before + hhi);
    }
    __syncthreads();
    prefix |= s_sel[0] << sh;
    pmask |= dm << sh;
    need -= (int)s_sel[1];
    __syncthreads();
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
        o[gt_b + min(eq_b, need)] = i + e;
        ++gt_b;
      } else if (key[e] == T) {
        if (eq_b < need) o[gt_b + eq_b] = i + e;
        ++eq_b;
      }
    }
    gt_run += tot & 0xFFFF;
    eq_run += tot >> 16;
  }
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
  if (vec)
    hipLaunchKernelGGL(topk_row_kernel<true>, dim3(rows), dim3(kThreads), 0, stream, logits,
                       logits_stride, row_len, k, out_idx);
  else
    hipLaunchKernelGGL(topk_row_kernel<false>, dim3(rows), dim3(kThreads), 0, stream, logits,
                       logits_stride, row_len, k, out_idx);
  return hipGetLastError() == hipSuccess ? SAI_OK : SAI_ELAUNCH;
}
