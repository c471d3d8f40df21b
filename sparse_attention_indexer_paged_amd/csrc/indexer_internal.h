// Library-internal pieces shared between the logits and top-k sources (not
// part of the C ABI).
#pragma once

#include "sai_device.h"

namespace sai {

// The per-row histograms the fused decode path passes from the logits
// kernel to the top-k: counts of the top kHistBits bits of each visible
// logit's order key (f32_order_key), kHistBins int32 per row.
constexpr int kHistBits = 10;
constexpr int kHistBins = 1 << kHistBits;

}  // namespace sai

// The paged logits launch (logits.hip) behind paged_mqa_logits,
// paged_mqa_logits_visible (clean = false) and paged_mqa_topk_slots (hist:
// the per-row histograms to add to, or null).  Returns an SAI_* status.
// Not exported from the library.
__attribute__((visibility("hidden"))) int sai_paged_logits(const void* q_fp8, const float* weights, const void* kv_cache, int64_t num_blocks,
                     const int32_t* block_table, int64_t bt_stride, const int32_t* context_lens,
                     int32_t batch, int32_t next_n, float* logits, int64_t logits_stride,
                     int32_t* row_len_out, int32_t* row_req_out, bool clean, int32_t* hist,
                     hipStream_t stream);
