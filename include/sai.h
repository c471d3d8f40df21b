/*
 * sai.h -- C ABI of the MI355X (gfx950) paged lightning-indexer library.
 *
 * The library implements DeepSeek-V3.2's sparse-attention indexer over a
 * paged fp8 K cache: the K-cache write, the query producer, fp8 paged MQA
 * logits, prefill logits over gathered K, per-row top-k and the
 * request-local -> global slot-id map.  Every call is a set of hand-written
 * HIP kernels launched on the caller's stream.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are DEVICE pointers owned by the caller; the library never
 *    allocates, frees or keeps them, and the entry points of this header
 *    hold no state between calls.  (The one piece of state in the library
 *    is the profiling aid of sai_profile.h: a per-thread event pair that the
 *    calling thread's next launch consumes.  It changes no result.)
 *    (Preallocated outputs written in place, as the review of
 *    cp_gather_indexer_k_quant_cache in vLLM PR #25869 asks for.)
 *  - Scalars are host values.  Validation reads host scalars only: no call
 *    reads device memory on the host, synchronises, or allocates, so every
 *    call can be captured into a hipGraph (the failure fixed by vLLM PR
 *    #36250 "[kernel] Fix FP8 paged MQA fallback for CUDA graph capture",
 *    Purpose, was a host read of a context length inside the op).
 *  - Device-side values outside their documented range (a context longer
 *    than the block table, a block id outside the pool, ...) are the
 *    caller's error; kernels bounds-check every address they form and never
 *    read or write outside the buffers described here; results for such
 *    entries are documented per call.
 *  - Return value: SAI_OK (0) or a negative SAI_E* code; nothing is launched
 *    when a code other than SAI_OK or SAI_ELAUNCH is returned.
 *  - Fixed shapes: 64 indexer heads, head_dim 128, 64-token cache blocks,
 *    top-k of at most 2048.
 *  - Alignment: q, K, the cache, the weights and the logits must be 16-byte
 *    aligned; strides are in elements.
 */
#ifndef SAI_H
#define SAI_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SAI_HEADS 64
#define SAI_HEAD_DIM 128
#define SAI_BLOCK_SIZE 64
/* one cache block: 64*128 fp8 e4m3fn values, then 64 fp32 scales */
#define SAI_BLOCK_BYTES 8448
#define SAI_TOPK_MAX 2048
#define SAI_NEXT_N_MAX 4

#define SAI_OK 0
#define SAI_EINVAL (-1)       /* null pointer, negative size, stride too small, misalignment */
#define SAI_EUNSUPPORTED (-2) /* shape outside what the kernels are built for */
#define SAI_EWORKSPACE (-3)   /* workspace missing or too small */
#define SAI_ELAUNCH (-4)      /* the HIP runtime rejected a launch */
#define SAI_ESCRATCH (-5)     /* needs more than the built-in scratch buffer (allocation-free entry) */

/* bytes of the built-in device scratch buffer of the allocation-free entry */
#define SAI_NOALLOC_SCRATCH_BYTES (16u << 20)

/* Human-readable name of a status code (static storage). */
const char* sai_status_string(int status);

/*
 * indexer_k_cache_write -- quantise K rows to fp8 and scatter them into the
 * paged indexer K cache.
 *
 * Quantiser (prhub summary of vLLM PR #47090, key source excerpt of
 * _fused_norm_rope_kernel, applied to one 128-value token row):
 *   amax = max_i |k_i|;  scale = max(amax * fl32(1/448), 1.1754944e-38);
 *   code_i = fp8_e4m3fn(k_i / scale), round to nearest even, saturating at
 *   +-448; all float32.
 * Layout (vLLM PR #25869, review of cp_gather_indexer_k_quant_cache): slot s
 * is token s % 64 of block s / 64; its codes go to bytes [t*128, t*128+128)
 * of the block and its scale to byte 8192 + 4t.
 *
 *   k_bf16        [n, k_row_stride] bf16, first 128 values of a row used
 *   k_row_stride  elements between rows (>= 128, multiple of 8)
 *   slot_mapping  [n] int64; a negative slot is skipped; a slot at or past
 *                 num_blocks*64 is skipped
 *   kv_cache      [num_blocks, 8448] uint8, written only at the owned bytes
 */
int indexer_k_cache_write(const void* k_bf16, int64_t k_row_stride,
                          const int64_t* slot_mapping, int64_t n,
                          void* kv_cache, int64_t num_blocks, hipStream_t stream);

/*
 * indexer_q_quant -- query producer: fp8 query codes with one scale per
 * token (over all 64x128 values), folded into that token's head weights.
 *
 * Same quantiser as indexer_k_cache_write over a whole token.  Because ReLU
 * is positively homogeneous, w*ReLU(s*x) = (w*s)*ReLU(x) for s > 0, so the
 * scale is folded: w_eff[r,h] = fl32(weights[r,h] * q_scale[r]).
 *
 *   q_bf16   [rows, 64, 128] bf16 (contiguous)
 *   weights  [rows, 64] fp32
 *   q_fp8    [rows, 64, 128] fp8 e4m3fn codes (output)
 *   w_eff    [rows, 64] fp32 (output)
 *   q_scale  [rows] fp32 (output, may be NULL)
 */
int indexer_q_quant(const void* q_bf16, const float* weights, int64_t rows,
                    void* q_fp8, float* w_eff, float* q_scale, hipStream_t stream);

/*
 * Fused producers.  The rotary embedding, the fp8 quantiser and the write
 * of its result in one kernel each: the indexer's analogue of the kernel
 * that rotates, quantises and stores MLA cache rows in one pass
 * (_fused_norm_rope_kernel, prhub summary of vLLM PR #47090, key source
 * excerpt).  The pages show that kernel storing the rotated pair r1, r2 at
 * positions 2i and 2i + 1 but print neither the rotation nor its tables;
 * the reading this library takes: for a row with token position
 * p = positions[t] and each pair i < rope_dim / 2,
 *   x[2i]     <- fl32(fl32(x[2i] * cos[p][i]) - fl32(x[2i+1] * sin[p][i]))
 *   x[2i + 1] <- fl32(fl32(x[2i+1] * cos[p][i]) + fl32(x[2i] * sin[p][i]))
 * in float32 without fused multiply-add (so the codes are reproducible bit
 * for bit); values at and past rope_dim are kept.  The quantiser then sees
 * the rotated values.
 *
 *   positions             int64, one per K token / query row (device)
 *   cos_table, sin_table  [table_rows, rope_dim / 2] fp32 (device); row p
 *                         holds position p's angles
 *   rope_dim              even, 0..128 (0: no rotation, the plain call)
 * A position outside [0, table_rows) gives NaN: NaN codes (0x7F) and a NaN
 * scale in the K cache, NaN codes, scale and folded weights for a query row
 * (never an out-of-bounds read).  SAI_EINVAL for an odd or out-of-range
 * rope_dim, a negative table_rows, or missing positions or tables when
 * rope_dim > 0.
 */

/*
 * indexer_k_rope_cache_write -- rotate the first rope_dim values of each K
 * row, then indexer_k_cache_write's quantiser and layout.  Other arguments,
 * skipping rules and errors as for indexer_k_cache_write.
 */
int indexer_k_rope_cache_write(const void* k_bf16, int64_t k_row_stride, const int64_t* positions,
                               const float* cos_table, const float* sin_table, int64_t table_rows,
                               int32_t rope_dim, const int64_t* slot_mapping, int64_t n,
                               void* kv_cache, int64_t num_blocks, hipStream_t stream);

/*
 * indexer_q_rope_quant -- rotate the first rope_dim values of every head of
 * each query row, then indexer_q_quant (one scale per token over all 64x128
 * rotated values, folded into that token's head weights).  Other arguments
 * and errors as for indexer_q_quant.
 */
int indexer_q_rope_quant(const void* q_bf16, const int64_t* positions, const float* cos_table,
                         const float* sin_table, int64_t table_rows, int32_t rope_dim,
                         const float* weights, int64_t rows, void* q_fp8, float* w_eff,
                         float* q_scale, hipStream_t stream);

/*
 * gather_indexer_k -- paged -> contiguous copy of K codes and scales for
 * prefill (vLLM PR #25869, review of cp_gather_indexer_k_quant_cache):
 * request b owns output rows [cu[b], cu[b+1]); token t < cu[b+1]-cu[b]
 * of request b is token t % 64 of block block_table[b*bt_stride + t/64].
 * Empty requests are skipped.  Rows not owned by any request (before cu[0]
 * or at/after cu[batch]) are left untouched.  A block id outside
 * [0, num_blocks) yields NaN codes (0x7F) and NaN scales for its tokens.
 *
 *   block_table   [batch, bt_stride] int32
 *   cu_seq_lens   [batch+1] int32, non-decreasing, cu[batch] <= total_tokens
 *   out_k_fp8     [total_tokens, 128] fp8 codes;  out_scale [total_tokens] fp32
 */
int gather_indexer_k(const void* kv_cache, int64_t num_blocks,
                     const int32_t* block_table, int64_t bt_stride,
                     const int32_t* cu_seq_lens, int32_t batch, int64_t total_tokens,
                     void* out_k_fp8, float* out_scale, hipStream_t stream);

/*
 * paged_mqa_logits -- fp8 paged MQA logits of the indexer (the op vLLM PR
 * #36250 names fp8_paged_mqa_logits; its formula, not printed on the pages,
 * is the DeepSeek-V3.2 lightning-indexer score):
 *
 *   logits[r, s] = k_scale[s] * sum_{h<64} w_eff[r, h] * max(q[r,h,:] . k[s,:], 0)
 *
 * for query row r = b*next_n + j (token j of request b) and request-local
 * key s < limit(r) = ctx_b - next_n + j + 1; columns limit(r) <= s <
 * logits_stride are -inf ("clean logits", vLLM PR #36250 review thread).
 * Every column of every row is written.  Dot products run on fp8 MFMA with
 * fp32 accumulation; the ReLU, head weights and scale are fp32 (fp32, not
 * fp16, dequantisation: vLLM PR #36250 review thread).
 *
 *   q_fp8         [batch*next_n, 64, 128] fp8 e4m3fn codes
 *   weights       [batch*next_n, 64] fp32 (w_eff of indexer_q_quant)
 *   kv_cache      [num_blocks, 8448] uint8 (layout of indexer_k_cache_write)
 *   block_table   [batch, bt_stride] int32, entry c = physical block of keys
 *                 [64c, 64c+64) of the request; only the first
 *                 ceil(ctx_b/64) entries are read
 *   context_lens  [batch] int32 (device); ctx_b is clamped to
 *                 [0, min(logits_stride, 64*bt_stride)]
 *   next_n        1..4 query tokens per request
 *   logits        [batch*next_n, logits_stride] fp32 (output)
 *   row_len_out   [batch*next_n] int32, limit(r) after clamping (may be NULL)
 *   row_req_out   [batch*next_n] int32, request b of row r (may be NULL)
 * A block id outside [0, num_blocks) makes that block's visible columns NaN.
 */
int paged_mqa_logits(const void* q_fp8, const float* weights, const void* kv_cache,
                     int64_t num_blocks, const int32_t* block_table, int64_t bt_stride,
                     const int32_t* context_lens, int32_t batch, int32_t next_n,
                     float* logits, int64_t logits_stride,
                     int32_t* row_len_out, int32_t* row_req_out, hipStream_t stream);

/*
 * paged_mqa_logits_visible -- paged_mqa_logits without the -inf fill: the
 * non-clean variant the review of vLLM PR #36250 sets beside "clean
 * logits", for a consumer that reads each row only up to its limit (the
 * top-k calls below do).  Columns of request b's key blocks,
 * [0, min(64*ceil(ctx_b/64), logits_stride)), are written exactly as
 * paged_mqa_logits writes them (-inf from the limit to the end of the last
 * block); later columns are left untouched.  Arguments and errors as for
 * paged_mqa_logits.
 */
int paged_mqa_logits_visible(const void* q_fp8, const float* weights, const void* kv_cache,
                             int64_t num_blocks, const int32_t* block_table, int64_t bt_stride,
                             const int32_t* context_lens, int32_t batch, int32_t next_n,
                             float* logits, int64_t logits_stride,
                             int32_t* row_len_out, int32_t* row_req_out, hipStream_t stream);

/*
 * mqa_logits -- prefill logits against contiguous K (the output of
 * gather_indexer_k).  Not one of the calls the pages name: the prefill path
 * scores gathered K (vLLM PR #25869, review of cp_gather_indexer_k_quant_cache;
 * ROCm/ATOM PR #1094, Technical Details, "sparse MLA prefill KV mapping"),
 * and no paged call takes contiguous K, so this entry is added.
 *
 * Same score as paged_mqa_logits.  Token p = cu[b] + i of request b sees the
 * request's keys 0..i (causal); column j is the request-local key index
 * (K row cu[b] + j).  Columns i+1 .. logits_stride-1 are -inf.  Rows of no
 * request are left untouched.
 *
 *   q_fp8 [total_tokens, 64, 128]; weights [total_tokens, 64];
 *   k_fp8 [total_tokens, 128]; k_scale [total_tokens];
 *   cu_seq_lens [batch+1] int32 (device), cu[batch] <= total_tokens;
 *   logits [total_tokens, logits_stride];
 *   row_len_out / row_req_out: [total_tokens] int32, i+1 and b (may be NULL)
 * A request longer than logits_stride is scored only on its first
 * logits_stride tokens and keys; its later rows are left untouched.
 */
int mqa_logits(const void* q_fp8, const float* weights, const void* k_fp8,
               const float* k_scale, const int32_t* cu_seq_lens, int32_t batch,
               int64_t total_tokens, float* logits, int64_t logits_stride,
               int32_t* row_len_out, int32_t* row_req_out, hipStream_t stream);

/*
 * mqa_logits_chunked -- prefill logits of a chunk of each request's queries
 * against the request's whole gathered context (chunked prefill, ragged
 * batches of such requests).  The pages fix the gather over cu_seq_lens
 * (vLLM PR #25869 review) and name the prefill KV mapping (ROCm/ATOM PR
 * #1094, Technical Details) without the causal rule; the rule taken is the
 * decode one: the queries are the last n_q = cu_q[b+1] - cu_q[b] of the
 * request's n_k = cu_k[b+1] - cu_k[b] tokens, so request-local query i sees
 * keys [0, n_k - n_q + i + 1) (none when that is <= 0).  Same score as
 * paged_mqa_logits; column j is the request-local key index (K row
 * cu_k[b] + j); columns past the limit are -inf.  A row whose limit exceeds
 * logits_stride is left untouched, as are rows of no request.  With
 * cu_k = cu_q this is mqa_logits.
 *
 *   q_fp8 [total_q, 64, 128]; weights [total_q, 64];
 *   k_fp8 [total_k, 128]; k_scale [total_k] (gather_indexer_k with cu_k);
 *   cu_seq_lens_q, cu_seq_lens_k [batch+1] int32 (device),
 *   cu_q[batch] <= total_q, cu_k[batch] <= total_k;
 *   logits [total_q, logits_stride];
 *   row_len_out / row_req_out: [total_q] int32, the row's limit and b (may be NULL)
 */
int mqa_logits_chunked(const void* q_fp8, const float* weights, const void* k_fp8,
                       const float* k_scale, const int32_t* cu_seq_lens_q,
                       const int32_t* cu_seq_lens_k, int32_t batch, int64_t total_q,
                       int64_t total_k, float* logits, int64_t logits_stride,
                       int32_t* row_len_out, int32_t* row_req_out, hipStream_t stream);

/*
 * topk_rows -- per-row top-k of the indexer logits (ROCm/ATOM PR #1094,
 * Technical Details: sparse top-k handed on in a 2-D index buffer).
 *
 * Row r ranks its columns s < n_r = clamp(row_len[r], 0, logits_stride) by
 * (larger logit, then lower index); -0.0 and +0.0 are equal.  It writes the
 * min(k, n_r) winners in ascending column order, then -1 up to k.  A NaN
 * (either sign, any payload) ranks below every number, -inf included, and
 * NaNs tie with each other, so they are taken only when a row has fewer
 * than k other columns, lowest index first (paged_mqa_logits writes NaN
 * for blocks outside the pool).
 *
 *   logits   [rows, logits_stride] fp32
 *   row_len  [rows] int32 (device)
 *   k        1..2048
 *   out_idx  [rows, k] int32 (output)
 *   workspace / workspace_bytes: scratch of at least
 *   topk_workspace_bytes(rows, logits_stride, k) bytes (may be NULL if that
 *   is 0); contents need no initialisation.  Rows of at most 16384
 *   columns, and of at most 65536 when rows < 512, are selected in one
 *   pass and need none.  Other rows wider than 16384 columns are cut into
 *   16384-column segments whose k winners (key and column) go to the
 *   workspace, 8 * rows * segments * k bytes, and are then merged; rows too
 *   wide for the merge (segments * k > 16384) need none.  A missing or
 *   short workspace returns SAI_EWORKSPACE and launches nothing.
 */
size_t topk_workspace_bytes(int32_t rows, int64_t logits_stride, int32_t k);
int topk_rows(const float* logits, int64_t logits_stride, const int32_t* row_len,
              int32_t rows, int32_t k, int32_t* out_idx,
              void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * topk_to_global_slots -- request-local top-k indices -> global paged KV
 * slot ids (ROCm/ATOM PR #1094, Technical Details):
 *   out[r, j] = block_table[b*bt_stride + i/64] * 64 + i % 64,
 * with i = topk_idx[r, j] and b = row_req[r].  -1 stays -1; so does an index
 * whose block-table entry is outside the table or negative, or a row whose
 * request is outside [0, batch).
 */
int topk_to_global_slots(const int32_t* topk_idx, const int32_t* row_req,
                         const int32_t* block_table, int64_t bt_stride, int32_t batch,
                         int32_t rows, int32_t k, int32_t* out_slots, hipStream_t stream);

/*
 * topk_rows_slots -- topk_rows and topk_to_global_slots in one call (ROCm/ATOM
 * PR #1094, Technical Details: the selected request-local indices and the
 * global slot ids of the sparse-attention cache they address).
 *
 * out_idx is what topk_rows writes and out_slots what topk_to_global_slots
 * writes for that out_idx; the slot ids are produced by the selection
 * kernels as they write each index, so the decode step needs no separate
 * slot pass.  Arguments as for those two calls: logits [rows, logits_stride],
 * row_len and row_req [rows], block_table [batch, bt_stride], out_idx and
 * out_slots [rows, k], workspace of topk_workspace_bytes(rows,
 * logits_stride, k) bytes.  Errors as for topk_rows, plus SAI_EINVAL for a
 * null row_req, block_table or out_slots when rows > 0.
 */
int topk_rows_slots(const float* logits, int64_t logits_stride, const int32_t* row_len,
                    const int32_t* row_req, const int32_t* block_table, int64_t bt_stride,
                    int32_t batch, int32_t rows, int32_t k, int32_t* out_idx, int32_t* out_slots,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * paged_mqa_topk_slots -- one decode step of the indexer: paged_mqa_logits
 * followed by topk_rows_slots, with the logits kernel handing the selection
 * each row's histogram of its logits (the fused logits -> top-k step beside
 * the "clean logits" of vLLM PR #36250, review thread: the selection starts
 * at the bin that holds the k-th largest logit instead of finding it from a
 * sample of the logits).
 *
 * Outputs are exactly those of the two calls: logits, row_len_out and
 * row_req_out as paged_mqa_logits writes them (both required here), out_idx
 * and out_slots as topk_rows_slots writes them from those logits (k indices
 * per row).  Arguments as for the two calls, plus
 *   hist        [rows, 1024] int32 device buffer, rows = batch * next_n, or
 *               NULL.  It must be all zero before the first call; every call
 *               that uses it adds the counts in the logits kernel and sets
 *               them back to zero in the selection, so it is zero again
 *               after the call.  Used when paged_mqa_topk_hist_bytes(rows,
 *               logits_stride) is non-zero (rows of at most 16384 columns,
 *               fewer than 512 rows); otherwise, and when NULL, the step runs
 *               the two calls unchanged and leaves hist untouched.
 *   hist_bytes  its size; SAI_EWORKSPACE if it is used and smaller than
 *               paged_mqa_topk_hist_bytes(rows, logits_stride).
 *   workspace   as for topk_rows_slots (needed only for rows cut into
 *               segments, see topk_workspace_bytes; those never use hist).
 * Errors: those of both calls, all checked before anything is launched.
 * A histogram that is not zero before the call changes no result (the
 * selection checks its bound as it checks a sampled one), only the time.
 * On 64 rows of at most 16384 keys the step measured 2 us slower than the
 * two plain calls: counting adds more to the logits kernel than starting
 * from the histogram saves in the selection.
 */
int paged_mqa_topk_slots(const void* q_fp8, const float* weights, const void* kv_cache,
                         int64_t num_blocks, const int32_t* block_table, int64_t bt_stride,
                         const int32_t* context_lens, int32_t batch, int32_t next_n, float* logits,
                         int64_t logits_stride, int32_t* row_len_out, int32_t* row_req_out, int32_t k,
                         int32_t* out_idx, int32_t* out_slots, int32_t* hist, size_t hist_bytes,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of paged_mqa_topk_slots' hist for this shape; 0 when the shape
 * does not use one (rows <= 0, logits_stride <= 0 or > 16384, rows >= 512). */
size_t paged_mqa_topk_hist_bytes(int32_t rows, int64_t logits_stride);

/*
 * topk_rows_slots_noalloc -- topk_rows_slots for callers that cannot
 * allocate device memory (code under hipGraph capture, tight serving loops,
 * harnesses that forbid hipMalloc): no workspace argument, and no call to
 * hipMalloc, hipFree or any allocating routine.
 *
 * Same arguments (minus the workspace), outputs and errors as
 * topk_rows_slots.  Rows cut into segments keep their segment candidates
 * in a buffer built into the library: a file-scope device array of
 * SAI_NOALLOC_SCRATCH_BYTES (16 MiB) that each device holds from the
 * library's load until the process ends.  A problem whose
 * topk_workspace_bytes(rows, logits_stride, k) exceeds that returns
 * SAI_ESCRATCH and launches nothing (e.g. 128 rows of 131072 columns at
 * k = 2048 fit exactly; 129 do not).  The first call on a device resolves
 * that device's array address (hipGetSymbolAddress, with the stream's
 * device made current for the lookup); the address is then kept.  Every
 * call on a device shares its one array, so calls that overlap on the same
 * device (other streams, other threads) race and must be serialised by the
 * caller; nothing needs clearing between calls.
 */
int topk_rows_slots_noalloc(const float* logits, int64_t logits_stride, const int32_t* row_len,
                            const int32_t* row_req, const int32_t* block_table, int64_t bt_stride,
                            int32_t batch, int32_t rows, int32_t k, int32_t* out_idx,
                            int32_t* out_slots, hipStream_t stream);

/*
 * mla_cache_write -- write tokens into the fp8 MLA cache that sparse MLA
 * decode reads ("fp8_ds_mla" layout; prhub summary of vLLM PR #47090, key
 * source excerpt of _fused_norm_rope_kernel, MLA_CACHE_DS_MLA branch).
 *
 * Entry of 656 bytes per token: bytes [0, 512) the latent values as fp8
 * e4m3fn codes, quantised per 128-value tile with the indexer's rule
 * (amax = max |tile|, scale = max(amax * fl32(1/448), 1.1754944e-38),
 * code = fp8(value / scale), round to nearest even, saturating, float32);
 * bytes [512, 528) the 4 tile scales (fp32); bytes [528, 656) the 64 RoPE
 * values, copied as bf16.  Token slot s is entry s % block_size of block
 * s / block_size; entries are 656 bytes apart, blocks block_size*656 bytes.
 * The RMS norm and the rotation that produce these values are the caller's.
 *
 *   kv_bf16        [n, kv_row_stride] bf16, first 512 values of a row used
 *                  (kv_row_stride >= 512, multiple of 8; 16-byte aligned base)
 *   kpe_bf16       [n, kpe_row_stride] bf16, first 64 values of a row used
 *                  (kpe_row_stride >= 64 and even; 4-byte aligned base)
 *   slot_mapping   [n] int64; a negative slot, or one at or past
 *                  num_blocks*block_size, is skipped
 *   cache          [num_blocks, block_size, 656] uint8 (16-byte aligned),
 *                  written only at the entries of the written slots
 */
int mla_cache_write(const void* kv_bf16, int64_t kv_row_stride, const void* kpe_bf16,
                    int64_t kpe_row_stride, const int64_t* slot_mapping, int64_t n, void* cache,
                    int64_t num_blocks, int32_t block_size, hipStream_t stream);

/*
 * sparse_mla_workspace_bytes -- bytes of device workspace sparse_mla_decode
 * needs for (rows, heads, k); 0 when it runs in one pass (or for arguments it
 * would reject).  The value depends only on the three arguments.
 */
size_t sparse_mla_workspace_bytes(int32_t rows, int32_t heads, int32_t k);

/*
 * sparse_mla_decode -- sparse MLA decode over the fp8 MLA cache: the
 * attention that consumes the global slot ids the indexer selects (ROCm/ATOM
 * PR #1094, Technical Details; cache layout as for mla_cache_write).  The
 * pages name this step without printing its arithmetic; this is the plain
 * absorbed-MLA reading.  For query row t, head h and the row's valid slots j
 * (0 <= id < num_blocks*block_size; -1 padding and out-of-range ids are
 * skipped, a repeated id counts each time it appears):
 *   s_j = sm_scale * (q_nope[t,h] . kv_j + q_pe[t,h] . kpe_j)
 *   out[t,h] = sum_j softmax(s)_j * kv_j,   lse[t,h] = ln sum_j exp(s_j)
 * with kv_j = code * tile scale (the 512 latent values) and kpe_j the stored
 * 64 RoPE values.  A row with no valid slot gives out = 0, lse = -inf.
 * Scores are accumulated in fp32 from exactly converted bf16 operands;
 * softmax weights times the tile scale are rounded to bf16 for the P.V
 * product (fp32 accumulation).
 *
 *   q_nope     [rows, heads, 512] bf16, contiguous, 16-byte aligned
 *   q_pe       [rows, heads, 64] bf16, contiguous, 16-byte aligned
 *   heads      a multiple of 16, at most 128
 *   cache      [num_blocks, block_size, 656] uint8, 16-byte aligned,
 *              num_blocks >= 1
 *   slots      [rows, k] int32 global slot ids (k >= 0; k = 0 gives empty rows)
 *   out        [rows, heads, 512] fp32, 16-byte aligned, fully written
 *   lse        [rows, heads] fp32 or NULL, fully written when given
 *   workspace  sparse_mla_workspace_bytes(rows, heads, k) bytes of device
 *              memory (16-byte aligned), NULL when that is 0; owned by the
 *              caller, contents need no initialisation and are scratch
 *              afterwards; calls sharing one workspace must not overlap
 * SAI_EUNSUPPORTED for heads outside the supported set; SAI_EWORKSPACE for a
 * missing or short workspace.  Two kernels when the workspace is used, one
 * otherwise, on `stream`.
 */
int sparse_mla_decode(const void* q_nope, const void* q_pe, int32_t rows, int32_t heads,
                      const void* cache, int64_t num_blocks, int32_t block_size,
                      const int32_t* slots, int32_t k, float sm_scale, float* out, float* lse,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SAI_H */
