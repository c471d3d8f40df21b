"""Exact CPU oracle for the paged lightning-indexer path (TEST INFRASTRUCTURE ONLY).

This package is the plain, slow, obviously-correct definition that the HIP path
is checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path never
calls it and shares no code, tables or constants with it.

Every function cites the web page (title + section) whose statement it follows.
Pages:
  * vLLM PR #25869 "[Model] Support Deepseek V3.2", code-review comment on
    ``cp_gather_indexer_k_quant_cache`` (the preallocated rewrite)  -> cache
    layout and the paged->contiguous gather.
  * vLLM PR #36250 "[kernel] Fix FP8 paged MQA fallback for CUDA graph
    capture", Purpose and review thread -> the op ``fp8_paged_mqa_logits``,
    per-request context lengths, fp32 dequantisation, -inf "clean logits".
  * prhub summary of vLLM PR #47090 (FlashMLA FP8 KV cache + BF16 query),
    key source excerpt of ``_fused_norm_rope_kernel`` -> the amax/448 dynamic
    fp8 quantiser with its FLT_MIN floor, and the rotated pair (r1, r2)
    stored at positions 2i, 2i + 1 (the fused producers' rotation).
  * ROCm/ATOM PR #1094 "Support DSv3.2 with sglang-ATOM plugin and sglang sparse
    MLA", Technical Details -> request-local top-k -> global paged KV indices,
    the 2-D top-k index buffer.

Parity status: every function here is pinned by tests/test_oracle_pins.py.
"""
from .indexer import (  # noqa: F401
    BLOCK, HEADS, DIM, BLOCK_BYTES, FLT_MIN, INV_448,
    e4m3fn_table, fp8_encode, quantize_rows, quantize_q,
    rope_rotate, quantize_q_rope, k_rope_cache_write,
    k_cache_write, gather_indexer_k, paged_mqa_logits, mqa_logits, mqa_logits_chunked,
    topk_rows, topk_to_global_slots, decode_limits,
)
from . import mla  # noqa: F401,E402  (fp8 MLA cache and sparse MLA decode)
