"""MI355X (gfx950) paged lightning indexer for DeepSeek-V3.2 sparse attention.

The compute lives in libsai.so (hand-written HIP kernels behind the C ABI of
include/sai.h); ``binding`` is its thin ctypes layer and ``synth`` draws the
seeded synthetic workloads.  Importing this package does not load the
library; the first call does, and raises if it has not been built.
"""
__all__ = [
    "indexer_k_cache_write", "indexer_q_quant", "gather_indexer_k", "paged_mqa_logits",
    "mqa_logits", "mqa_logits_chunked", "topk_rows", "topk_workspace_bytes", "topk_to_global_slots", "decode_indexer",
    "mla_cache_write", "sparse_mla_decode", "sparse_mla_workspace_bytes",
]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
