"""ctypes binding of libsai.so (argument marshalling only).

Each function has the name of the C entry point it calls (include/sai.h),
checks dtypes, devices, shapes and contiguity of the torch tensors, passes
their device pointers and the current HIP stream, and raises on a non-zero
status.  Every step of the indexer runs in the library's HIP kernels; torch
only provides device memory and the stream.  There is no fallback: without
the built library every call raises.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsai.so")

HEADS = 64
DIM = 128
BLOCK = 64
BLOCK_BYTES = 8448
TOPK_MAX = 2048

_c_void_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64

# name -> argtypes (restype int unless listed in _RESTYPE)
SIGNATURES = {
    "sai_status_string": [ctypes.c_int],
    "sai_time_next_launch": [_c_void_p, _c_void_p],
    "sai_time_span": [_c_void_p, _c_void_p],
    "indexer_k_cache_write": [_c_void_p, _i64, _c_void_p, _i64, _c_void_p, _i64, _c_void_p],
    "indexer_q_quant": [_c_void_p, _c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p, _c_void_p],
    "indexer_k_rope_cache_write": [_c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p, _i64, _i32,
                                   _c_void_p, _i64, _c_void_p, _i64, _c_void_p],
    "indexer_q_rope_quant": [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i32, _c_void_p, _i64,
                             _c_void_p, _c_void_p, _c_void_p, _c_void_p],
    "gather_indexer_k": [_c_void_p, _i64, _c_void_p, _i64, _c_void_p, _i32, _i64, _c_void_p,
                         _c_void_p, _c_void_p],
    "paged_mqa_logits": [_c_void_p, _c_void_p, _c_void_p, _i64, _c_void_p, _i64, _c_void_p, _i32,
                         _i32, _c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p],
    "paged_mqa_logits_visible": [_c_void_p, _c_void_p, _c_void_p, _i64, _c_void_p, _i64, _c_void_p, _i32,
                                 _i32, _c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p],
    "mqa_logits": [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i64, _c_void_p,
                   _i64, _c_void_p, _c_void_p, _c_void_p],
    "mqa_logits_chunked": [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32,
                           _i64, _i64, _c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p],
    "topk_workspace_bytes": [_i32, _i64, _i32],
    "topk_rows": [_c_void_p, _i64, _c_void_p, _i32, _i32, _c_void_p, _c_void_p, ctypes.c_size_t,
                  _c_void_p],
    "topk_to_global_slots": [_c_void_p, _c_void_p, _c_void_p, _i64, _i32, _i32, _i32, _c_void_p,
                             _c_void_p],
    "topk_rows_slots": [_c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p, _i64, _i32, _i32, _i32,
                        _c_void_p, _c_void_p, _c_void_p, ctypes.c_size_t, _c_void_p],
    "topk_rows_slots_noalloc": [_c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p, _i64, _i32, _i32,
                                _i32, _c_void_p, _c_void_p, _c_void_p],
    "mla_cache_write": [_c_void_p, _i64, _c_void_p, _i64, _c_void_p, _i64, _c_void_p, _i64, _i32,
                        _c_void_p],
    "sparse_mla_workspace_bytes": [_i32, _i32, _i32],
    "paged_mqa_topk_hist_bytes": [_i32, _i64],
    "paged_mqa_topk_slots": [_c_void_p, _c_void_p, _c_void_p, _i64, _c_void_p, _i64, _c_void_p, _i32, _i32,
                             _c_void_p, _i64, _c_void_p, _c_void_p, _i32, _c_void_p, _c_void_p, _c_void_p,
                             ctypes.c_size_t, _c_void_p, ctypes.c_size_t, _c_void_p],
    "sparse_mla_decode": [_c_void_p, _c_void_p, _i32, _i32, _c_void_p, _i64, _i32, _c_void_p, _i32,
                          ctypes.c_float, _c_void_p, _c_void_p, _c_void_p, ctypes.c_size_t, _c_void_p],
}
_RESTYPE = {"sai_status_string": ctypes.c_char_p, "topk_workspace_bytes": ctypes.c_size_t,
            "sparse_mla_workspace_bytes": ctypes.c_size_t, "paged_mqa_topk_hist_bytes": ctypes.c_size_t}

_lib = None


def load():
    """Load libsai.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m sparse_attention_indexer_paged_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, args in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = _RESTYPE.get(name, ctypes.c_int)
        _lib = lib
    return _lib


def status_string(code):
    return load().sai_status_string(code).decode()


def _check(code, name):
    if code != 0:
        raise RuntimeError(f"{name} failed: {status_string(code)} ({code})")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t, dtype, name, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_rows(t, dtype, name):
    """A 2-D GPU tensor whose rows may be strided but whose elements within a
    row are contiguous (the C ABI takes the row stride)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be 2-D with contiguous rows")


def _out(t, dtype, name, shape):
    """Caller-provided outputs: the kernels write every element of ``shape``
    (row pitch = the row length), so the tensor must be exactly that."""
    _need(t, dtype, name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


# ---------------------------------------------------------------- calls
def indexer_k_cache_write(k_bf16, slot_mapping, kv_cache):
    """Quantise K rows [n, 128] bf16 into the paged cache [num_blocks, 8448] u8 in place."""
    _need(k_bf16, torch.bfloat16, "k_bf16", 2)
    _need(slot_mapping, torch.int64, "slot_mapping", 1)
    _need(kv_cache, torch.uint8, "kv_cache", 2)
    if k_bf16.shape[1] != DIM or kv_cache.shape[1] != BLOCK_BYTES:
        raise ValueError("k_bf16 must be [n,128] and kv_cache [num_blocks, 8448]")
    if slot_mapping.shape[0] != k_bf16.shape[0]:
        raise ValueError("slot_mapping must have one entry per K row")
    if k_bf16.shape[0] == 0:
        return kv_cache
    _check(load().indexer_k_cache_write(_ptr(k_bf16), k_bf16.stride(0), _ptr(slot_mapping),
                                        k_bf16.shape[0], _ptr(kv_cache), kv_cache.shape[0],
                                        _stream()), "indexer_k_cache_write")
    return kv_cache


def _rope_tables(cos_table, sin_table, rope_dim):
    _need(cos_table, torch.float32, "cos_table", 2)
    _need(sin_table, torch.float32, "sin_table", 2)
    if cos_table.shape != sin_table.shape:
        raise ValueError("cos_table and sin_table must have the same shape [positions, rope_dim/2]")
    rope_dim = 2 * cos_table.shape[1] if rope_dim is None else int(rope_dim)
    if rope_dim > 2 * cos_table.shape[1]:
        raise ValueError("the tables hold fewer than rope_dim/2 columns")
    if cos_table.shape[1] != rope_dim // 2:
        raise ValueError("the kernels index the tables with rope_dim/2 columns per row")
    return rope_dim


def indexer_k_rope_cache_write(k_bf16, positions, cos_table, sin_table, slot_mapping, kv_cache,
                               rope_dim=None):
    """Fused K producer: rotate the first rope_dim values of each K row [n, 128]
    bf16 by its position (positions [n] int64; cos/sin tables [P, rope_dim/2]
    fp32), quantise to fp8 and write into the paged cache in place.  K rows
    may be strided (the C call takes the row stride)."""
    _need_rows(k_bf16, torch.bfloat16, "k_bf16")
    _need(positions, torch.int64, "positions", 1)
    _need(slot_mapping, torch.int64, "slot_mapping", 1)
    _need(kv_cache, torch.uint8, "kv_cache", 2)
    rope_dim = _rope_tables(cos_table, sin_table, rope_dim)
    n = k_bf16.shape[0]
    if k_bf16.shape[1] != DIM or kv_cache.shape[1] != BLOCK_BYTES:
        raise ValueError("k_bf16 must be [n,128] and kv_cache [num_blocks, 8448]")
    if slot_mapping.shape[0] != n or positions.shape[0] != n:
        raise ValueError("slot_mapping and positions need one entry per K row")
    if n == 0:
        return kv_cache
    _check(load().indexer_k_rope_cache_write(_ptr(k_bf16), k_bf16.stride(0), _ptr(positions),
                                             _ptr(cos_table), _ptr(sin_table), cos_table.shape[0],
                                             rope_dim, _ptr(slot_mapping), n, _ptr(kv_cache),
                                             kv_cache.shape[0], _stream()),
           "indexer_k_rope_cache_write")
    return kv_cache


def indexer_q_rope_quant(q_bf16, positions, cos_table, sin_table, weights, rope_dim=None, q_fp8=None,
                         w_eff=None, q_scale=None):
    """Fused query producer: rotate the first rope_dim values of every head of
    each query row q [T,64,128] bf16 by its position (positions [T] int64),
    then quantise as indexer_q_quant -> (q_fp8, w_eff, q_scale)."""
    _need(q_bf16, torch.bfloat16, "q_bf16", 3)
    _need(positions, torch.int64, "positions", 1)
    _need(weights, torch.float32, "weights", 2)
    rope_dim = _rope_tables(cos_table, sin_table, rope_dim)
    T = q_bf16.shape[0]
    if tuple(q_bf16.shape[1:]) != (HEADS, DIM) or tuple(weights.shape) != (T, HEADS):
        raise ValueError("q_bf16 must be [T,64,128] and weights [T,64]")
    if positions.shape[0] != T:
        raise ValueError("positions needs one entry per query row")
    dev = q_bf16.device
    q_fp8 = torch.empty((T, HEADS, DIM), dtype=torch.uint8, device=dev) if q_fp8 is None else q_fp8
    w_eff = torch.empty((T, HEADS), dtype=torch.float32, device=dev) if w_eff is None else w_eff
    q_scale = torch.empty((T,), dtype=torch.float32, device=dev) if q_scale is None else q_scale
    _out(q_fp8, torch.uint8, "q_fp8", (T, HEADS, DIM))
    _out(w_eff, torch.float32, "w_eff", (T, HEADS))
    _out(q_scale, torch.float32, "q_scale", (T,))
    _check(load().indexer_q_rope_quant(_ptr(q_bf16), _ptr(positions), _ptr(cos_table), _ptr(sin_table),
                                       cos_table.shape[0], rope_dim, _ptr(weights), T, _ptr(q_fp8),
                                       _ptr(w_eff), _ptr(q_scale), _stream()), "indexer_q_rope_quant")
    return q_fp8, w_eff, q_scale


MLA_ENTRY_BYTES = 656


def mla_cache_write(kv_bf16, kpe_bf16, slot_mapping, cache):
    """Write latent rows kv [n, 512] bf16 and RoPE rows kpe [n, 64] bf16 into the
    fp8 MLA cache [num_blocks, block_size, 656] u8 in place."""
    _need_rows(kv_bf16, torch.bfloat16, "kv_bf16")
    _need_rows(kpe_bf16, torch.bfloat16, "kpe_bf16")
    _need(slot_mapping, torch.int64, "slot_mapping", 1)
    _need(cache, torch.uint8, "cache", 3)
    n = kv_bf16.shape[0]
    if kv_bf16.shape[1] < 512 or kpe_bf16.shape[1] < 64 or cache.shape[2] != MLA_ENTRY_BYTES:
        raise ValueError("kv_bf16 must be [n,>=512], kpe_bf16 [n,>=64], cache [blocks, block_size, 656]")
    if kpe_bf16.shape[0] != n or slot_mapping.shape[0] != n:
        raise ValueError("kpe_bf16 and slot_mapping need one row per kv row")
    if n == 0:
        return cache
    _check(load().mla_cache_write(_ptr(kv_bf16), kv_bf16.stride(0), _ptr(kpe_bf16), kpe_bf16.stride(0),
                                  _ptr(slot_mapping), n, _ptr(cache), cache.shape[0], cache.shape[1],
                                  _stream()), "mla_cache_write")
    return cache


def sparse_mla_workspace_bytes(rows, heads, k):
    return int(load().sparse_mla_workspace_bytes(rows, heads, k))


def sparse_mla_decode(q_nope, q_pe, cache, slots, sm_scale, out=None, lse=None, workspace=None):
    """Sparse MLA decode: q_nope [T,H,512] bf16, q_pe [T,H,64] bf16, cache
    [num_blocks, block_size, 656] u8, slots [T,K] int32 global slot ids (-1 or
    out-of-range ids skipped) -> (out [T,H,512] fp32, lse [T,H] fp32)."""
    _need(q_nope, torch.bfloat16, "q_nope", 3)
    _need(q_pe, torch.bfloat16, "q_pe", 3)
    _need(cache, torch.uint8, "cache", 3)
    _need(slots, torch.int32, "slots", 2)
    T, H = q_nope.shape[:2]
    K = slots.shape[1]
    if q_nope.shape[2] != 512 or tuple(q_pe.shape) != (T, H, 64) or cache.shape[2] != MLA_ENTRY_BYTES:
        raise ValueError("q_nope must be [T,H,512], q_pe [T,H,64], cache [blocks, block_size, 656]")
    if slots.shape[0] != T:
        raise ValueError("slots needs one row per query row")
    dev = q_nope.device
    out = torch.empty((T, H, 512), dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty((T, H), dtype=torch.float32, device=dev) if lse is None else lse
    _out(out, torch.float32, "out", (T, H, 512))
    _out(lse, torch.float32, "lse", (T, H))
    if T == 0:
        return out, lse
    ws_bytes = sparse_mla_workspace_bytes(T, H, K)
    if workspace is None and ws_bytes:
        workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().sparse_mla_decode(_ptr(q_nope), _ptr(q_pe), T, H, _ptr(cache), cache.shape[0],
                                    cache.shape[1], _ptr(slots), K, float(sm_scale), _ptr(out),
                                    _ptr(lse), _ptr(workspace), ws_len, _stream()),
           "sparse_mla_decode")
    return out, lse


def indexer_q_quant(q_bf16, weights, q_fp8=None, w_eff=None, q_scale=None):
    """q [T,64,128] bf16, weights [T,64] fp32 -> (q_fp8 u8 [T,64,128], w_eff [T,64], q_scale [T])."""
    _need(q_bf16, torch.bfloat16, "q_bf16", 3)
    _need(weights, torch.float32, "weights", 2)
    T = q_bf16.shape[0]
    if tuple(q_bf16.shape[1:]) != (HEADS, DIM) or tuple(weights.shape) != (T, HEADS):
        raise ValueError("q_bf16 must be [T,64,128] and weights [T,64]")
    dev = q_bf16.device
    q_fp8 = torch.empty((T, HEADS, DIM), dtype=torch.uint8, device=dev) if q_fp8 is None else q_fp8
    w_eff = torch.empty((T, HEADS), dtype=torch.float32, device=dev) if w_eff is None else w_eff
    q_scale = torch.empty((T,), dtype=torch.float32, device=dev) if q_scale is None else q_scale
    _out(q_fp8, torch.uint8, "q_fp8", (T, HEADS, DIM))
    _out(w_eff, torch.float32, "w_eff", (T, HEADS))
    _out(q_scale, torch.float32, "q_scale", (T,))
    _check(load().indexer_q_quant(_ptr(q_bf16), _ptr(weights), T, _ptr(q_fp8), _ptr(w_eff),
                                  _ptr(q_scale), _stream()), "indexer_q_quant")
    return q_fp8, w_eff, q_scale


def gather_indexer_k(kv_cache, block_table, cu_seq_lens, total_tokens, out_k=None, out_scale=None):
    """Paged -> contiguous K for prefill: (k_fp8 u8 [total,128], k_scale f32 [total])."""
    _need(kv_cache, torch.uint8, "kv_cache", 2)
    _need(block_table, torch.int32, "block_table", 2)
    _need(cu_seq_lens, torch.int32, "cu_seq_lens", 1)
    batch = cu_seq_lens.shape[0] - 1
    if block_table.shape[0] < batch:
        raise ValueError("block_table has fewer rows than requests")
    dev = kv_cache.device
    out_k = torch.empty((total_tokens, DIM), dtype=torch.uint8, device=dev) if out_k is None else out_k
    out_scale = torch.empty((total_tokens,), dtype=torch.float32, device=dev) if out_scale is None else out_scale
    _out(out_k, torch.uint8, "out_k", (total_tokens, DIM))
    _out(out_scale, torch.float32, "out_scale", (total_tokens,))
    _check(load().gather_indexer_k(_ptr(kv_cache), kv_cache.shape[0], _ptr(block_table),
                                   block_table.stride(0), _ptr(cu_seq_lens), batch, total_tokens,
                                   _ptr(out_k), _ptr(out_scale), _stream()), "gather_indexer_k")
    return out_k, out_scale


def paged_mqa_logits(q_fp8, weights, kv_cache, block_table, context_lens, width=None,
                     logits=None, row_len=None, row_req=None, clean=True):
    """Decode logits.  q_fp8 u8 [B, next_n, 64, 128]; weights f32 [B*next_n, 64];
    block_table i32 [B, bt_width]; context_lens i32 [B].  Row width defaults to
    bt_width*64.  Returns (logits f32 [B*next_n, width], row_len i32, row_req i32).
    clean=False calls paged_mqa_logits_visible (columns past each request's
    last key block are left as they were)."""
    _need(q_fp8, torch.uint8, "q_fp8", 4)
    _need(weights, torch.float32, "weights", 2)
    _need(kv_cache, torch.uint8, "kv_cache", 2)
    _need(block_table, torch.int32, "block_table", 2)
    _need(context_lens, torch.int32, "context_lens", 1)
    B, next_n = q_fp8.shape[0], q_fp8.shape[1]
    if tuple(q_fp8.shape[2:]) != (HEADS, DIM) or tuple(weights.shape) != (B * next_n, HEADS):
        raise ValueError("q_fp8 must be [B,next_n,64,128] and weights [B*next_n,64]")
    if context_lens.shape[0] != B or block_table.shape[0] != B:
        raise ValueError("context_lens and block_table need one row per request")
    rows = B * next_n
    width = block_table.shape[1] * BLOCK if width is None else width
    dev = q_fp8.device
    logits = torch.empty((rows, width), dtype=torch.float32, device=dev) if logits is None else logits
    row_len = torch.empty((rows,), dtype=torch.int32, device=dev) if row_len is None else row_len
    row_req = torch.empty((rows,), dtype=torch.int32, device=dev) if row_req is None else row_req
    _out(logits, torch.float32, "logits", (rows, width))
    _out(row_len, torch.int32, "row_len", (rows,))
    _out(row_req, torch.int32, "row_req", (rows,))
    name = "paged_mqa_logits" if clean else "paged_mqa_logits_visible"
    _check(getattr(load(), name)(_ptr(q_fp8), _ptr(weights), _ptr(kv_cache), kv_cache.shape[0],
                                 _ptr(block_table), block_table.stride(0), _ptr(context_lens),
                                 B, next_n, _ptr(logits), logits.stride(0), _ptr(row_len),
                                 _ptr(row_req), _stream()), name)
    return logits, row_len, row_req


def mqa_logits(q_fp8, weights, k_fp8, k_scale, cu_seq_lens, width, logits=None, row_len=None,
               row_req=None):
    """Prefill logits over contiguous K.  q_fp8 u8 [total,64,128]; weights f32
    [total,64]; k_fp8 u8 [total,128]; k_scale f32 [total]; cu_seq_lens i32 [B+1]."""
    _need(q_fp8, torch.uint8, "q_fp8", 3)
    _need(weights, torch.float32, "weights", 2)
    _need(k_fp8, torch.uint8, "k_fp8", 2)
    _need(k_scale, torch.float32, "k_scale", 1)
    _need(cu_seq_lens, torch.int32, "cu_seq_lens", 1)
    total = q_fp8.shape[0]
    if k_fp8.shape[0] != total or k_scale.shape[0] != total or weights.shape[0] != total:
        raise ValueError("q, weights, k and k_scale need one row per token")
    batch = cu_seq_lens.shape[0] - 1
    dev = q_fp8.device
    logits = torch.empty((total, width), dtype=torch.float32, device=dev) if logits is None else logits
    row_len = torch.empty((total,), dtype=torch.int32, device=dev) if row_len is None else row_len
    row_req = torch.empty((total,), dtype=torch.int32, device=dev) if row_req is None else row_req
    _out(logits, torch.float32, "logits", (total, width))
    _out(row_len, torch.int32, "row_len", (total,))
    _out(row_req, torch.int32, "row_req", (total,))
    _check(load().mqa_logits(_ptr(q_fp8), _ptr(weights), _ptr(k_fp8), _ptr(k_scale),
                             _ptr(cu_seq_lens), batch, total, _ptr(logits), logits.stride(0),
                             _ptr(row_len), _ptr(row_req), _stream()), "mqa_logits")
    return logits, row_len, row_req


def mqa_logits_chunked(q_fp8, weights, k_fp8, k_scale, cu_q, cu_k, width, logits=None, row_len=None,
                       row_req=None):
    """Chunked-prefill logits: request b's queries (rows cu_q[b]..cu_q[b+1]) are
    the last tokens of its context (K rows cu_k[b]..cu_k[b+1]).  q_fp8 u8
    [total_q,64,128]; weights f32 [total_q,64]; k_fp8 u8 [total_k,128]; k_scale
    f32 [total_k]; cu_q, cu_k i32 [B+1]."""
    _need(q_fp8, torch.uint8, "q_fp8", 3)
    _need(weights, torch.float32, "weights", 2)
    _need(k_fp8, torch.uint8, "k_fp8", 2)
    _need(k_scale, torch.float32, "k_scale", 1)
    _need(cu_q, torch.int32, "cu_q", 1)
    _need(cu_k, torch.int32, "cu_k", 1)
    total_q, total_k = q_fp8.shape[0], k_fp8.shape[0]
    if weights.shape[0] != total_q or k_scale.shape[0] != total_k:
        raise ValueError("weights need one row per query, k_scale one per key")
    if cu_q.shape[0] != cu_k.shape[0]:
        raise ValueError("cu_q and cu_k need one entry per request plus one")
    batch = cu_q.shape[0] - 1
    dev = q_fp8.device
    logits = torch.empty((total_q, width), dtype=torch.float32, device=dev) if logits is None else logits
    row_len = torch.empty((total_q,), dtype=torch.int32, device=dev) if row_len is None else row_len
    row_req = torch.empty((total_q,), dtype=torch.int32, device=dev) if row_req is None else row_req
    _out(logits, torch.float32, "logits", (total_q, width))
    _out(row_len, torch.int32, "row_len", (total_q,))
    _out(row_req, torch.int32, "row_req", (total_q,))
    _check(load().mqa_logits_chunked(_ptr(q_fp8), _ptr(weights), _ptr(k_fp8), _ptr(k_scale), _ptr(cu_q),
                                     _ptr(cu_k), batch, total_q, total_k, _ptr(logits), logits.stride(0),
                                     _ptr(row_len), _ptr(row_req), _stream()), "mqa_logits_chunked")
    return logits, row_len, row_req


def topk_workspace_bytes(rows, logits_stride, k):
    return int(load().topk_workspace_bytes(rows, logits_stride, k))


def topk_rows(logits, row_len, k=TOPK_MAX, out=None, workspace=None):
    """Top-k column indices per row (ascending, -1 padded): int32 [rows, k]."""
    _need(logits, torch.float32, "logits", 2)
    _need(row_len, torch.int32, "row_len", 1)
    rows = logits.shape[0]
    if row_len.shape[0] != rows:
        raise ValueError("row_len needs one entry per row")
    dev = logits.device
    out = torch.empty((rows, k), dtype=torch.int32, device=dev) if out is None else out
    _out(out, torch.int32, "out", (rows, k))
    ws_bytes = topk_workspace_bytes(rows, logits.stride(0), k)
    if ws_bytes and workspace is None:
        workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
    _check(load().topk_rows(_ptr(logits), logits.stride(0), _ptr(row_len), rows, k, _ptr(out),
                            _ptr(workspace), workspace.numel() if workspace is not None else 0,
                            _stream()), "topk_rows")
    return out


def topk_to_global_slots(topk_idx, row_req, block_table, out=None):
    """Request-local top-k indices -> global paged KV slot ids (int32, -1 kept)."""
    _need(topk_idx, torch.int32, "topk_idx", 2)
    _need(row_req, torch.int32, "row_req", 1)
    _need(block_table, torch.int32, "block_table", 2)
    rows, k = topk_idx.shape
    out = torch.empty_like(topk_idx) if out is None else out
    _out(out, torch.int32, "out", (rows, k))
    _check(load().topk_to_global_slots(_ptr(topk_idx), _ptr(row_req), _ptr(block_table),
                                       block_table.stride(0), block_table.shape[0], rows, k,
                                       _ptr(out), _stream()), "topk_to_global_slots")
    return out


def topk_rows_slots(logits, row_len, row_req, block_table, k=TOPK_MAX, out=None, slots=None,
                    workspace=None):
    """topk_rows and topk_to_global_slots in one call: (idx, slots), int32 [rows, k] each."""
    _need(logits, torch.float32, "logits", 2)
    _need(row_len, torch.int32, "row_len", 1)
    _need(row_req, torch.int32, "row_req", 1)
    _need(block_table, torch.int32, "block_table", 2)
    rows = logits.shape[0]
    if row_len.shape[0] != rows or row_req.shape[0] != rows:
        raise ValueError("row_len and row_req need one entry per row")
    dev = logits.device
    out = torch.empty((rows, k), dtype=torch.int32, device=dev) if out is None else out
    slots = torch.empty((rows, k), dtype=torch.int32, device=dev) if slots is None else slots
    _out(out, torch.int32, "out", (rows, k))
    _out(slots, torch.int32, "slots", (rows, k))
    ws_bytes = topk_workspace_bytes(rows, logits.stride(0), k)
    if ws_bytes and workspace is None:
        workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
    _check(load().topk_rows_slots(_ptr(logits), logits.stride(0), _ptr(row_len), _ptr(row_req),
                                  _ptr(block_table), block_table.stride(0), block_table.shape[0],
                                  rows, k, _ptr(out), _ptr(slots), _ptr(workspace),
                                  workspace.numel() if workspace is not None else 0, _stream()),
           "topk_rows_slots")
    return out, slots


def topk_rows_slots_noalloc(logits, row_len, row_req, block_table, k=TOPK_MAX, out=None, slots=None):
    """topk_rows_slots through the allocation-free entry point (segment
    candidates in the library's built-in device buffer).  Pass ``out`` and
    ``slots`` to allocate nothing at all; otherwise they are allocated here,
    outside the C call."""
    _need(logits, torch.float32, "logits", 2)
    _need(row_len, torch.int32, "row_len", 1)
    _need(row_req, torch.int32, "row_req", 1)
    _need(block_table, torch.int32, "block_table", 2)
    rows = logits.shape[0]
    if row_len.shape[0] != rows or row_req.shape[0] != rows:
        raise ValueError("row_len and row_req need one entry per row")
    dev = logits.device
    out = torch.empty((rows, k), dtype=torch.int32, device=dev) if out is None else out
    slots = torch.empty((rows, k), dtype=torch.int32, device=dev) if slots is None else slots
    _out(out, torch.int32, "out", (rows, k))
    _out(slots, torch.int32, "slots", (rows, k))
    _check(load().topk_rows_slots_noalloc(_ptr(logits), logits.stride(0), _ptr(row_len), _ptr(row_req),
                                          _ptr(block_table), block_table.stride(0), block_table.shape[0],
                                          rows, k, _ptr(out), _ptr(slots), _stream()),
           "topk_rows_slots_noalloc")
    return out, slots


def paged_mqa_topk_hist_bytes(rows, logits_stride):
    return load().paged_mqa_topk_hist_bytes(rows, logits_stride)


def paged_mqa_topk_slots(q_fp8, weights, kv_cache, block_table, context_lens, k=TOPK_MAX, width=None,
                         hist=None, logits=None, row_len=None, row_req=None, out=None, slots=None,
                         workspace=None):
    """One decode step through the fused entry: the logits kernel also counts
    each row's logits into ``hist`` (int32 [rows, 1024], zero on entry and
    left zero) and the selection starts from those counts.  Returns (logits,
    row_len, row_req, idx, slots).  ``hist`` is allocated zeroed here when
    the shape uses one and none is passed; keep and pass it back to allocate
    nothing per step."""
    _need(q_fp8, torch.uint8, "q_fp8", 4)
    _need(weights, torch.float32, "weights", 2)
    _need(kv_cache, torch.uint8, "kv_cache", 2)
    _need(block_table, torch.int32, "block_table", 2)
    _need(context_lens, torch.int32, "context_lens", 1)
    B, next_n = q_fp8.shape[0], q_fp8.shape[1]
    if tuple(q_fp8.shape[2:]) != (HEADS, DIM) or tuple(weights.shape) != (B * next_n, HEADS):
        raise ValueError("q_fp8 must be [B,next_n,64,128] and weights [B*next_n,64]")
    if context_lens.shape[0] != B or block_table.shape[0] != B:
        raise ValueError("context_lens and block_table need one row per request")
    rows = B * next_n
    width = block_table.shape[1] * BLOCK if width is None else width
    dev = q_fp8.device
    logits = torch.empty((rows, width), dtype=torch.float32, device=dev) if logits is None else logits
    row_len = torch.empty((rows,), dtype=torch.int32, device=dev) if row_len is None else row_len
    row_req = torch.empty((rows,), dtype=torch.int32, device=dev) if row_req is None else row_req
    out = torch.empty((rows, k), dtype=torch.int32, device=dev) if out is None else out
    slots = torch.empty((rows, k), dtype=torch.int32, device=dev) if slots is None else slots
    _out(logits, torch.float32, "logits", (rows, width))
    _out(row_len, torch.int32, "row_len", (rows,))
    _out(row_req, torch.int32, "row_req", (rows,))
    _out(out, torch.int32, "out", (rows, k))
    _out(slots, torch.int32, "slots", (rows, k))
    hist_bytes = paged_mqa_topk_hist_bytes(rows, width) if rows else 0
    if hist is None and hist_bytes:
        hist = torch.zeros((rows, 1024), dtype=torch.int32, device=dev)
    if hist is not None:
        _need(hist, torch.int32, "hist")
    ws_bytes = 0 if hist_bytes else (topk_workspace_bytes(rows, width, k) if rows else 0)
    if ws_bytes and workspace is None:
        workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
    _check(load().paged_mqa_topk_slots(
        _ptr(q_fp8), _ptr(weights), _ptr(kv_cache), kv_cache.shape[0], _ptr(block_table),
        block_table.stride(0), _ptr(context_lens), B, next_n, _ptr(logits), logits.stride(0),
        _ptr(row_len), _ptr(row_req), k, _ptr(out), _ptr(slots), _ptr(hist),
        hist.numel() * 4 if hist is not None else 0, _ptr(workspace),
        workspace.numel() if workspace is not None else 0, _stream()), "paged_mqa_topk_slots")
    return logits, row_len, row_req, out, slots


def decode_indexer(q_fp8, weights, kv_cache, block_table, context_lens, k=TOPK_MAX, width=None,
                   clean=True):
    """The decode hot path: logits -> top-k -> global slot ids, one stream, no
    host sync.  clean=False skips the -inf fill past each request's key blocks
    (the top-k reads a row only up to its limit; same indices and slot ids)."""
    logits, row_len, row_req = paged_mqa_logits(q_fp8, weights, kv_cache, block_table,
                                                context_lens, width, clean=clean)
    idx, slots = topk_rows_slots(logits, row_len, row_req, block_table, k)
    return logits, idx, slots
