"""Exact CPU definition of the fp8 MLA cache and of sparse MLA decode over it
(TEST INFRASTRUCTURE ONLY: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may use this module; it shares nothing with the HIP kernels).

Cache entry ("fp8_ds_mla" layout; prhub summary of vLLM PR #47090, key source
excerpt of ``_fused_norm_rope_kernel``, the MLA_CACHE_DS_MLA branch):
    bytes   0..511  the 512 latent values kv_c as fp8 e4m3fn codes, quantised
                    per 128-value tile: amax = max |tile|,
                    scale = max(amax * fl32(1/448), 1.1754944e-38),
                    code = fp8(value / scale) (float32 arithmetic)
    bytes 512..527  the 4 tile scales, float32
    bytes 528..655  the 64 RoPE values k_pe, bfloat16
    = 656 bytes per token.  Token slot s lives in block s // block_size at
    entry s % block_size; entries are 656 bytes apart and a block holds
    block_size entries.

Sparse MLA decode (the consumer of the global slot ids; ROCm/ATOM PR #1094,
Technical Details, "sparse MLA decode" reading the converted global paged KV
indices).  The pages name the op but do not print its arithmetic; this module
takes the plain absorbed-MLA reading: for query row t and head h
    score_j = sm_scale * (q_nope[t,h] . kv_j + q_pe[t,h] . kpe_j)
over the row's valid slots j (slot id >= 0 and inside the cache), where kv_j
is the dequantised latent (code * tile scale) and kpe_j the stored RoPE part;
    p = softmax(score),  out[t,h] = sum_j p_j kv_j,  lse[t,h] = log sum_j exp(score_j).
A row with no valid slot gives out = 0 and lse = -inf.  Everything is fp64.
"""
import numpy as np

from .indexer import FLT_MIN, INV_448, e4m3fn_table, fp8_encode

KV_DIM = 512          # latent (NoPE) values per token
TILE = 128            # values per quantisation tile
TILES = KV_DIM // TILE
ROPE_DIM = 64
ENTRY_BYTES = KV_DIM + 4 * TILES + 2 * ROPE_DIM   # 656
SCALE_OFF = KV_DIM                                 # 512
ROPE_OFF = KV_DIM + 4 * TILES                      # 528

_TABLE = e4m3fn_table()


def f32_to_bf16_bits(x):
    """float32 -> bfloat16 bit pattern, round to nearest even (the cast the
    excerpt applies to the RoPE part: ``.to(tl.bfloat16)``).  Finite inputs."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f64(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def quantize_tiles(kv):
    """Per-tile dynamic fp8 quantisation of latent rows (the excerpt's
    tile_amax / tile_scale / cast, all float32).
    kv: float32 [N, 512].  Returns (codes uint8 [N, 512], scales float32 [N, 4])."""
    kv = np.asarray(kv, dtype=np.float32).reshape(-1, TILES, TILE)
    amax = np.max(np.abs(kv), axis=-1)
    scale = np.maximum(amax * INV_448, FLT_MIN).astype(np.float32)
    y = (kv / scale[..., None]).astype(np.float32)
    return fp8_encode(y).reshape(-1, KV_DIM), scale


def mla_cache_write(kv_c, k_pe, slot_mapping, cache):
    """Write tokens into the fp8 MLA cache, in place.
    kv_c: float32 [N, 512]; k_pe: float32 [N, 64] (both bf16-representable in
    practice; k_pe is stored as bf16 with round to nearest even);
    slot_mapping: int [N]; a negative slot, or one past the cache's
    num_blocks*block_size entries, is skipped;
    cache: uint8 [num_blocks, block_size, 656] (modified)."""
    codes, scale = quantize_tiles(kv_c)
    rope = f32_to_bf16_bits(np.asarray(k_pe, dtype=np.float32))
    slots = np.asarray(slot_mapping, dtype=np.int64)
    bs = cache.shape[1]
    for i, s in enumerate(slots):
        if s < 0 or s >= cache.shape[0] * bs:
            continue
        e = cache[s // bs, s % bs]
        e[:SCALE_OFF] = codes[i]
        e[SCALE_OFF:ROPE_OFF] = scale[i].view(np.uint8)
        e[ROPE_OFF:ENTRY_BYTES] = rope[i].view(np.uint8)
    return cache


def mla_entry(cache, slot):
    """Decode one entry: (kv float64 [512], kpe float64 [64])."""
    bs = cache.shape[1]
    e = cache[slot // bs, slot % bs]
    scale = e[SCALE_OFF:ROPE_OFF].copy().view(np.float32).astype(np.float64)
    kv = _TABLE[e[:SCALE_OFF]].reshape(TILES, TILE) * scale[:, None]
    kpe = bf16_bits_to_f64(e[ROPE_OFF:ENTRY_BYTES].copy().view(np.uint16))
    return kv.reshape(KV_DIM), kpe


def sparse_mla_decode(q_nope, q_pe, cache, slots, sm_scale, with_abs=False):
    """q_nope float [T, H, 512], q_pe float [T, H, 64], slots int [T, K]
    (global slot ids, -1 padded; ids outside the cache are skipped like -1).
    Returns (out float64 [T, H, 512], lse float64 [T, H]); with ``with_abs``
    also sum_j softmax(score)_j |kv_j| [T, H, 512], the magnitude that bounds
    how far rounding the softmax weights can move ``out``."""
    q_nope = np.asarray(q_nope, dtype=np.float64)
    q_pe = np.asarray(q_pe, dtype=np.float64)
    slots = np.asarray(slots, dtype=np.int64)
    T, H = q_nope.shape[:2]
    n_slots = cache.shape[0] * cache.shape[1]
    out = np.zeros((T, H, KV_DIM))
    out_abs = np.zeros((T, H, KV_DIM))
    lse = np.full((T, H), -np.inf)
    for t in range(T):
        valid = [s for s in slots[t] if 0 <= s < n_slots]
        if not valid:
            continue
        ents = [mla_entry(cache, s) for s in valid]
        kv = np.stack([e[0] for e in ents])      # [n, 512]
        kpe = np.stack([e[1] for e in ents])     # [n, 64]
        score = sm_scale * (q_nope[t] @ kv.T + q_pe[t] @ kpe.T)   # [H, n]
        m = score.max(axis=1, keepdims=True)
        p = np.exp(score - m)
        z = p.sum(axis=1, keepdims=True)
        out[t] = (p / z) @ kv
        out_abs[t] = (p / z) @ np.abs(kv)
        lse[t] = (m + np.log(z))[:, 0]
    return (out, lse, out_abs) if with_abs else (out, lse)
