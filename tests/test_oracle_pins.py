"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test ties one oracle function to something it does not compute: a value
printed in a golden fixture derived by hand from a definition on the pages, a
library routine (torch's float8_e4m3fn), a closed form, brute force on a tiny
input, or an invariant of the method.  No test here needs a GPU.
"""
import itertools
import math
import os
import struct

import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_indexer_paged_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f32(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


def _f32_round(x):
    """Round a Python float (double) to the nearest float32 via struct (RNE)."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


# ---------------------------------------------------------------- fp8 table
def test_e4m3fn_table_matches_torch_on_all_codes():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(O.e4m3fn_table(), ref, equal_nan=True)


def test_e4m3fn_table_matches_hand_derived_golden():
    t = O.e4m3fn_table()
    n = 0
    for line in open(os.path.join(GOLDEN, "e4m3fn_codes.txt")):
        if line.startswith("#") or not line.strip():
            continue
        code, val = line.split()
        code = int(code, 16)
        if val == "nan":
            assert math.isnan(t[code])
        else:
            v = float(val)
            assert t[code] == v and math.copysign(1, t[code]) == math.copysign(1, v), hex(code)
        n += 1
    assert n >= 20


def test_e4m3fn_table_structure():
    t = O.e4m3fn_table()
    pos = t[:127]
    assert np.all(np.diff(pos) > 0)              # codes 0..126 strictly increasing
    assert pos[-1] == 448.0
    assert np.array_equal(t[128:255], -pos)      # sign bit mirrors
    assert np.isnan(t[127]) and np.isnan(t[255])
    # every finite value times 2^9 is an integer below 2^18
    ints = pos * 512
    assert np.all(ints == np.round(ints)) and ints.max() < 2 ** 18


# ---------------------------------------------------------------- encoder
def _torch_cast(y):
    return torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_fp8_encode_matches_torch_at_every_midpoint():
    pos = O.e4m3fn_table()[:127]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (pos[:-1] + pos[1:]) / 2)  # exact in f32
    pts = [mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0)),
           pos.astype(np.float32)]
    y = np.concatenate(pts + [-p for p in pts])
    assert np.array_equal(O.fp8_encode(y), _torch_cast(y))


def test_fp8_encode_ties_go_to_even_code():
    pos = O.e4m3fn_table()[:127]
    for c in range(126):
        mid = np.float32((pos[c] + pos[c + 1]) / 2)
        got = int(O.fp8_encode(np.array([mid]))[0])
        assert got == (c if c % 2 == 0 else c + 1)


def test_fp8_encode_matches_torch_on_random_values():
    rng = np.random.default_rng(7)
    y = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 0.1, 1, 30, 200)])
    y = np.clip(y, -448, 448).astype(np.float32)
    assert np.array_equal(O.fp8_encode(y), _torch_cast(y))


def test_fp8_encode_saturates_and_keeps_sign_of_zero():
    y = np.array([448.0, 448.5, 464.0, 1e6, -460.0, 0.0, -0.0, -1e-30], dtype=np.float32)
    assert O.fp8_encode(y).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x00, 0x80, 0x80]


# ---------------------------------------------------------------- quantiser
def _golden_quant():
    d = {}
    for line in open(os.path.join(GOLDEN, "quantizer_worked.txt")):
        if line.startswith("#") or not line.strip():
            continue
        k, *v = line.split()
        d[k] = v
    return d


def test_quantize_rows_matches_hand_worked_example():
    g = _golden_quant()
    assert O.INV_448.view(np.uint32) == int(g["inv448_bits"][0], 16)
    x = np.array([[float(v) for v in g["x"]]], dtype=np.float32)
    codes, scale = O.quantize_rows(x)
    assert scale.view(np.uint32)[0] == int(g["scale_bits"][0], 16)
    assert codes[0].tolist() == [int(c, 16) for c in g["codes"]]
    codes, scale = O.quantize_rows(np.zeros((3, 128), np.float32))
    assert np.all(scale.view(np.uint32) == int(g["zero_scale_bits"][0], 16))
    assert not codes.any()


def test_quantize_rows_scale_is_float32_product():
    rng = np.random.default_rng(3)
    x = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(rng.standard_normal((500, 128)).astype(np.float32)))
    _, scale = O.quantize_rows(x)
    for r in range(500):
        amax = max(abs(float(v)) for v in x[r])
        want = max(_f32_round(amax * float(O.INV_448)), float(O.FLT_MIN))
        assert float(scale[r]) == want


def test_quantize_rows_amax_maps_to_448_and_error_bound():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2000, 128)).astype(np.float32) * rng.uniform(1e-3, 1e3, (2000, 1)).astype(np.float32)
    codes, scale = O.quantize_rows(x)
    t = O.e4m3fn_table()
    am = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(t[codes[np.arange(2000), am]]) == 448.0)
    # round-to-nearest: error at most half the local spacing (2^-4 relative
    # for normals, 2^-10 absolute in the subnormal range), times the scale
    deq = t[codes] * scale[:, None].astype(np.float64)
    err = np.abs(deq - x.astype(np.float64))
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * scale[:, None]) * (1 + 1e-6)
    assert np.all(err <= bound)


def test_quantize_q_folds_scale_into_weights():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((3, 64, 128)).astype(np.float32)
    w = rng.standard_normal((3, 64)).astype(np.float32)
    codes, w_eff, qs = O.quantize_q(q, w)
    c2, s2 = O.quantize_rows(q.reshape(3, -1))
    assert np.array_equal(codes.reshape(3, -1), c2) and np.array_equal(qs, s2)
    for r in range(3):
        for h in range(64):
            assert float(w_eff[r, h]) == _f32_round(float(w[r, h]) * float(qs[r]))


# ---------------------------------------------------------------- helpers
def _one_block_cache(nblocks=4):
    return np.zeros((nblocks, O.BLOCK_BYTES), dtype=np.uint8)


def _set_token(cache, blk, off, codes, scale):
    cache[blk, off * 128:(off + 1) * 128] = codes
    cache[blk, 8192 + 4 * off:8192 + 4 * off + 4] = np.frombuffer(np.float32(scale).tobytes(), np.uint8)


def _small_workload(ctx, next_n, bt_width, num_blocks, seed):
    """A quantised paged workload built with the oracle's own quantiser."""
    wl = synth.custom(len(ctx), next_n, ctx, num_blocks, bt_width, seed)
    pool = wl.poisoned_pool()
    O.k_cache_write(synth.bf16_bits_to_f32(wl.k_all()), wl.slot_mapping(), pool)
    qc, weff, _ = O.quantize_q(synth.bf16_bits_to_f32(wl.q()), wl.w())
    return wl, pool, qc.reshape(wl.batch, next_n, 64, 128), weff


# ---------------------------------------------------------------- layout
def test_cache_layout_matches_golden():
    g = {}
    for line in open(os.path.join(GOLDEN, "cache_layout.txt")):
        if line.startswith("#") or not line.strip():
            continue
        k, *v = line.split()
        g[k] = [int(x) for x in v]
    assert O.BLOCK == g["block_size"][0] and O.DIM == g["head_dim"][0]
    assert O.BLOCK_BYTES == g["block_bytes"][0]
    cache = _one_block_cache(1)
    k = np.zeros((1, 128), np.float32)
    k[0, 0] = 1.0
    O.k_cache_write(k, np.array([5]), cache)
    nz = np.nonzero(cache[0])[0]
    lo, hi = g["token5_values"]
    slo, shi = g["token5_scale"]
    assert set(nz.tolist()) <= set(range(lo, hi)) | set(range(slo, shi))
    assert cache[0, lo] == 0x7E
    assert cache[0, slo:shi].view(np.float32)[0] == np.float32(1.0) * O.INV_448


def test_k_cache_write_skips_negative_slots_and_touches_only_owned_bytes():
    cache = np.full((3, O.BLOCK_BYTES), 0xAB, dtype=np.uint8)
    k = np.random.default_rng(1).standard_normal((4, 128)).astype(np.float32)
    O.k_cache_write(k, np.array([-1, 64 + 3, 2 * 64 + 63, -5]), cache)
    assert np.all(cache[0] == 0xAB)
    codes, scale = O.quantize_rows(k)
    assert np.array_equal(cache[1, 3 * 128:4 * 128], codes[1])
    assert cache[1, 8192 + 12:8192 + 16].view(np.float32)[0] == scale[1]
    assert np.array_equal(cache[2, 63 * 128:64 * 128], codes[2])
    owned = np.zeros(O.BLOCK_BYTES, bool)
    owned[3 * 128:4 * 128] = True
    owned[8192 + 12:8192 + 16] = True
    assert np.all(cache[1][~owned] == 0xAB)


# ---------------------------------------------------------------- logits: closed forms
def _paged_single(q_tok, k_tok, kscale, w, ctx=None):
    """Place keys k_tok [S,128] (codes) into a paged cache through a shuffled
    block table and score one query row q_tok [64,128] (codes)."""
    S = k_tok.shape[0]
    nb = -(-S // 64)
    perm = np.random.default_rng(S).permutation(nb + 2)[:nb]
    cache = np.zeros((nb + 2, O.BLOCK_BYTES), np.uint8)
    for s in range(S):
        _set_token(cache, perm[s // 64], s % 64, k_tok[s], kscale[s])
    bt = perm[None, :].astype(np.int32)
    ctx = S if ctx is None else ctx
    return O.paged_mqa_logits(q_tok[None, None], w[None].astype(np.float32), cache, bt,
                              np.array([ctx]), 1, nb * 64)[0]


def test_logits_all_ones_closed_form():
    S = 70
    q = np.full((64, 128), 0x38, np.uint8)          # 1.0
    k = np.full((S, 128), 0x38, np.uint8)
    rng = np.random.default_rng(0)
    w = rng.standard_normal(64).astype(np.float32)
    ks = rng.uniform(0.5, 2, S).astype(np.float32)
    L = _paged_single(q, k, ks, w)
    want = ks.astype(np.float64) * 128.0 * math.fsum(float(x) for x in w)
    assert np.allclose(L[:S], want, rtol=1e-13, atol=0)
    assert np.all(np.isneginf(L[S:]))


def test_logits_one_hot_picks_head_dim_and_key():
    S = 64
    t = O.e4m3fn_table()
    q = np.zeros((64, 128), np.uint8)
    k = np.zeros((S, 128), np.uint8)
    q[7, 19] = 0x40        # head 7, dim 19: 2.0
    k[11, 19] = 0x6E       # key 11, dim 19: 112
    k[12, 20] = 0x6E       # key 12, other dim: no overlap
    w = np.zeros(64, np.float32)
    w[7] = 0.25
    w[8] = 100.0           # a head with zero query must not contribute
    q[9, 19] = 0x40        # head 9 sees the same positive dot product ...
    w[9] = -0.5            # ... through a negative weight: ReLU is on the dot, not on w*dot
    ks = np.full(S, 0.5, np.float32)
    L = _paged_single(q, k, ks, w)
    want = np.zeros(S)
    want[11] = 0.5 * (0.25 - 0.5) * t[0x40] * t[0x6E]
    assert np.array_equal(L[:S], want)


def test_logits_relu_drops_negative_dots_and_alternating_signs_cancel():
    S = 3
    q = np.full((64, 128), 0x38, np.uint8)
    k = np.zeros((S, 128), np.uint8)
    k[0] = 0xB8                                    # all -1: d = -128 -> ReLU 0
    k[1, 0::2], k[1, 1::2] = 0x38, 0xB8            # +1/-1 alternating: d = 0
    k[2] = 0x30                                    # all 0.5: d = 64
    w = np.full(64, 2.0 ** -6, np.float32)         # mean over heads
    ks = np.array([3.0, 3.0, 0.25], np.float32)
    L = _paged_single(q, k, ks, w)
    assert L[0] == 0.0 and L[1] == 0.0
    assert L[2] == 0.25 * 64.0


def test_logits_brute_force_tiny_pure_python():
    """P3: an independent dense route: torch's fp8 decode, plain Python loops."""
    wl, pool, qc, weff = _small_workload([70, 5], 2, 3, 8, seed=11)
    L = O.paged_mqa_logits(qc, weff, pool, wl.block_table, wl.ctx, 2, wl.width)
    dec = lambda a: torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e4m3fn).double().tolist()
    for b in range(2):
        c = int(wl.ctx[b])
        keys, scales = [], []
        for s in range(c):
            blk = int(wl.block_table[b][s // 64])
            keys.append(dec(pool[blk, (s % 64) * 128:(s % 64 + 1) * 128]))
            scales.append(float(pool[blk, 8192 + 4 * (s % 64):8192 + 4 * (s % 64) + 4].view(np.float32)[0]))
        for j in range(2):
            r = b * 2 + j
            qrow = [dec(qc[b, j, h]) for h in range(64)]
            lim = c - 2 + j + 1
            for s in range(wl.width):
                if s >= lim:
                    assert L[r, s] == -math.inf
                    continue
                tot = 0.0
                for h in range(64):
                    d = sum(a * bb for a, bb in zip(qrow[h], keys[s]))
                    tot += float(weff[r, h]) * max(d, 0.0)
                assert math.isclose(L[r, s], scales[s] * tot, rel_tol=1e-12, abs_tol=1e-300)


# ---------------------------------------------------------------- logits: invariants
def test_causal_mask_poison_invariance():
    """P4: bytes at or past each request's context never reach a result."""
    wl, pool, qc, weff = _small_workload([100, 130, 64], 2, 4, 16, seed=12)
    L = O.paged_mqa_logits(qc, weff, pool, wl.block_table, wl.ctx, 2, wl.width)
    bad = pool.copy()
    for b, c in enumerate(wl.ctx.tolist()):
        for s in range(c, 4 * 64):
            blk = wl.block_table[b][s // 64]
            if blk < 0:
                continue
            bad[blk, (s % 64) * 128:(s % 64 + 1) * 128] = 0xFF
            bad[blk, 8192 + 4 * (s % 64):8192 + 4 * (s % 64) + 4] = \
                np.frombuffer(np.float32(np.inf).tobytes(), np.uint8)
    used = set(wl.block_table[wl.block_table >= 0].tolist())
    for x in range(16):
        if x not in used:
            bad[x] = 0x7F
    L2 = O.paged_mqa_logits(qc, weff, bad, wl.block_table, wl.ctx, 2, wl.width)
    assert np.array_equal(L, L2)
    lim, _ = O.decode_limits(wl.ctx, 2)
    for r in range(6):
        assert np.all(np.isfinite(L[r, :lim[r]])) and np.all(np.isneginf(L[r, lim[r]:]))


def test_block_table_permutation_invariance():
    """P5: moving physical blocks and rewriting the table changes nothing."""
    wl, pool, qc, weff = _small_workload([200, 77], 1, 4, 12, seed=13)
    L = O.paged_mqa_logits(qc, weff, pool, wl.block_table, wl.ctx, 1, wl.width)
    pi = np.random.default_rng(99).permutation(12)
    pool2 = np.empty_like(pool)
    pool2[pi] = pool
    bt2 = np.where(wl.block_table >= 0, pi[np.maximum(wl.block_table, 0)], -1).astype(np.int32)
    L2 = O.paged_mqa_logits(qc, weff, pool2, bt2, wl.ctx, 1, wl.width)
    assert np.array_equal(L, L2)


def test_decode_next_n_equals_prefill_on_gathered_k():
    """P6: B=1, next_n=N, ctx=N on the paged cache == prefill on its gather."""
    N = 37
    wl, pool, qc, weff = _small_workload([N], N, 1, 4, seed=14)
    Ld = O.paged_mqa_logits(qc, weff, pool, wl.block_table, wl.ctx, N, 64)
    cu = np.array([0, N])
    kv, ks = O.gather_indexer_k(pool, wl.block_table, cu, N)
    Lp = O.mqa_logits(qc.reshape(N, 64, 128), weff, kv, ks, cu, 64)
    assert np.array_equal(Ld, Lp)


def test_chunked_prefill_equals_paged_decode_with_next_n():
    """Chunked prefill: the last N tokens of each request scored against its
    gathered context == paged decode with next_n = N (a different route: the
    paged cache and the decode limit rule)."""
    N, ctx = 5, [150, 97, 64]
    wl, pool, qc, weff = _small_workload(ctx, N, 3, 12, seed=15)
    Ld = O.paged_mqa_logits(qc, weff, pool, wl.block_table, wl.ctx, N, 192)
    cu_k = np.concatenate([[0], np.cumsum(ctx)])
    kv, ks = O.gather_indexer_k(pool, wl.block_table, cu_k, int(cu_k[-1]))
    cu_q = np.arange(len(ctx) + 1) * N
    Lc = O.mqa_logits_chunked(qc.reshape(-1, 64, 128), weff, kv, ks, cu_q, cu_k, 192)
    assert np.array_equal(Ld, Lc)


def test_chunked_prefill_whole_request_is_prefill_and_batching_is_invisible():
    """n_q = n_k reduces to mqa_logits; in a ragged batch each request's rows
    equal that request scored alone."""
    rng = np.random.default_rng(16)
    n_q, n_k = [7, 1, 12, 0, 3], [30, 1, 12, 9, 70]
    cu_q = np.concatenate([[0], np.cumsum(n_q)])
    cu_k = np.concatenate([[0], np.cumsum(n_k)])
    q = O.fp8_encode(rng.standard_normal((cu_q[-1], 64, 128)).astype(np.float32))
    w = rng.standard_normal((cu_q[-1], 64)).astype(np.float32)
    k = O.fp8_encode(rng.standard_normal((cu_k[-1], 128)).astype(np.float32))
    ks = (rng.random(cu_k[-1]) + 0.5).astype(np.float32)
    L = O.mqa_logits_chunked(q, w, k, ks, cu_q, cu_k, 80)
    for b in range(len(n_q)):
        qs, ksl = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
        one = O.mqa_logits_chunked(q[qs], w[qs], k[ksl], ks[ksl], [0, n_q[b]], [0, n_k[b]], 80)
        assert np.array_equal(L[qs], one)
        if n_q[b] == n_k[b]:
            assert np.array_equal(one, O.mqa_logits(q[qs], w[qs], k[ksl], ks[ksl], [0, n_q[b]], 80))
        for i in range(n_q[b]):  # the limit rule, column by column
            lim = n_k[b] - n_q[b] + i + 1
            assert np.all(np.isfinite(one[i, :lim])) and np.all(np.isneginf(one[i, lim:]))


def test_chunked_prefill_short_context_and_width_clamp():
    """A context shorter than its chunk leaves leading rows with no visible
    key (all -inf); a row whose limit exceeds the width is not written."""
    rng = np.random.default_rng(17)
    q = O.fp8_encode(rng.standard_normal((6, 64, 128)).astype(np.float32))
    w = np.ones((6, 64), np.float32)
    k = O.fp8_encode(rng.standard_normal((10, 128)).astype(np.float32))
    ks = np.ones(10, np.float32)
    L = O.mqa_logits_chunked(q, w, k, ks, [0, 4, 6], [0, 2, 10], 7)
    # request 0: n_q 4, n_k 2 -> limits 0, 0, 1, 2
    assert np.all(np.isneginf(L[0])) and np.all(np.isneginf(L[1]))
    assert np.isfinite(L[2, 0]) and np.all(np.isneginf(L[2, 1:]))
    assert np.all(np.isfinite(L[3, :2])) and np.all(np.isneginf(L[3, 2:]))
    # request 1: n_q 2, n_k 8 -> limits 7 (= width: written) and 8 (> width: not written)
    assert np.all(np.isfinite(L[4]))
    assert np.all(np.isnan(L[5]))


def test_non_clean_logits_differ_only_past_the_last_block_and_keep_the_top_k():
    """The non-clean variant equals clean logits on every request's key
    blocks and leaves the rest unwritten; the top-k, which reads a row only
    up to its limit, is the same on both."""
    ctx = [1, 64, 65, 130]
    wl, pool, qc, weff = _small_workload(ctx, 2, 4, 12, seed=18)
    clean = O.paged_mqa_logits(qc, weff, pool, wl.block_table, wl.ctx, 2, 256)
    vis = O.paged_mqa_logits(qc, weff, pool, wl.block_table, wl.ctx, 2, 256, clean=False)
    lim, _ = O.decode_limits(wl.ctx, 2)
    for b, c in enumerate(ctx):
        end = -(-c // 64) * 64
        rows = slice(2 * b, 2 * b + 2)
        assert np.array_equal(vis[rows, :end], clean[rows, :end])
        assert np.all(np.isnan(vis[rows, end:])) and np.all(np.isneginf(clean[rows, end:]))
    assert np.array_equal(O.topk_rows(vis, lim, 16), O.topk_rows(clean, lim, 16))


def test_exact_power_of_two_scaling():
    """P7: scaling w or every k_scale by 2^m scales the logits by exactly 2^m."""
    wl, pool, qc, weff = _small_workload([150, 33], 2, 3, 8, seed=15)
    L = O.paged_mqa_logits(qc, weff, pool, wl.block_table, wl.ctx, 2, wl.width)
    L2 = O.paged_mqa_logits(qc, (weff * np.float32(8.0)).astype(np.float32), pool,
                            wl.block_table, wl.ctx, 2, wl.width)
    assert np.array_equal(L2, L * 8.0)
    pool3 = pool.copy()
    sc = pool3[:, 8192:].copy().view(np.float32) * np.float32(0.25)
    pool3[:, 8192:] = sc.view(np.uint8)
    L3 = O.paged_mqa_logits(qc, weff, pool3, wl.block_table, wl.ctx, 2, wl.width)
    assert np.array_equal(L3, L * 0.25)


def test_decode_limits():
    lim, req = O.decode_limits([10, 3], 2)
    assert lim.tolist() == [9, 10, 2, 3] and req.tolist() == [0, 0, 1, 1]


# ---------------------------------------------------------------- top-k
def _brute_topk(vals, k):
    """The unique set S with every member beating every non-member under
    (larger value, then lower index), found by enumerating subsets."""
    n = len(vals)
    m = min(k, n)
    beats = lambda s, t: vals[s] > vals[t] or (vals[s] == vals[t] and s < t)
    found = [S for S in itertools.combinations(range(n), m)
             if all(beats(s, t) for s in S for t in range(n) if t not in S)]
    assert len(found) == 1
    return list(found[0])


def test_topk_matches_subset_enumeration_with_forced_ties():
    rng = np.random.default_rng(21)
    for trial in range(300):
        n = int(rng.integers(1, 12))
        k = int(rng.integers(1, 8))
        vals = rng.integers(-3, 3, n).astype(np.float32)
        vals[rng.random(n) < 0.2] = -0.0
        vals[rng.random(n) < 0.1] = -np.inf
        width = n + int(rng.integers(0, 3))
        row = np.full(width, np.nan, np.float32)   # never read past row_len
        row[:n] = vals
        got = O.topk_rows(row[None], [n], k)[0]
        want = _brute_topk([float(v) + 0.0 for v in vals], k)
        assert got.tolist() == want + [-1] * (k - len(want))


def test_topk_special_cases():
    k = 8
    L = np.zeros((5, 20), np.float32)
    L[1] = np.arange(20)                 # strictly increasing -> last k
    L[2] = -np.arange(20)                # strictly decreasing -> first k
    L[3, :] = 1.0
    L[3, 4] = -0.0
    L[3, 5] = 0.0                        # -0 == +0 tie; not in top anyway
    L[4, ::2] = -0.0                     # all zero of both signs -> 0..7
    out = O.topk_rows(L, [20, 20, 20, 20, 20], k)
    assert out[0].tolist() == list(range(8))
    assert out[1].tolist() == list(range(12, 20))
    assert out[2].tolist() == list(range(8))
    assert out[3].tolist() == [0, 1, 2, 3, 6, 7, 8, 9]
    assert out[4].tolist() == list(range(8))
    short = O.topk_rows(L, [5, 0, 20, 3, 8], k)
    assert short[0].tolist() == [0, 1, 2, 3, 4, -1, -1, -1]
    assert short[1].tolist() == [-1] * 8
    assert short[3].tolist() == [0, 1, 2, -1, -1, -1, -1, -1]
    assert short[4].tolist() == list(range(8))


def test_topk_matches_numpy_stable_argsort():
    rng = np.random.default_rng(22)
    L = rng.standard_normal((20, 3000)).astype(np.float32)
    L[:, ::7] = np.round(L[:, ::7])      # many ties
    lens = rng.integers(0, 3000, 20)
    out = O.topk_rows(L, lens, 256)
    for r in range(20):
        n = int(lens[r])
        order = np.argsort(-L[r, :n].astype(np.float64), kind="stable")[:256]
        want = np.sort(order)
        assert out[r, :want.size].tolist() == want.tolist()
        assert np.all(out[r, want.size:] == -1)


# ---------------------------------------------------------------- slots / gather
def test_gather_semantics_full_blocks_remainder_and_empty_request():
    cache = np.zeros((6, O.BLOCK_BYTES), np.uint8)
    for blk in range(6):
        for off in range(64):
            _set_token(cache, blk, off, np.full(128, (blk * 64 + off) % 251, np.uint8),
                       float(blk * 1000 + off))
    bt = np.array([[4, 1, -1], [0, -1, -1], [5, 2, 3]], np.int32)
    cu = np.array([0, 100, 100, 230])
    v, s = O.gather_indexer_k(cache, bt, cu, 230)
    for t in range(100):
        blk = bt[0][t // 64]
        assert s[t] == blk * 1000 + t % 64 and v[t, 0] == (blk * 64 + t % 64) % 251
    for t in range(130):
        blk = bt[2][t // 64]
        assert s[100 + t] == blk * 1000 + t % 64 and v[100 + t, 5] == (blk * 64 + t % 64) % 251


def test_slot_round_trip():
    """P9: the bytes at each selected slot equal the gathered row of that key."""
    wl, pool, qc, weff = _small_workload([300, 90], 1, 5, 20, seed=16)
    L = O.paged_mqa_logits(qc, weff, pool, wl.block_table, wl.ctx, 1, wl.width)
    lim, req = O.decode_limits(wl.ctx, 1)
    top = O.topk_rows(L, lim, 128)
    slots = O.topk_to_global_slots(top, req, wl.block_table)
    cu = np.concatenate([[0], np.cumsum(wl.ctx)])
    kv, ks = O.gather_indexer_k(pool, wl.block_table, cu, int(cu[-1]))
    for r in range(2):
        for i, sl in zip(top[r].tolist(), slots[r].tolist()):
            if i < 0:
                assert sl == -1
                continue
            assert 0 <= sl < 64 * 20
            blk, off = sl // 64, sl % 64
            assert np.array_equal(pool[blk, off * 128:(off + 1) * 128], kv[cu[r] + i])
            assert pool[blk, 8192 + 4 * off:8192 + 4 * off + 4].view(np.float32)[0] == ks[cu[r] + i]


def test_slot_map_hand_values_and_unmapped_indices():
    """Slot ids worked by hand from the map block_table[b][i // 64] * 64 + i % 64
    (ROCm/ATOM PR #1094, Technical Details), and -1 for every index the table
    does not map: padding, a negative table entry, a column past the table and
    a request that is not a row of the table (negative or too large)."""
    bt = np.array([[5, 9, -1], [2, 0, 7]], np.int32)
    idx = np.array([[0, 63, 64, 127, -1, 128, 191, 192],
                    [0, 1, 64, 130, 191, -1, -1, -1],
                    [0, 1, 2, 3, 4, 5, 6, 7],
                    [0, 1, 2, 3, 4, 5, 6, 7]], np.int32)
    req = np.array([0, 1, 5, -1], np.int32)
    got = O.topk_to_global_slots(idx, req, bt)
    # row 0: block 5 -> 320.., block 9 -> 576.., entry -1 and column 3 (past the table) -> -1
    assert got[0].tolist() == [320, 383, 576, 639, -1, -1, -1, -1]
    # row 1: block 2 -> 128, 129; block 0 -> 0; block 7 -> 448 + 2 = 450, 448 + 63 = 511
    assert got[1].tolist() == [128, 129, 0, 450, 511, -1, -1, -1]
    assert got[2].tolist() == [-1] * 8
    assert got[3].tolist() == [-1] * 8
    assert got.dtype == np.int32


def test_topk_nan_ranks_below_every_number_and_ties_by_index():
    """NaN (either sign, any payload) ranks after -inf; NaNs tie, so the
    lower index wins among them.  Worked by hand on a 7-column row."""
    bits = np.array([0x3F800000, 0x7FC00000, 0xFF800000, 0xFFC00001, 0x40000000,
                     0x7F800001, 0xBF800000], np.uint32)        # 1, NaN, -inf, -NaN, 2, NaN, -1
    L = bits.view(np.float32)[None, :]
    for k, want in [(2, [0, 4]), (4, [0, 2, 4, 6]), (5, [0, 1, 2, 4, 6]), (6, [0, 1, 2, 3, 4, 6]),
                    (7, [0, 1, 2, 3, 4, 5, 6])]:
        got = O.topk_rows(L, np.array([7]), k)[0]
        assert got.tolist() == want, (k, got)
    # only NaNs: the lowest indices
    N = np.full((1, 10), np.nan, np.float32)
    assert O.topk_rows(N, np.array([10]), 3)[0].tolist() == [0, 1, 2]
