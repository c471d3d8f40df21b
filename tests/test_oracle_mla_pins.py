"""Pins of the fp8 MLA cache / sparse MLA decode oracle (oracle.mla) against
facts it does not compute: bytes derived by hand from the layout on the pages
(prhub summary of vLLM PR #47090, key source excerpt, MLA_CACHE_DS_MLA
branch), closed forms of softmax attention, and invariants.  CPU only."""
import math

import numpy as np
import pytest

import oracle as O

M = O.mla


def _cache(num_blocks=4, bs=64):
    return np.zeros((num_blocks, bs, M.ENTRY_BYTES), dtype=np.uint8)


def test_entry_layout_hand_derived():
    """Tile 0 all 1.0: scale = fl32(1/448) (bits 0x3B124925) and every code is
    448 = 1.75*2^8 -> 0x7E; tile 1 all 0: scale = FLT_MIN (0x00800000), codes 0;
    tile 2: 448 at dim 0 and -224 at dim 1 -> scale 1.0*... (amax 448: scale =
    fl32(448*fl32(1/448)) = 1.0), codes 0x7E and 0xF6 (-224 = -1.75*2^7);
    tile 3: 0.5 everywhere but 1.0 -> 1.0/scale = 448 -> 0x7E, 0.5/scale = 224
    -> 0x76.  RoPE stored as bf16: 1.0 -> 0x3F80, -2.5 -> 0xC020."""
    kv = np.zeros((1, 512), np.float32)
    kv[0, 0:128] = 1.0
    kv[0, 256] = 448.0
    kv[0, 257] = -224.0
    kv[0, 384:512] = 0.5
    kv[0, 384] = 1.0
    kpe = np.zeros((1, 64), np.float32)
    kpe[0, 0], kpe[0, 63] = 1.0, -2.5
    c = M.mla_cache_write(kv, kpe, [70], _cache())
    e = c[1, 6]
    scales = e[512:528].copy().view(np.uint32)
    assert scales[0] == 0x3B124925
    assert scales[1] == 0x00800000
    assert e[512 + 8:512 + 12].view(np.float32)[0] == 1.0
    assert np.all(e[0:128] == 0x7E)
    assert np.all(e[128:256] == 0)
    assert e[256] == 0x7E and e[257] == 0xF6 and np.all(e[258:384] == 0)
    assert e[384] == 0x7E and np.all(e[385:512] == 0x76)
    rope = e[528:656].copy().view(np.uint16)
    assert rope[0] == 0x3F80 and rope[63] == 0xC020 and np.all(rope[1:63] == 0)
    # nothing else written
    c2 = c.copy()
    c2[1, 6] = 0
    assert not c2.any()


def test_negative_slot_skipped_and_positions():
    rng = np.random.default_rng(1)
    kv = rng.standard_normal((3, 512)).astype(np.float32)
    kpe = rng.standard_normal((3, 64)).astype(np.float32)
    c = M.mla_cache_write(kv, kpe, [0, -1, 129], _cache(bs=64))
    M.mla_cache_write(kv, kpe, [4 * 64, 10 ** 6, -7], c)        # past the cache: skipped
    assert c[0, 0].any() and c[2, 1].any()
    c[0, 0] = 0
    c[2, 1] = 0
    assert not c.any()


def test_roundtrip_within_fp8_error():
    """Decoded latents are within the e4m3 rounding bound of the inputs:
    relative 2^-4 for normal codes, absolute scale*2^-10 below them."""
    rng = np.random.default_rng(2)
    kv = (rng.standard_normal((5, 512)) * np.exp(rng.standard_normal((5, 1)) * 3)).astype(np.float32)
    kpe = rng.standard_normal((5, 64)).astype(np.float32)
    c = M.mla_cache_write(kv, kpe, np.arange(5) * 7, _cache())
    for i in range(5):
        dec, pe = M.mla_entry(c, i * 7)
        scale = np.repeat(c.reshape(-1, M.ENTRY_BYTES)[i * 7, 512:528].copy().view(np.float32), 128)
        err = np.abs(dec - kv[i])
        assert np.all(err <= np.maximum(np.abs(kv[i]) * 2.0 ** -4, scale * 2.0 ** -10) * (1 + 1e-6))
        assert np.all(np.abs(pe - kpe[i]) <= np.abs(kpe[i]) * 2.0 ** -8)


def _hand_entries(c, rows):
    """Write entries byte by byte: scale 1.0 for every tile, codes of small
    exact values, RoPE in bf16.  rows: list of (slot, {dim: code}, {rope: bits})."""
    bs = c.shape[1]
    for slot, codes, rope in rows:
        e = c[slot // bs, slot % bs]
        e[:] = 0
        e[512:528] = np.array([1.0] * 4, np.float32).view(np.uint8)
        for d, code in codes.items():
            e[d] = code
        r = np.zeros(64, np.uint16)
        for d, bits in rope.items():
            r[d] = bits
        e[528:656] = r.view(np.uint8)


# e4m3 codes: 1.0 = 0x38, 2.0 = 0x40, 0.5 = 0x30, -1.0 = 0xB8; bf16 1.0 = 0x3F80
def test_single_slot_is_that_entry():
    c = _cache()
    _hand_entries(c, [(5, {0: 0x38, 300: 0x40}, {2: 0x3F80})])
    q = np.zeros((1, 2, 512))
    q[0, 0, 0], q[0, 1, 300] = 3.0, -1.0
    qpe = np.zeros((1, 2, 64))
    qpe[0, 0, 2] = 0.5
    out, lse = M.sparse_mla_decode(q, qpe, c, [[-1, 5, -1]], 0.25)
    kv = np.zeros(512)
    kv[0], kv[300] = 1.0, 2.0
    assert np.array_equal(out[0, 0], kv) and np.array_equal(out[0, 1], kv)
    assert lse[0, 0] == 0.25 * (3.0 + 0.5) and lse[0, 1] == 0.25 * -2.0


def test_equal_scores_give_the_mean():
    c = _cache()
    _hand_entries(c, [(1, {0: 0x38}, {}), (2, {0: 0x40, 1: 0x30}, {}), (70, {1: 0xB8}, {})])
    out, lse = M.sparse_mla_decode(np.zeros((1, 1, 512)), np.zeros((1, 1, 64)), c, [[1, 2, 70]], 1.0)
    want = np.zeros(512)
    want[0], want[1] = (1.0 + 2.0) / 3, (0.5 - 1.0) / 3
    assert np.allclose(out[0, 0], want, rtol=0, atol=1e-15)
    assert math.isclose(lse[0, 0], math.log(3), rel_tol=1e-15)


def test_two_slots_logistic():
    """out = sigma(s1-s2) kv1 + sigma(s2-s1) kv2, lse = log(e^s1 + e^s2)."""
    c = _cache()
    _hand_entries(c, [(3, {0: 0x38}, {}), (4, {0: 0x40, 5: 0x38}, {})])
    q = np.zeros((1, 1, 512))
    q[0, 0, 0] = 1.0          # s1 = 1*1.0, s2 = 1*2.0 (times sm_scale)
    out, lse = M.sparse_mla_decode(q, np.zeros((1, 1, 64)), c, [[4, 3]], 0.7)
    s1, s2 = 0.7 * 1.0, 0.7 * 2.0
    p1 = 1.0 / (1.0 + math.exp(s2 - s1))
    assert math.isclose(out[0, 0, 0], p1 * 1.0 + (1 - p1) * 2.0, rel_tol=1e-14)
    assert math.isclose(out[0, 0, 5], (1 - p1) * 1.0, rel_tol=1e-14)
    assert math.isclose(lse[0, 0], math.log(math.exp(s1) + math.exp(s2)), rel_tol=1e-14)


def test_order_padding_and_out_of_range_invariance():
    rng = np.random.default_rng(3)
    c = _cache(num_blocks=3)
    kv = rng.standard_normal((6, 512)).astype(np.float32)
    kpe = rng.standard_normal((6, 64)).astype(np.float32)
    slots = [2, 9, 64, 100, 150, 191]
    M.mla_cache_write(kv, kpe, slots, c)
    q = rng.standard_normal((1, 3, 512))
    qpe = rng.standard_normal((1, 3, 64))
    a, la = M.sparse_mla_decode(q, qpe, c, [slots], 0.05)
    b, lb = M.sparse_mla_decode(q, qpe, c, [[191, -1, 64, 2, 10 ** 6, 150, 9, -5, 100]], 0.05)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-13) and np.allclose(la, lb, rtol=1e-13)


def test_empty_row():
    out, lse = M.sparse_mla_decode(np.ones((2, 1, 512)), np.ones((2, 1, 64)), _cache(), [[-1, -1], [-1, 10 ** 9]], 1.0)
    assert not out.any() and np.all(np.isneginf(lse))


def test_softmax_shift_invariance():
    """Adding the same constant to every score (a q_pe component against a
    RoPE dim all slots share) changes lse by that constant and out not at all."""
    rng = np.random.default_rng(4)
    c = _cache()
    kv = rng.standard_normal((4, 512)).astype(np.float32)
    kpe = np.zeros((4, 64), np.float32)
    kpe[:, 7] = 1.0
    M.mla_cache_write(kv, kpe, [1, 2, 3, 4], c)
    q = rng.standard_normal((1, 1, 512))
    qpe0 = np.zeros((1, 1, 64))
    qpe1 = qpe0.copy()
    qpe1[0, 0, 7] = 5.0
    a, la = M.sparse_mla_decode(q, qpe0, c, [[1, 2, 3, 4]], 0.3)
    b, lb = M.sparse_mla_decode(q, qpe1, c, [[1, 2, 3, 4]], 0.3)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-14)
    assert math.isclose(lb[0, 0] - la[0, 0], 0.3 * 5.0, rel_tol=1e-12)
