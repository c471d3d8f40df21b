"""The fp8 quantisers of the producers (K-cache write, query producer, MLA
cache write) on values whose quotient x / scale lies at or next to a
rounding tie of the e4m3 grid: there a quotient computed any other way than
the IEEE float32 division the oracle takes (for instance x * (1 / scale))
rounds to a different code, so these rows pin the kernels' division and
their ties-to-even.  Codes, scales and folded weights are compared with the
oracle bit for bit."""
import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_indexer_paged_amd import binding as sai
from sparse_attention_indexer_paged_amd import synth

from gpu_common import DEV, bf16_tensor

pytestmark = pytest.mark.gpu

# row maxima 1.75 * 2^k: their float32 scale 2^(k-8) is exact, so many
# quotients land exactly on ties (ties to even through the fallback)
EXACT_AMAX = [1.75, 7.0, 0.4375, 112.0]


def _say(msg):
    print(msg, flush=True)


def _pairs():
    """(row maximum, value) bf16 pairs, both positive: for every bf16
    maximum in [2^-7, 2^15) the values within 12 binades below it whose code
    through a multiply by fl32(1/scale) differs from the code of
    fl32(x / scale); and for the exact-scale maxima the values whose
    quotient is a tie or next to one."""
    out = []
    for ab in list(range(0x3C00, 0x4700)) + [int(synth.f32_to_bf16_bits(np.array([a], np.float32))[0])
                                             for a in EXACT_AMAX]:
        amax = synth.bf16_bits_to_f32(np.array([ab], np.uint16))[0]
        bits = np.arange(max(1, ab - 0x0C00), ab + 1, dtype=np.uint16)
        x = synth.bf16_bits_to_f32(bits)
        scale = np.maximum(amax * O.INV_448, O.FLT_MIN).astype(np.float32)
        inv = (np.float32(1.0) / scale).astype(np.float32)
        y_div = (x / scale).astype(np.float32)
        pick = O.fp8_encode(y_div) != O.fp8_encode((x * inv).astype(np.float32))
        if (scale.view(np.uint32) & 0x7FFFFF) == 0:
            u = y_div.view(np.uint32)
            pick |= (u >= 0x3C800000) & (np.abs((u & 0xFFFFF).astype(np.int64) - 0x80000) <= 4)
        out += [(ab, int(b)) for b in bits[pick]]
    return out


def _rows(width, seed, tile=128, limit=None):
    """Rows of `width` bf16 values in tiles of `tile` (one quantiser scale
    each: 128 for the K row and the MLA tile, the whole token for the
    query), one (maximum, value) pair per tile: the maximum, the value with
    both signs, -0 and +0, and small filler values."""
    pairs = _pairs()[:limit]
    rng = np.random.default_rng(seed)
    tiles = width // tile
    n_rows = -(-len(pairs) // tiles)
    out = np.zeros((n_rows * tiles, tile), np.uint16)
    for t, (ab, xb) in enumerate(pairs):
        amax = synth.bf16_bits_to_f32(np.array([ab], np.uint16))[0]
        fill = synth.f32_to_bf16_bits((rng.random(tile - 3) * amax / 64).astype(np.float32))
        out[t, :3] = [ab, xb, xb | 0x8000]
        out[t, 3:] = fill | ((rng.random(tile - 3) < 0.5).astype(np.uint16) << 15)
        out[t, 3:5] = [0x8000, 0x0000]             # -0 and +0 beside nonzero values: codes 0x80, 0x00
        out[t] = out[t][rng.permutation(tile)]
    for t in range(len(pairs), out.shape[0]):      # padding tiles reuse the first pair
        out[t] = out[0]
    return out.reshape(n_rows, width), len(pairs)


def test_hard_values_exist():
    """The search finds values a plain multiply would get wrong (else the
    cases below pin nothing)."""
    pairs = _pairs()
    assert len(pairs) > 500, len(pairs)


def test_k_cache_write_ties_bit_exact():
    rows, _ = _rows(128, seed=1)
    _say(f"indexer_k_cache_write: {rows.shape[0]} rows of tie-adjacent values")
    nb = -(-rows.shape[0] // 64) + 2
    slots = np.random.default_rng(2).permutation(nb * 64)[: rows.shape[0]].astype(np.int64)
    pool = torch.zeros((nb, synth.BLOCK_BYTES), dtype=torch.uint8, device=DEV)
    sai.indexer_k_cache_write(bf16_tensor(rows), torch.from_numpy(slots).to(DEV), pool)
    torch.cuda.synchronize()
    want = O.k_cache_write(synth.bf16_bits_to_f32(rows), slots, np.zeros((nb, synth.BLOCK_BYTES), np.uint8))
    assert np.array_equal(pool.cpu().numpy(), want)


def test_q_quant_ties_bit_exact():
    rows, _ = _rows(64 * 128, seed=3, tile=64 * 128, limit=300)
    _say(f"indexer_q_quant: {rows.shape[0]} tokens of tie-adjacent values")
    q = rows.reshape(-1, 64, 128)
    w = np.random.default_rng(4).standard_normal((q.shape[0], 64)).astype(np.float32)
    qf, weff, qs = sai.indexer_q_quant(bf16_tensor(q), torch.from_numpy(w).to(DEV))
    torch.cuda.synchronize()
    codes, w_want, s_want = O.quantize_q(synth.bf16_bits_to_f32(q), w)
    assert np.array_equal(qf.cpu().numpy(), codes)
    assert np.array_equal(weff.cpu().numpy().view(np.int32), w_want.view(np.int32))
    assert np.array_equal(qs.cpu().numpy().view(np.int32), s_want.view(np.int32))


def test_mla_cache_write_ties_bit_exact():
    rows, _ = _rows(512, seed=5)
    _say(f"mla_cache_write: {rows.shape[0]} latent rows of tie-adjacent tiles")
    rng = np.random.default_rng(6)
    pe = synth.f32_to_bf16_bits(rng.standard_normal((rows.shape[0], 64)).astype(np.float32))
    bs = 64
    nb = -(-rows.shape[0] // bs) + 2
    slots = rng.permutation(nb * bs)[: rows.shape[0]].astype(np.int64)
    cache = torch.zeros((nb, bs, 656), dtype=torch.uint8, device=DEV)
    sai.mla_cache_write(bf16_tensor(rows), bf16_tensor(pe), torch.from_numpy(slots).to(DEV), cache)
    torch.cuda.synchronize()
    want = O.mla.mla_cache_write(synth.bf16_bits_to_f32(rows), synth.bf16_bits_to_f32(pe), slots,
                                 np.zeros((nb, bs, 656), np.uint8))
    assert np.array_equal(cache.cpu().numpy(), want)
