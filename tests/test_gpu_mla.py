"""GPU parity of the fp8 MLA cache writer against the CPU oracle (bit-exact
bytes, untouched entries left alone)."""
import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_indexer_paged_amd import binding as sai
from sparse_attention_indexer_paged_amd import synth

from gpu_common import DEV, GpuWorkload, bf16_tensor

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _inputs(n, seed):
    rng = np.random.default_rng(seed)
    kv = rng.standard_normal((n, 512)).astype(np.float32)
    kv *= np.exp(rng.standard_normal((n, 4, 1)) * 4).astype(np.float32).repeat(128, axis=1).reshape(n, 512)
    kv[0, 128:256] = 0.0                          # all-zero tile -> FLT_MIN scale
    kv[1, :128] = -0.0
    kv[2, 256:384] = 3.0                          # constant tile
    kv[3, 384:] *= 1e-30                          # tiny tile (subnormal codes)
    kv[4, 0] = 2.0 ** -133                        # bf16 subnormal next to zeros
    kv[4, 1:128] = 0.0
    kpe = rng.standard_normal((n, 64)).astype(np.float32) * 10
    return synth.f32_to_bf16_bits(kv), synth.f32_to_bf16_bits(kpe)


@pytest.mark.parametrize("block_size,num_blocks", [(64, 6), (16, 20)])
def test_mla_cache_write_bit_exact(block_size, num_blocks):
    _say(f"mla_cache_write: block_size {block_size}, {num_blocks} blocks")
    n = 300
    kv_bits, kpe_bits = _inputs(n, 11 + block_size)
    rng = np.random.default_rng(7)
    nslots = num_blocks * block_size
    slots = rng.permutation(nslots)[:n].astype(np.int64)
    slots[::17] = -1                               # skipped
    slots[5::23] = nslots + np.arange(len(slots[5::23]))   # past the cache: skipped
    cache_np = np.full((num_blocks, block_size, 656), 0xA5, np.uint8)
    ref = O.mla.mla_cache_write(synth.bf16_bits_to_f32(kv_bits), synth.bf16_bits_to_f32(kpe_bits),
                                slots, cache_np.copy())
    cache = torch.from_numpy(cache_np).to(DEV)
    # row strides wider than the used width (kv [n, 576], kpe [n, 80])
    kv_wide = torch.zeros((n, 576), dtype=torch.bfloat16, device=DEV)
    kv_wide[:, :512] = bf16_tensor(kv_bits)
    kpe_wide = torch.zeros((n, 80), dtype=torch.bfloat16, device=DEV)
    kpe_wide[:, :64] = bf16_tensor(kpe_bits)
    sai.mla_cache_write(kv_wide[:, :512], kpe_wide[:, :64], torch.from_numpy(slots).to(DEV), cache)
    got = cache.cpu().numpy()
    if not np.array_equal(got, ref):
        diff = np.argwhere(got != ref)
        raise AssertionError(f"{len(diff)} bytes differ, first at {diff[:5].tolist()}")


# ------------------------------------------------------------ sparse decode
# Tolerance, from the kernel's arithmetic: scores are fp32 sums of exact
# bf16 x bf16 products (each fp8 code and each bf16 input converts exactly),
# so their error is a few fp32 ulps of the summed magnitudes.  The P.V
# product takes each softmax weight times its tile scale rounded to bf16
# (relative error <= 2^-9), which moves out[t,h,d] by at most
# 2^-9 * sum_j p_j |kv_j[d]|.  The bound used, 2^-8 * that sum, leaves room
# for the score and exp2 errors.  lse is a log of an fp32 sum of exp2 values.
def _mla_tol(out_abs):
    return 2.0 ** -8 * out_abs + 1e-30


LSE_ATOL, LSE_RTOL = 1e-4, 1e-5


def _mla_cache(num_blocks, block_size, seed):
    """A cache written by the oracle's writer from seeded bf16 rows whose
    tiles span a wide range of magnitudes."""
    n = num_blocks * block_size
    rng = np.random.default_rng(seed)
    kv = rng.standard_normal((n, 512)).astype(np.float32)
    kv *= np.exp(rng.standard_normal((n, 4, 1)) * 1.5).astype(np.float32).repeat(128, axis=1).reshape(n, 512)
    kpe = rng.standard_normal((n, 64)).astype(np.float32) * 2
    kv = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(kv))
    kpe = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(kpe))
    cache = np.zeros((num_blocks, block_size, 656), np.uint8)
    return O.mla.mla_cache_write(kv, kpe, np.arange(n), cache)


def _mla_query(T, H, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    qn = synth.f32_to_bf16_bits(rng.standard_normal((T, H, 512)).astype(np.float32) * scale)
    qp = synth.f32_to_bf16_bits(rng.standard_normal((T, H, 64)).astype(np.float32) * scale)
    return qn, qp


def _check_decode(qn_bits, qp_bits, cache_np, slots_np, sm_scale, rows=None):
    cache = torch.from_numpy(cache_np).to(DEV)
    out, lse = sai.sparse_mla_decode(bf16_tensor(qn_bits), bf16_tensor(qp_bits), cache,
                                     torch.from_numpy(slots_np).to(DEV), sm_scale)
    torch.cuda.synchronize()
    rows = np.arange(slots_np.shape[0]) if rows is None else rows
    ref, ref_lse, ref_abs = O.mla.sparse_mla_decode(
        synth.bf16_bits_to_f32(qn_bits[rows]), synth.bf16_bits_to_f32(qp_bits[rows]), cache_np,
        slots_np[rows], sm_scale, with_abs=True)
    got = out.cpu().numpy().astype(np.float64)[rows]
    got_lse = lse.cpu().numpy().astype(np.float64)[rows]
    err = np.abs(got - ref)
    tol = _mla_tol(ref_abs)
    bad = ~(err <= tol)
    if bad.any():
        i = np.argwhere(bad)[:5]
        raise AssertionError(f"{bad.sum()} outputs outside tolerance, first {i.tolist()}: "
                             f"got {got[tuple(i.T)]} want {ref[tuple(i.T)]} tol {tol[tuple(i.T)]}")
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(got_lse), fin), "lse finiteness differs"
    assert np.all(got_lse[~fin] == -np.inf)
    assert np.all(got[~fin] == 0.0), "empty rows must give zeros"
    lerr = np.abs(got_lse[fin] - ref_lse[fin])
    assert np.all(lerr <= LSE_ATOL + LSE_RTOL * np.abs(ref_lse[fin])), f"lse max err {lerr.max()}"
    return float((err / np.maximum(tol, 1e-300)).max())


@pytest.mark.parametrize("T,H,K,block_size,num_blocks", [
    (5, 16, 100, 64, 12),    # 16-head workgroups, ragged tail, split path
    (3, 32, 130, 64, 12),    # 16-head workgroups, two groups
    (3, 64, 261, 16, 40),    # 64-head workgroups, block size 16
    (2, 128, 2048, 64, 80),  # full top-k width, two 64-head groups, many splits
    (256, 64, 64, 64, 30),   # 64-head workgroups, one split (no combine)
])
def test_sparse_mla_decode_parity(T, H, K, block_size, num_blocks):
    _say(f"sparse_mla_decode: T {T} H {H} K {K} block_size {block_size}")
    cache_np = _mla_cache(num_blocks, block_size, 100 + H)
    n = num_blocks * block_size
    rng = np.random.default_rng(H + K)
    slots = np.stack([rng.choice(n, K, replace=K > n) for _ in range(T)]).astype(np.int32)
    slots[0, K // 2:] = -1                      # padded row
    if T > 1:
        slots[1, ::7] = -1                      # holes
        slots[1, 3::11] = n + 5                 # past the cache: skipped
        slots[1, 5::13] = -1000
        slots[1, 1] = slots[1, 0]               # repeated id counts twice
    qn, qp = _mla_query(T, H, 7 + K)
    r = _check_decode(qn, qp, cache_np, slots, 1.0 / np.sqrt(576.0))
    _say(f"  worst err / tol = {r:.3f}")


@pytest.mark.parametrize("H", [16, 64])
def test_sparse_mla_decode_empty_and_peaked(H):
    _say(f"sparse_mla_decode: empty rows, k = 0, a peaked softmax, H {H}")
    cache_np = _mla_cache(4, 64, 5)
    qn, qp = _mla_query(3, H, 9, scale=4.0)     # large scores: near one-hot weights
    slots = np.full((3, 70), -1, np.int32)
    slots[1, :40] = np.arange(40)
    slots[2, 69] = 255                          # one slot, last position
    _check_decode(qn, qp, cache_np, slots, 1.0 / np.sqrt(576.0))
    # k = 0: every row empty
    out, lse = sai.sparse_mla_decode(bf16_tensor(qn), bf16_tensor(qp), torch.from_numpy(cache_np).to(DEV),
                                     torch.zeros((3, 0), dtype=torch.int32, device=DEV), 0.1)
    torch.cuda.synchronize()
    assert torch.all(out == 0).item() and torch.all(lse == float("-inf")).item()


@pytest.mark.parametrize("H", [16, 64])
def test_sparse_mla_decode_rising_scores(H):
    """Slots ordered by increasing score, so that the running maximum keeps
    growing across chunks (every rescale path of the online softmax)."""
    _say(f"sparse_mla_decode: rising scores, H {H}")
    T, K, bs, nb = 2, 1000, 64, 20
    cache_np = _mla_cache(nb, bs, 21)
    rng = np.random.default_rng(22)
    base = rng.standard_normal(512).astype(np.float32)
    qn = np.stack([np.stack([base * (1.0 + 0.02 * h) for h in range(H)])] * T)
    qn_bits = synth.f32_to_bf16_bits(qn * 0.5)
    qp_bits = synth.f32_to_bf16_bits(np.zeros((T, H, 64), np.float32))
    q0 = synth.bf16_bits_to_f32(qn_bits[0, 0]).astype(np.float64)
    ids = rng.choice(nb * bs, K, replace=False)
    order = np.argsort([q0 @ O.mla.mla_entry(cache_np, int(i))[0] for i in ids])
    slots = np.stack([ids[order], ids[order[::-1]]]).astype(np.int32)  # rising, falling
    _check_decode(qn_bits, qp_bits, cache_np, slots, 1.0 / np.sqrt(576.0))


@pytest.mark.parametrize("H", [16, 64])
def test_sparse_mla_decode_poisoned_entry_zero(H):
    """Skipped ids (padding, out of range, past the end of a split) must not
    let the bytes of any entry reach the result: entry 0 holds NaN codes, a
    NaN scale and NaN RoPE values, and no row names slot 0."""
    _say(f"sparse_mla_decode: NaN-poisoned entry 0 behind skipped ids, H {H}")
    T, K, bs, nb = 3, 150, 64, 10
    cache_np = _mla_cache(nb, bs, 31)
    cache_np[0, 0, :512] = 0x7F
    cache_np[0, 0, 512:528] = np.frombuffer(np.full(4, np.nan, np.float32).tobytes(), np.uint8)
    cache_np[0, 0, 528:] = 0xFF
    rng = np.random.default_rng(32)
    slots = np.stack([rng.choice(np.arange(1, nb * bs), K, replace=False) for _ in range(T)]).astype(np.int32)
    slots[0, ::3] = -1
    slots[1, 5::9] = nb * bs + 3
    slots[2, 100:] = -1
    qn, qp = _mla_query(T, H, 33)
    _check_decode(qn, qp, cache_np, slots, 1.0 / np.sqrt(576.0))


@pytest.mark.parametrize("T,H", [(2, 64), (256, 64), (3, 16)])
def test_sparse_mla_decode_graph_capture_replays_match_eager(T, H):
    """Captured in a HIP graph (split + combine, one pass, 16-head kernel),
    replayed three times with eager calls in between: every replay equals
    the eager result bit for bit."""
    _say(f"sparse_mla_decode: graph capture, T {T} H {H}")
    K, bs, nb = 300, 64, 12
    cache = torch.from_numpy(_mla_cache(nb, bs, 81)).to(DEV)
    rng = np.random.default_rng(82)
    slots = torch.from_numpy(np.stack([rng.choice(nb * bs, K, replace=False) for _ in range(T)]).astype(np.int32)).to(DEV)
    slots[0, ::4] = -1
    qn, qp = _mla_query(T, H, 83)
    qn, qp = bf16_tensor(qn), bf16_tensor(qp)
    ws_bytes = sai.sparse_mla_workspace_bytes(T, H, K)
    ws = torch.empty((max(ws_bytes, 16),), dtype=torch.uint8, device=DEV)
    out = torch.empty((T, H, 512), dtype=torch.float32, device=DEV)
    lse = torch.empty((T, H), dtype=torch.float32, device=DEV)
    scale = 1.0 / np.sqrt(576.0)
    eo, el = sai.sparse_mla_decode(qn, qp, cache, slots, scale, workspace=ws)
    eo, el = eo.clone(), el.clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sai.sparse_mla_decode(qn, qp, cache, slots, scale, out=out, lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sai.sparse_mla_decode(qn, qp, cache, slots, scale, out=out, lse=lse, workspace=ws)
    for rep in range(3):
        out.fill_(-7.0)
        lse.fill_(-7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eo) and torch.equal(lse, el), f"replay {rep} differs"
        o2, l2 = sai.sparse_mla_decode(qn, qp, cache, slots, scale, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o2, eo) and torch.equal(l2, el)


def test_sparse_mla_decode_full_size_sampled():
    """The decode workload's shape (64 rows, 128 heads, top-2048 over a
    640-block cache), one pass on the GPU, four rows checked."""
    T, H, K, bs, nb = 64, 128, 2048, 64, 640
    _say(f"sparse_mla_decode full size: T {T} H {H} K {K}")
    cache_np = _mla_cache(nb, bs, 3)
    rng = np.random.default_rng(4)
    slots = np.stack([rng.choice(nb * bs, K, replace=False) for _ in range(T)]).astype(np.int32)
    slots[5, 1000:] = -1
    qn, qp = _mla_query(T, H, 6)
    _check_decode(qn, qp, cache_np, slots, 1.0 / np.sqrt(576.0), rows=np.array([0, 5, 31, 63]))


def test_sparse_mla_decode_cache_past_4_gib():
    """A 4.3 GB MLA cache (105 000 blocks of 64 entries): the selected slots
    sit past byte 2^32.  The oracle runs on a compact copy of those entries."""
    nb, bs, T, H, K = 105_000, 64, 2, 64, 300
    _say(f"sparse_mla_decode with a {nb}-block cache (entries past 4 GiB)")
    rng = np.random.default_rng(71)
    lo = (2 ** 32) // 656 + 1
    ids = rng.choice(np.arange(lo, nb * bs), (T, K), replace=False).astype(np.int32)
    ids[1, ::5] = -1
    flat = np.unique(ids[ids >= 0])
    small = _mla_cache(-(-len(flat) // bs), bs, 72)          # oracle-written entries
    ent = small.reshape(-1, 656)[:len(flat)]
    cache = torch.zeros((nb, bs, 656), dtype=torch.uint8, device=DEV)
    cflat = cache.view(-1, 656)
    cflat[torch.from_numpy(flat.astype(np.int64)).to(DEV)] = torch.from_numpy(ent).to(DEV)
    qn, qp = _mla_query(T, H, 73)
    out, lse = sai.sparse_mla_decode(bf16_tensor(qn), bf16_tensor(qp), cache, torch.from_numpy(ids).to(DEV),
                                     1.0 / np.sqrt(576.0))
    torch.cuda.synchronize()
    remap = np.full(ids.shape, -1, np.int32)
    remap[ids >= 0] = np.searchsorted(flat, ids[ids >= 0])
    host = ent.reshape(len(flat), 1, 656)
    ref, ref_lse, ref_abs = O.mla.sparse_mla_decode(synth.bf16_bits_to_f32(qn), synth.bf16_bits_to_f32(qp),
                                                    host, remap, 1.0 / np.sqrt(576.0), with_abs=True)
    got = out.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= _mla_tol(ref_abs))
    assert np.all(np.abs(lse.cpu().numpy() - ref_lse) <= LSE_ATOL + LSE_RTOL * np.abs(ref_lse))
    del cache, cflat
    torch.cuda.empty_cache()


def test_indexer_then_sparse_mla_decode_end_to_end():
    """The whole decode chain: indexer logits -> top-k -> global slot ids ->
    sparse MLA decode over those ids, on one stream; the oracle runs the
    same chain (its top-k on the GPU's logits, as everywhere the selection is
    decided in the kernel's fp32), and the attention output is compared."""
    ctx, nn, H = [3000, 700, 64, 2049], 2, 64
    _say(f"indexer -> sparse MLA decode: contexts {ctx}, next_n {nn}, {H} heads")
    wl = synth.custom(len(ctx), nn, ctx, num_blocks=120, bt_width=60, seed=91)
    g = GpuWorkload(wl)
    logits, idx, slots = sai.decode_indexer(g.q_fp8.view(len(ctx), nn, 64, 128), g.w_eff, g.pool,
                                            g.block_table, g.ctx, k=512)
    mla_np = _mla_cache(wl.num_blocks, 64, 92)
    mla = torch.from_numpy(mla_np).to(DEV)
    qn, qp = _mla_query(wl.rows, H, 93)
    out, lse = sai.sparse_mla_decode(bf16_tensor(qn), bf16_tensor(qp), mla, slots, 1.0 / np.sqrt(576.0))
    torch.cuda.synchronize()
    lim, req = O.decode_limits(wl.ctx, nn)
    want_idx = O.topk_rows(logits.cpu().numpy(), lim, 512)
    want_slots = O.topk_to_global_slots(want_idx, req, wl.block_table)
    assert np.array_equal(idx.cpu().numpy(), want_idx)
    assert np.array_equal(slots.cpu().numpy(), want_slots)
    ref, ref_lse, ref_abs = O.mla.sparse_mla_decode(synth.bf16_bits_to_f32(qn), synth.bf16_bits_to_f32(qp),
                                                    mla_np, want_slots, 1.0 / np.sqrt(576.0), with_abs=True)
    got = out.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= _mla_tol(ref_abs))
    fin = np.isfinite(ref_lse)
    assert np.all(np.abs(lse.cpu().numpy()[fin] - ref_lse[fin]) <= LSE_ATOL + LSE_RTOL * np.abs(ref_lse[fin]))
