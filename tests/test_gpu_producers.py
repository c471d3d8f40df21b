"""Fused producers (rotary embedding + fp8 quantiser + cache write / weight
fold) on the GPU against the oracle, bit-exact: cache bytes, query codes,
folded weights and scales (NaN results compared by bit pattern)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_indexer_paged_amd import binding as sai
from sparse_attention_indexer_paged_amd import synth

from gpu_common import DEV, assert_logits_close, bf16_tensor

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _tables(P, rope_dim, base=10000.0):
    half = max(rope_dim // 2, 1)
    f = base ** (-2.0 * np.arange(half) / max(rope_dim, 1))
    ang = np.arange(P)[:, None] * f[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _bits(t):
    return t.contiguous().view(torch.int32).cpu().numpy() if t.dtype == torch.float32 else t.cpu().numpy()


@pytest.mark.parametrize("rope_dim", [64, 128, 2])
def test_k_rope_cache_write_bit_exact(rope_dim):
    _say(f"indexer_k_rope_cache_write: rope_dim {rope_dim}")
    wl = synth.custom(3, 1, [300, 65, 1000], num_blocks=40, bt_width=20, seed=71 + rope_dim)
    k = wl.k_all()
    slots = wl.slot_mapping().copy()
    n = len(slots)
    P = 1200
    rng = np.random.default_rng(rope_dim)
    pos = rng.integers(0, P, n).astype(np.int64)
    pos[[5, 77, 400]] = [P, -1, P + 1000]          # outside the table: NaN codes and scale
    slots[[6, 300]] = -1                            # skipped
    c, s = _tables(P, rope_dim)
    # rows inside a wider tensor (row stride 136 elements)
    wide = np.zeros((n, 136), np.uint16)
    wide[:, :128] = k
    kt = bf16_tensor(wide)[:, :128]
    pool = torch.from_numpy(wl.poisoned_pool()).to(DEV)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    sai.indexer_k_rope_cache_write(kt, T(pos), T(c), T(s), T(slots), pool)
    torch.cuda.synchronize()
    want = O.k_rope_cache_write(synth.bf16_bits_to_f32(k), pos, c, s, rope_dim, slots, wl.poisoned_pool())
    assert np.array_equal(pool.cpu().numpy(), want)


def test_q_rope_quant_bit_exact():
    _say("indexer_q_rope_quant: 37 rows, rope_dim 64, out-of-table positions")
    rng = np.random.default_rng(72)
    T_ = 37
    q = synth.f32_to_bf16_bits(rng.standard_normal((T_, 64, 128)).astype(np.float32))
    w = (rng.standard_normal((T_, 64)) / 64).astype(np.float32)
    P = 500
    pos = rng.integers(0, P, T_).astype(np.int64)
    pos[[3, 20]] = [P, -5]
    c, s = _tables(P, 64)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    qf, weff, qs = sai.indexer_q_rope_quant(bf16_tensor(q), T(pos), T(c), T(s), T(w))
    torch.cuda.synchronize()
    codes, w_eff, scale = O.quantize_q_rope(synth.bf16_bits_to_f32(q), pos, c, s, 64, w)
    assert np.array_equal(qf.cpu().numpy(), codes)
    assert np.array_equal(_bits(weff), w_eff.view(np.int32))
    assert np.array_equal(_bits(qs), scale.view(np.int32))


def test_identity_tables_and_rope_dim_zero_match_the_plain_producers():
    _say("fused producers with identity tables / rope_dim 0 == plain producers")
    rng = np.random.default_rng(73)
    n = 200
    k = bf16_tensor(synth.f32_to_bf16_bits(rng.standard_normal((n, 128)).astype(np.float32)))
    slots = torch.from_numpy(rng.permutation(16 * 64)[:n].astype(np.int64)).to(DEV)
    pos = torch.from_numpy(rng.integers(0, 50, n).astype(np.int64)).to(DEV)
    ones = torch.ones((50, 64), dtype=torch.float32, device=DEV)
    zeros = torch.zeros((50, 64), dtype=torch.float32, device=DEV)
    a = torch.zeros((16, 8448), dtype=torch.uint8, device=DEV)
    b = torch.zeros_like(a)
    c = torch.zeros_like(a)
    sai.indexer_k_cache_write(k, slots, a)
    sai.indexer_k_rope_cache_write(k, pos, ones, zeros, slots, b)
    sai.indexer_k_rope_cache_write(k, pos, ones[:, :0], zeros[:, :0], slots, c, rope_dim=0)
    q = bf16_tensor(synth.f32_to_bf16_bits(rng.standard_normal((9, 64, 128)).astype(np.float32)))
    w = torch.from_numpy(rng.standard_normal((9, 64)).astype(np.float32)).to(DEV)
    p = sai.indexer_q_quant(q, w)
    r = sai.indexer_q_rope_quant(q, pos[:9], ones, zeros, w)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)
    for x, y in zip(p, r):
        assert np.array_equal(_bits(x), _bits(y))


def test_table_rows_zero_gives_nan():
    _say("fused producers with an empty table: every position outside it")
    rng = np.random.default_rng(74)
    k = bf16_tensor(synth.f32_to_bf16_bits(rng.standard_normal((3, 128)).astype(np.float32)))
    slots = torch.tensor([0, 1, 2], dtype=torch.int64, device=DEV)
    pos = torch.tensor([0, 1, 2], dtype=torch.int64, device=DEV)
    table = torch.zeros((1, 32), dtype=torch.float32, device=DEV)   # a real pointer; 0 rows passed
    pool = torch.zeros((1, 8448), dtype=torch.uint8, device=DEV)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert sai.load().indexer_k_rope_cache_write(P(k), 128, P(pos), P(table), P(table), 0, 64, P(slots), 3,
                                                 P(pool), 1, stream) == 0
    torch.cuda.synchronize()
    p = pool.cpu().numpy()[0]
    assert (p[:384] == 0x7F).all() and np.isnan(p[8192:8204].view(np.float32)).all()


def test_fused_producers_feed_the_decode_chain():
    """K and q produced by the fused kernels (positions = token index in the
    request; query j of a request with context c at position c - next_n + j),
    then paged logits -> top-k -> slot ids, against the same chain in the
    oracle."""
    _say("decode chain from the fused producers: 3 requests, next_n 2")
    nn = 2
    wl = synth.custom(3, nn, [700, 130, 2500], num_blocks=80, bt_width=45, seed=75)
    P = 4096
    c, s = _tables(P, 64)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    pool = torch.from_numpy(wl.poisoned_pool()).to(DEV)
    ref_pool = wl.poisoned_pool()
    for b in range(wl.batch):
        kb = wl.k_request(b)
        pos = np.arange(len(kb), dtype=np.int64)
        sai.indexer_k_rope_cache_write(bf16_tensor(kb), T(pos), T(c), T(s), T(wl.slots_request(b)), pool)
        O.k_rope_cache_write(synth.bf16_bits_to_f32(kb), pos, c, s, 64, wl.slots_request(b), ref_pool)
    qpos = np.concatenate([np.arange(nn) + int(cx) - nn for cx in wl.ctx]).astype(np.int64)
    qf, weff, _ = sai.indexer_q_rope_quant(bf16_tensor(wl.q()), T(qpos), T(c), T(s), T(wl.w()))
    bt = T(wl.block_table)
    logits, idx, slots = sai.decode_indexer(qf.view(wl.batch, nn, 64, 128), weff, pool, bt, T(wl.ctx))
    torch.cuda.synchronize()
    assert np.array_equal(pool.cpu().numpy(), ref_pool)
    qc, we, _ = O.quantize_q_rope(synth.bf16_bits_to_f32(wl.q()), qpos, c, s, 64, wl.w())
    assert np.array_equal(qf.cpu().numpy(), qc)
    ref = O.paged_mqa_logits(qc.reshape(wl.batch, nn, 64, 128), we, ref_pool, wl.block_table, wl.ctx, nn,
                             wl.width)
    gl = logits.cpu().numpy()
    assert_logits_close(gl, ref, "fused-producer decode")
    lim, req = O.decode_limits(wl.ctx, nn)
    want = O.topk_rows(gl, lim, 2048)
    assert np.array_equal(idx.cpu().numpy(), want)
    assert np.array_equal(slots.cpu().numpy(), O.topk_to_global_slots(want, req, wl.block_table))


def test_fused_producers_graph_capture_replays_match_eager():
    """Both fused producers captured in one hipGraph: every replay writes the
    bytes the eager calls wrote, with eager work between replays."""
    _say("hipGraph capture of the fused producers")
    rng = np.random.default_rng(76)
    n = 300
    q = bf16_tensor(synth.f32_to_bf16_bits(rng.standard_normal((n, 64, 128)).astype(np.float32)))
    wt = torch.from_numpy((rng.standard_normal((n, 64)) / 64).astype(np.float32)).to(DEV)
    k = bf16_tensor(synth.f32_to_bf16_bits(rng.standard_normal((n, 128)).astype(np.float32)))
    slot_np = rng.permutation(20 * 64)[:n].astype(np.int64)
    slot_np[::37] = -1
    slot = torch.from_numpy(slot_np).to(DEV)
    pos = torch.from_numpy(rng.integers(-2, 600, n).astype(np.int64)).to(DEV)
    cn, sn = _tables(512, 64)
    c, s = torch.from_numpy(cn).to(DEV), torch.from_numpy(sn).to(DEV)
    icache = torch.zeros((20, 8448), dtype=torch.uint8, device=DEV)
    qf = torch.empty((n, 64, 128), dtype=torch.uint8, device=DEV)
    weff = torch.empty((n, 64), dtype=torch.float32, device=DEV)
    qs = torch.empty((n,), dtype=torch.float32, device=DEV)
    outs = (qf, weff, qs, icache)

    def run():
        sai.indexer_q_rope_quant(q, pos, c, s, wt, q_fp8=qf, w_eff=weff, q_scale=qs)
        sai.indexer_k_rope_cache_write(k, pos, c, s, slot, icache)

    def reset():
        qf.fill_(0xA5)
        weff.fill_(-7)
        qs.fill_(-7)
        icache.zero_()

    run()
    torch.cuda.synchronize()
    eager = [_bits(t) for t in outs]
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        run()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        reset()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert np.array_equal(_bits(a), b), f"replay {rep} differs"
        reset()
        run()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert np.array_equal(_bits(a), b)
