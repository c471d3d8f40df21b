"""The fused decode step (paged_mqa_topk_slots): the logits kernel counts a
histogram of each row's logits and the selection starts from it.  Logits
against the oracle's, indices and slot ids against the oracle's top-k and
slot map over the GPU's logits (bit-exact), and the histogram back at zero
after every call; then stale histograms, ties, NaN rows, the shapes that fall
back to the two plain calls, and a captured graph."""
import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_indexer_paged_amd import binding as sai
from sparse_attention_indexer_paged_amd import synth

from gpu_common import DEV, GpuWorkload, OracleWorkload, assert_logits_close, bf16_tensor

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _q(g, wl):
    return g.q_fp8.view(wl.batch, max(wl.next_n, 1), 64, 128)


def _check(wl, g, res, k, width, o=None):
    logits, row_len, row_req, idx, slots = res
    torch.cuda.synchronize()
    nn = max(wl.next_n, 1)
    lim, req = O.decode_limits(wl.ctx, nn)
    lim = np.minimum(lim.clip(min=0), width)
    assert np.array_equal(row_len.cpu().numpy(), lim)
    assert np.array_equal(row_req.cpu().numpy(), req)
    gl = logits.cpu().numpy()
    if o is not None:
        ref = O.paged_mqa_logits(o.q_codes.reshape(wl.batch, nn, 64, 128), o.w_eff, o.pool,
                                 wl.block_table, wl.ctx, nn, width)
        assert_logits_close(gl, ref, wl.name)
    want = O.topk_rows(gl, lim, k)
    assert np.array_equal(idx.cpu().numpy(), want)
    assert np.array_equal(slots.cpu().numpy(), O.topk_to_global_slots(want, req, wl.block_table))


@pytest.mark.parametrize("next_n,k", [(1, 2048), (2, 2048), (4, 100), (3, 1)])
def test_fused_step_matches_oracle(next_n, k):
    """Ragged contexts (shorter than k, one block, several thousand keys),
    every next_n; the histogram is zero after the call and a second call
    with it gives the same result."""
    ctx = [5000, 2047 + next_n, 64, 9000, next_n, 12000, 3001][: 7 if next_n < 4 else 6]
    _say(f"paged_mqa_topk_slots: next_n={next_n}, k={k}, contexts {ctx}")
    wl = synth.custom(len(ctx), next_n, ctx, num_blocks=600, bt_width=200, seed=300 + next_n)
    g = GpuWorkload(wl)
    o = OracleWorkload(wl)
    rows = len(ctx) * next_n
    assert sai.paged_mqa_topk_hist_bytes(rows, wl.width) == rows * 4096
    hist = torch.zeros((rows, 1024), dtype=torch.int32, device=DEV)
    res = sai.paged_mqa_topk_slots(_q(g, wl), g.w_eff, g.pool, g.block_table, g.ctx, k, hist=hist)
    _check(wl, g, res, k, wl.width, o)
    assert int(hist.abs().sum()) == 0
    again = sai.paged_mqa_topk_slots(_q(g, wl), g.w_eff, g.pool, g.block_table, g.ctx, k, hist=hist)
    torch.cuda.synchronize()
    for a, b in zip(res, again):
        assert torch.equal(a, b)
    assert int(hist.abs().sum()) == 0


def test_fused_step_equals_the_two_plain_calls_at_decode_shape():
    """64 requests of 4096..16384 keys (the decode workload's shape): the
    fused step's outputs equal paged_mqa_logits + topk_rows_slots exactly."""
    wl = synth.make(1)
    _say(f"paged_mqa_topk_slots vs the two calls: {wl.name}")
    g = GpuWorkload(wl, poison=False)
    q = _q(g, wl)
    fused = sai.paged_mqa_topk_slots(q, g.w_eff, g.pool, g.block_table, g.ctx, 2048)
    logits, row_len, row_req = sai.paged_mqa_logits(q, g.w_eff, g.pool, g.block_table, g.ctx)
    idx, slots = sai.topk_rows_slots(logits, row_len, row_req, g.block_table, 2048)
    torch.cuda.synchronize()
    for a, b in zip(fused, (logits, row_len, row_req, idx, slots)):
        assert torch.equal(a, b)
    # every row against the oracle's top-k over these logits
    gl = logits.cpu().numpy()
    want = O.topk_rows(gl, row_len.cpu().numpy(), 2048)
    assert np.array_equal(fused[3].cpu().numpy(), want)


def test_fused_step_stale_histogram_is_still_exact():
    """A histogram left non-zero (garbage counts, counts of another batch)
    changes no result, and the call leaves it at zero."""
    ctx = [7000, 3000, 11000, 2500]
    _say(f"paged_mqa_topk_slots: stale histograms, contexts {ctx}")
    wl = synth.custom(4, 1, ctx, num_blocks=400, bt_width=180, seed=311)
    g = GpuWorkload(wl)
    gen = torch.Generator(device="cpu").manual_seed(5)
    for hist in (torch.randint(0, 5000, (4, 1024), generator=gen, dtype=torch.int32),
                 torch.full((4, 1024), 3, dtype=torch.int32),
                 torch.zeros((4, 1024), dtype=torch.int32).index_fill_(1, torch.tensor([1023]), 1 << 20)):
        hist = hist.to(DEV)
        res = sai.paged_mqa_topk_slots(_q(g, wl), g.w_eff, g.pool, g.block_table, g.ctx, 2048, hist=hist)
        _check(wl, g, res, 2048, wl.width)
        assert int(hist.abs().sum()) == 0


def test_fused_step_ties_and_nan_rows():
    """Request 0: every key the same (the whole row ties, the k-th bin holds
    it all); request 1: two distinct keys alternating; request 2: a block
    id outside the pool (NaN columns, which rank last)."""
    ctx = [6000, 5000, 4000]
    _say(f"paged_mqa_topk_slots: ties and NaN rows, contexts {ctx}")
    wl = synth.custom(3, 2, ctx, num_blocks=300, bt_width=100, seed=313)
    g = GpuWorkload(wl)
    k0 = wl.k_request(0)
    same = np.repeat(k0[:1], ctx[0], axis=0)
    sai.indexer_k_cache_write(bf16_tensor(same), torch.from_numpy(wl.slots_request(0)).to(DEV), g.pool)
    k1 = wl.k_request(1)
    two = np.where((np.arange(ctx[1]) % 2 == 0)[:, None], k1[:1], k1[1:2])
    sai.indexer_k_cache_write(bf16_tensor(two), torch.from_numpy(wl.slots_request(1)).to(DEV), g.pool)
    bt = g.block_table.clone()
    bt[2, 10] = wl.num_blocks + 5
    wl.block_table = bt.cpu().numpy()
    res = sai.paged_mqa_topk_slots(_q(g, wl), g.w_eff, g.pool, bt, g.ctx, 2048)
    _check(wl, g, res, 2048, wl.width)
    gl = res[0].cpu().numpy()
    assert np.unique(gl[0, :ctx[0] - 1]).size == 1
    assert np.isnan(gl[4, 640:704]).all()


def test_fused_step_odd_width_and_fallback_shapes():
    """An odd row pitch (4-byte loads in the selection), rows wider than
    16384 columns and 512 rows or more: the last two take the two plain
    calls and leave a passed histogram untouched."""
    wl = synth.custom(5, 1, [3000, 9000, 1, 2100, 5000], num_blocks=400, bt_width=150, seed=317)
    g = GpuWorkload(wl)
    width = wl.width + 3
    _say(f"paged_mqa_topk_slots: width {width}")
    res = sai.paged_mqa_topk_slots(_q(g, wl), g.w_eff, g.pool, g.block_table, g.ctx, 2048, width=width)
    _check(wl, g, res, 2048, width)

    wl = synth.custom(3, 2, [30000, 17000, 2000], num_blocks=900, bt_width=500, seed=319)
    g = GpuWorkload(wl)
    _say(f"paged_mqa_topk_slots: width {wl.width} (segmented selection)")
    assert sai.paged_mqa_topk_hist_bytes(6, wl.width) == 0
    marker = torch.full((6, 1024), 9, dtype=torch.int32, device=DEV)
    res = sai.paged_mqa_topk_slots(_q(g, wl), g.w_eff, g.pool, g.block_table, g.ctx, 2048, hist=marker)
    _check(wl, g, res, 2048, wl.width)
    assert bool((marker == 9).all())

    ctx = list(np.random.default_rng(7).integers(1, 4000, size=260))
    wl = synth.custom(260, 2, ctx, num_blocks=260 * 63, bt_width=63, seed=321)
    g = GpuWorkload(wl, poison=False)
    _say("paged_mqa_topk_slots: 520 rows (many-row selection)")
    assert sai.paged_mqa_topk_hist_bytes(520, wl.width) == 0
    res = sai.paged_mqa_topk_slots(_q(g, wl), g.w_eff, g.pool, g.block_table, g.ctx, 2048)
    _check(wl, g, res, 2048, wl.width)


def test_fused_step_graph_capture_replays_match_eager():
    """The fused step with a kept histogram captured in a hipGraph: every
    replay equals the eager result, with eager work between replays, and the
    histogram is zero after each."""
    wl = synth.custom(8, 2, [9000, 4000, 16000, 2049, 7000, 100, 12000, 3000], num_blocks=1200,
                      bt_width=256, seed=323)
    _say("hipGraph capture of paged_mqa_topk_slots, batch 8, next_n 2")
    g = GpuWorkload(wl)
    q = _q(g, wl)
    hist = torch.zeros((16, 1024), dtype=torch.int32, device=DEV)
    eager = [t.clone() for t in sai.paged_mqa_topk_slots(q, g.w_eff, g.pool, g.block_table, g.ctx, 2048,
                                                         hist=hist)]
    torch.cuda.synchronize()
    _check(wl, g, eager, 2048, wl.width)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sai.paged_mqa_topk_slots(q, g.w_eff, g.pool, g.block_table, g.ctx, 2048, hist=hist)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = sai.paged_mqa_topk_slots(q, g.w_eff, g.pool, g.block_table, g.ctx, 2048, hist=hist)
    for rep in range(3):
        for t in out:
            t.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(out, eager):
            assert torch.equal(a, b), f"replay {rep} differs"
        assert int(hist.abs().sum()) == 0
        again = sai.paged_mqa_topk_slots(q, g.w_eff, g.pool, g.block_table, g.ctx, 2048, hist=hist)
        torch.cuda.synchronize()
        for a, b in zip(again, eager):
            assert torch.equal(a, b)
