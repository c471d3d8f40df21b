"""Parity at the full workload sizes, in the launch configuration the benchmark
times.

Decode workloads (batch 64 / MTP batch 128 x 2 / long-context batch 32): the
logits of EVERY row against the oracle, which scores each request in well
under a second.  Prefill workloads (8192 tokens; four 2048-token chunks):
every 8th row plus the rows at tile, key-chunk and request boundaries.  Top-k
and slot ids on every row of every workload, bit-exact, against the oracle's
selection run on the GPU's own logits."""
import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_indexer_paged_amd import binding as sai
from sparse_attention_indexer_paged_amd import synth

from gpu_common import DEV, GpuWorkload, OracleWorkload, assert_logits_close, oracle_topk

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _decode_config(cfg):
    wl = synth.make(cfg)
    _say(f"config {cfg} ({wl.name}): building on GPU")
    g = GpuWorkload(wl)
    nn = wl.next_n
    q = g.q_fp8.view(wl.batch, nn, 64, 128)
    logits, idx, slots = sai.decode_indexer(q, g.w_eff, g.pool, g.block_table, g.ctx)
    row_len, row_req = O.decode_limits(wl.ctx, nn)
    torch.cuda.synchronize()
    gl, gi, gs = logits.cpu().numpy(), idx.cpu().numpy(), slots.cpu().numpy()
    del g, logits, idx, slots
    _say(f"config {cfg}: oracle cache and logits of all {wl.rows} rows")
    o = OracleWorkload(wl)
    ref = O.paged_mqa_logits(o.q_codes.reshape(wl.batch, nn, 64, 128), o.w_eff, o.pool,
                             wl.block_table, wl.ctx, nn, wl.width)
    worst = assert_logits_close(gl, ref, wl.name)
    _say(f"config {cfg}: logits ok on all {wl.rows} rows, worst err/tol {worst:.3g}")
    want = oracle_topk(gl, row_len)
    assert np.array_equal(gi, want)
    want_s = O.topk_to_global_slots(want, row_req, wl.block_table)
    assert np.array_equal(gs, want_s)
    # report (not assert) overlap with the selection on the oracle's own logits
    ref_top = oracle_topk(ref, row_len)
    ov = np.mean([len(set(a[a >= 0]) & set(b[b >= 0])) / max(1, (b >= 0).sum())
                  for a, b in zip(want, ref_top)])
    _say(f"config {cfg}: top-k bit-exact on all rows; overlap with oracle-logit top-k {ov:.5f}")
    return wl, gl


def _prefill_rows(cu_q, stride=8):
    """Every ``stride``-th row, the rows on both sides of every 64-row tile
    and 1024-column key-chunk boundary, and the first, second, last and
    second-to-last rows of every request."""
    total = int(cu_q[-1])
    rows = set(range(0, total, stride))
    for r in range(total):
        if r % 64 in (1, 63) or r % 1024 in (1023, 1):
            rows.add(r)
    for a, b in zip(cu_q[:-1], cu_q[1:]):
        a, b = int(a), int(b)
        if b > a:
            rows.update({a, min(a + 1, b - 1), b - 1, max(b - 2, a)})
    return sorted(r for r in rows if 0 <= r < total)


def test_config1_decode_b64():
    _decode_config(1)


def test_config2_mtp_decode_b128_next_n2():
    wl, _ = _decode_config(2)
    assert (wl.ctx < 2048).sum() == 32


def test_config4_long_decode_b32_128k():
    _decode_config(4)


def test_config3_prefill_8192():
    wl = synth.make(3)
    _say("config 3 (prefill 8192): building on GPU")
    g = GpuWorkload(wl)
    total = wl.total_tokens
    kv, ks = sai.gather_indexer_k(g.pool, g.block_table, g.cu, total)
    logits, row_len, row_req = sai.mqa_logits(g.q_fp8, g.w_eff, kv, ks, g.cu, wl.width)
    idx = sai.topk_rows(logits, row_len, 2048)
    slots = sai.topk_to_global_slots(idx, row_req, g.block_table)
    torch.cuda.synchronize()
    gl, gi, gs = logits.cpu().numpy(), idx.cpu().numpy(), slots.cpu().numpy()
    gkv, gks = kv.cpu().numpy(), ks.cpu().numpy()
    rl, rq = row_len.cpu().numpy(), row_req.cpu().numpy()
    del g, kv, ks, logits, idx, slots
    rows = _prefill_rows(wl.cu_q)
    _say(f"config 3: oracle on {len(rows)} rows")
    o = OracleWorkload(wl, q_rows=rows)
    rv, rs = O.gather_indexer_k(o.pool, wl.block_table, wl.cu_seq_lens, total)
    assert np.array_equal(gkv, rv)
    assert np.array_equal(gks.view(np.uint32), rs.view(np.uint32))
    ref = O.mqa_logits(o.q_codes, o.w_eff, rv, rs, wl.cu_seq_lens, wl.width, rows=rows)
    worst = assert_logits_close(gl[rows], ref[rows], wl.name)
    _say(f"config 3: logits ok on {len(rows)} rows, worst err/tol {worst:.3g}")
    assert np.array_equal(rl, np.arange(1, total + 1))
    assert np.array_equal(rq, np.zeros(total, np.int32))
    want = oracle_topk(gl, rl)
    assert np.array_equal(gi, want)
    assert np.array_equal(gs, O.topk_to_global_slots(want, rq, wl.block_table))
    _say("config 3: top-k and slot ids bit-exact on all rows")


def test_config5_chunked_prefill():
    """Four prompts at contexts 16384 / 8192 / 6144 / 2048, each scoring its
    last 2048 tokens against the gathered context (the bench's chunked-prefill
    workload at full size): logits on every 8th row and the boundary rows, row
    limits, top-k and slot ids on every row."""
    wl = synth.make(5)
    _say("config 5 (chunked prefill): building on GPU")
    g = GpuWorkload(wl)
    total_k = wl.total_tokens
    cu_q = torch.from_numpy(wl.cu_q).to(DEV)
    kv, ks = sai.gather_indexer_k(g.pool, g.block_table, g.cu, total_k)
    logits, row_len, row_req = sai.mqa_logits_chunked(g.q_fp8, g.w_eff, kv, ks, cu_q, g.cu, wl.width)
    idx = sai.topk_rows(logits, row_len, 2048)
    slots = sai.topk_to_global_slots(idx, row_req, g.block_table)
    torch.cuda.synchronize()
    gl, gi, gs = logits.cpu().numpy(), idx.cpu().numpy(), slots.cpu().numpy()
    gkv = kv.cpu().numpy()
    rl, rq = row_len.cpu().numpy(), row_req.cpu().numpy()
    del g, kv, ks, logits, idx, slots
    rows = _prefill_rows(wl.cu_q)
    _say(f"config 5: oracle on {len(rows)} rows")
    o = OracleWorkload(wl, q_rows=rows)
    rv, rs = O.gather_indexer_k(o.pool, wl.block_table, wl.cu_seq_lens, total_k)
    assert np.array_equal(gkv, rv)
    ref = O.mqa_logits_chunked(o.q_codes, o.w_eff, rv, rs, wl.cu_q, wl.cu_seq_lens, wl.width, rows=rows)
    worst = assert_logits_close(gl[rows], ref[rows], wl.name)
    _say(f"config 5: logits ok on {len(rows)} rows, worst err/tol {worst:.3g}")
    n_q = np.diff(wl.cu_q)
    want_len = np.concatenate([int(c) - int(n) + np.arange(int(n)) + 1 for c, n in zip(wl.ctx, n_q)])
    assert np.array_equal(rl, want_len)
    assert np.array_equal(rq, np.repeat(np.arange(wl.batch), n_q))
    want = oracle_topk(gl, want_len)
    assert np.array_equal(gi, want)
    assert np.array_equal(gs, O.topk_to_global_slots(want, rq, wl.block_table))
    _say("config 5: top-k and slot ids bit-exact on all rows")
