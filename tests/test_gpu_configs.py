"""Parity at the full workload sizes, in the launch configuration the benchmark
times: logits on sampled rows against the oracle (which computes those rows
one by one), top-k and slot ids on every row, bit-exact, against the
oracle's selection run on the GPU's own logits."""
import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_indexer_paged_amd import binding as sai
from sparse_attention_indexer_paged_amd import synth

from gpu_common import DEV, GpuWorkload, OracleWorkload, assert_logits_close

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _decode_config(cfg, sample_requests):
    wl = synth.make(cfg)
    _say(f"config {cfg} ({wl.name}): building on GPU")
    g = GpuWorkload(wl)
    nn = wl.next_n
    q = g.q_fp8.view(wl.batch, nn, 64, 128)
    logits, idx, slots = sai.decode_indexer(q, g.w_eff, g.pool, g.block_table, g.ctx)
    row_len, row_req = O.decode_limits(wl.ctx, nn)
    torch.cuda.synchronize()
    _say(f"config {cfg}: oracle on requests {sample_requests}")
    o = OracleWorkload(wl, requests=sample_requests)
    rows = [b * nn + j for b in sample_requests for j in range(nn)]
    ref = O.paged_mqa_logits(o.q_codes.reshape(wl.batch, nn, 64, 128), o.w_eff, o.pool,
                             wl.block_table, wl.ctx, nn, wl.width, rows=rows)
    gl = logits.cpu().numpy()
    worst = assert_logits_close(gl[rows], ref[rows], wl.name)
    _say(f"config {cfg}: logits ok on {len(rows)} rows, worst err/tol {worst:.3g}")
    want = O.topk_rows(gl, row_len, 2048)
    assert np.array_equal(idx.cpu().numpy(), want)
    want_s = O.topk_to_global_slots(want, row_req, wl.block_table)
    assert np.array_equal(slots.cpu().numpy(), want_s)
    # report (not assert) overlap with the selection on the oracle's own logits
    ref_top = O.topk_rows(ref[rows], row_len[rows], 2048)
    got = want[rows]
    ov = np.mean([len(set(a[a >= 0]) & set(b[b >= 0])) / max(1, (b >= 0).sum())
                  for a, b in zip(got, ref_top)])
    _say(f"config {cfg}: top-k bit-exact on all rows; overlap with oracle-logit top-k {ov:.5f}")
    return wl, gl


def test_config1_decode_b64():
    _decode_config(1, sample_requests=[0, 1, 17, 40, 63])


def test_config2_mtp_decode_b128_next_n2():
    wl = synth.make(2)
    short = [b for b in range(wl.batch) if wl.ctx[b] < 2048][:3]
    long_ = [int(np.argmax(wl.ctx)), int(np.argmin(np.where(wl.ctx >= 2048, wl.ctx, 1 << 30)))]
    _, gl = _decode_config(2, sample_requests=sorted(set(short + long_ + [5])))
    assert (wl.ctx < 2048).sum() == 32


def test_config4_long_decode_b32_128k():
    _decode_config(4, sample_requests=[0, 31])


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
    o = OracleWorkload(wl)
    rv, rs = O.gather_indexer_k(o.pool, wl.block_table, wl.cu_seq_lens, total)
    assert np.array_equal(kv.cpu().numpy(), rv)
    assert np.array_equal(ks.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    rows = [0, 1, 2, 63, 64, 65, 1000, 2046, 2047, 2048, 4095, 4096, 6000, 8190, 8191]
    ref = O.mqa_logits(o.q_codes, o.w_eff, rv, rs, wl.cu_seq_lens, wl.width, rows=rows)
    gl = logits.cpu().numpy()
    worst = assert_logits_close(gl[rows], ref[rows], wl.name)
    _say(f"config 3: logits ok on {len(rows)} rows, worst err/tol {worst:.3g}")
    rl = row_len.cpu().numpy()
    assert np.array_equal(rl, np.arange(1, total + 1))
    want = O.topk_rows(gl, rl, 2048)
    assert np.array_equal(idx.cpu().numpy(), want)
    assert np.array_equal(slots.cpu().numpy(), O.topk_to_global_slots(want, row_req.cpu().numpy(),
                                                                     wl.block_table))


def test_config5_chunked_prefill():
    """Four prompts at contexts 16384 / 8192 / 6144 / 2048, each scoring its
    last 2048 tokens against the gathered context (the bench's chunked-prefill
    workload at full size): logits on sampled rows, row limits on every row,
    top-k and slot ids on sampled rows."""
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
    o = OracleWorkload(wl)
    rv, rs = O.gather_indexer_k(o.pool, wl.block_table, wl.cu_seq_lens, total_k)
    assert np.array_equal(kv.cpu().numpy(), rv)
    rows = [0, 1, 2047, 2048, 2049, 4095, 4096, 5000, 6143, 6144, 6145, 8190, 8191]
    ref = O.mqa_logits_chunked(o.q_codes, o.w_eff, rv, rs, wl.cu_q, wl.cu_seq_lens, wl.width, rows=rows)
    gl = logits.cpu().numpy()
    worst = assert_logits_close(gl[rows], ref[rows], wl.name)
    _say(f"config 5: logits ok on {len(rows)} rows, worst err/tol {worst:.3g}")
    n_q = np.diff(wl.cu_q)
    want_len = np.concatenate([int(c) - int(n) + np.arange(int(n)) + 1 for c, n in zip(wl.ctx, n_q)])
    assert np.array_equal(row_len.cpu().numpy(), want_len)
    assert np.array_equal(row_req.cpu().numpy(), np.repeat(np.arange(wl.batch), n_q))
    want = O.topk_rows(gl[rows], want_len[rows], 2048)
    assert np.array_equal(idx.cpu().numpy()[rows], want)
    assert np.array_equal(slots.cpu().numpy()[rows],
                          O.topk_to_global_slots(want, row_req.cpu().numpy()[rows], wl.block_table))
