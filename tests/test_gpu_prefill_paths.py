"""Prefill logits (mqa_logits / mqa_logits_chunked) through the paths the
workgroup-per-tile kernel takes besides the aligned fast one, against the
oracle: rows written with 4-byte stores (an odd row pitch, a logits base that
is not 16-byte aligned), tiles whose rows are only partly in the request,
requests of one and two tokens, and rows that see no key."""
import ctypes

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


def _p(t, offset_elems=0):
    return ctypes.c_void_p(t.data_ptr() + offset_elems * t.element_size())


@pytest.mark.parametrize("stride,pad", [(333, 0), (336, 1)])
def test_prefill_odd_pitch_and_unaligned_rows(stride, pad):
    """Requests of 301 (a last tile with one row), 2 and 67 tokens.  Rows of
    333 columns (a pitch that is not a multiple of 4), or of 336 columns
    starting one float into the buffer (a base that is not 16-byte aligned):
    both take the 4-byte store path.  The buffer's first `pad` floats keep
    their sentinel."""
    ctx = [301, 2, 67]
    _say(f"mqa_logits: contexts {ctx}, row pitch {stride}, base offset {pad} floats")
    wl = synth.custom(3, 0, ctx, num_blocks=12, bt_width=5, seed=81 + pad)
    g = GpuWorkload(wl)
    o = OracleWorkload(wl)
    total = wl.total_tokens
    kv, ks = sai.gather_indexer_k(g.pool, g.block_table, g.cu, total)
    flat = torch.full((total * stride + pad,), 4321.0, dtype=torch.float32, device=DEV)
    rl = torch.full((total,), -7, dtype=torch.int32, device=DEV)
    rr = torch.full((total,), -7, dtype=torch.int32, device=DEV)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = sai.load().mqa_logits(_p(g.q_fp8), _p(g.w_eff), _p(kv), _p(ks), _p(g.cu), 3, total, _p(flat, pad),
                               stride, _p(rl), _p(rr), stream)
    assert rc == 0
    torch.cuda.synchronize()
    got = flat.cpu().numpy()
    assert np.all(got[:pad] == 4321.0)
    rv, rs = O.gather_indexer_k(o.pool, wl.block_table, wl.cu_seq_lens, total)
    ref = O.mqa_logits(o.q_codes, o.w_eff, rv, rs, wl.cu_seq_lens, stride)
    assert_logits_close(got[pad:].reshape(total, stride), ref, "prefill, 4-byte store path")
    assert rl.cpu().tolist() == list(range(1, 302)) + [1, 2] + list(range(1, 68))
    assert rr.cpu().tolist() == [0] * 301 + [1] * 2 + [2] * 67


def test_chunked_prefill_rows_that_see_no_key_and_partial_tiles():
    """Chunks longer than their contexts (rows at the front see nothing and
    are all -inf), chunks whose last tile holds 1-3 rows, at an odd width
    (4-byte stores)."""
    ctx, n_q = [5, 130, 1, 66], [9, 131, 3, 66]
    width = 131
    _say(f"mqa_logits_chunked: contexts {ctx}, chunks {n_q}, width {width}")
    wl = synth.custom(len(ctx), 0, ctx, num_blocks=sum(-(-c // 64) for c in ctx) + 3,
                      bt_width=max(-(-c // 64) for c in ctx) + 1, seed=83)
    g = GpuWorkload(wl)
    o = OracleWorkload(wl)
    cu_k = np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32)
    cu_q = np.concatenate([[0], np.cumsum(n_q)]).astype(np.int32)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    rng = np.random.default_rng(84)
    qbits = synth.f32_to_bf16_bits(rng.standard_normal((tq, 64, 128)).astype(np.float32))
    w = (rng.standard_normal((tq, 64)) / 64).astype(np.float32)
    qf, weff, _ = sai.indexer_q_quant(bf16_tensor(qbits), torch.from_numpy(w).to(DEV))
    ck, cq = torch.from_numpy(cu_k).to(DEV), torch.from_numpy(cu_q).to(DEV)
    kv, ks = sai.gather_indexer_k(g.pool, g.block_table, ck, tk)
    logits = torch.full((tq, width), 99.0, dtype=torch.float32, device=DEV)
    logits, row_len, row_req = sai.mqa_logits_chunked(qf, weff, kv, ks, cq, ck, width, logits=logits)
    torch.cuda.synchronize()
    rv, rs = O.gather_indexer_k(o.pool, wl.block_table, cu_k, tk)
    qc, ow, _ = O.quantize_q(synth.bf16_bits_to_f32(qbits), w)
    ref = O.mqa_logits_chunked(qc, ow, rv, rs, cu_q, cu_k, width)
    got = logits.cpu().numpy()
    assert_logits_close(got, ref, "chunked prefill, rows that see nothing")
    want_len = [max(c - n + i + 1, 0) for c, n in zip(ctx, n_q) for i in range(n)]
    assert row_len.cpu().tolist() == want_len
    blind = np.array(want_len) == 0
    assert blind.sum() == 4 + 1 + 2 and np.all(np.isneginf(got[blind]))
