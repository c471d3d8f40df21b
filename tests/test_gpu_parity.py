"""GPU parity of every entry point against the CPU oracle on small seeded
inputs that still span several 64-key blocks, ragged tails, poisoned stale
bytes and every next_n; integer and byte outputs bit-exact, logits within
1e-4 + 1e-3*|ref|."""
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


# ---------------------------------------------------------------- producers
def test_k_cache_write_bit_exact_tiny_decode():
    _say("k_cache_write: tiny decode workload")
    wl = synth.make(0)
    g = GpuWorkload(wl)
    o = OracleWorkload(wl)
    assert np.array_equal(g.pool.cpu().numpy(), o.pool)


def test_k_cache_write_edge_values():
    _say("k_cache_write: edge values")
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    x[0] = 0.0                                  # all zero -> FLT_MIN scale
    x[1] = -0.0
    x[2, :] = 3.0                               # constant row
    x[3] *= 1e30                                # huge
    x[4] *= 1e-30                               # tiny (normal)
    x[5, ::2] = 0.0
    x[6] = np.where(np.arange(128) % 2, 1e-3, -448.0)
    x[7, 0] = 2.0 ** -133                       # bf16 subnormal next to zeros
    x[7, 1:] = 0.0
    x[8] = rng.standard_normal(128) * 1e-38     # subnormal-heavy row
    bits = synth.f32_to_bf16_bits(x)
    xf = synth.bf16_bits_to_f32(bits)
    slots = np.arange(64, dtype=np.int64) * 3 % 190 - 1       # includes -1 (skipped)
    pool_np = np.full((3, synth.BLOCK_BYTES), 0x5A, np.uint8)
    ref = O.k_cache_write(xf, slots, pool_np.copy())
    pool = torch.from_numpy(pool_np).to(DEV)
    sai.indexer_k_cache_write(bf16_tensor(bits), torch.from_numpy(slots).to(DEV), pool)
    got = pool.cpu().numpy()
    if not np.array_equal(got, ref):
        diff = np.argwhere(got != ref)
        raise AssertionError(f"{len(diff)} bytes differ, first at {diff[:5].tolist()}")


def test_q_quant_bit_exact():
    _say("q_quant: tiny decode queries + edge rows")
    wl = synth.make(0)
    q = synth.bf16_bits_to_f32(wl.q())
    w = wl.w()
    q = np.concatenate([q, np.zeros((1, 64, 128), np.float32), q[:1] * 1e-20])
    w = np.concatenate([w, w[:1], w[:1]])
    bits = synth.f32_to_bf16_bits(q)
    qf = synth.bf16_bits_to_f32(bits)
    codes, weff, qs = O.quantize_q(qf, w)
    gc, gw, gs = sai.indexer_q_quant(bf16_tensor(bits), torch.from_numpy(w).to(DEV))
    assert np.array_equal(gc.cpu().numpy(), codes)
    assert np.array_equal(gs.cpu().numpy().view(np.uint32), qs.view(np.uint32))
    assert np.array_equal(gw.cpu().numpy().view(np.uint32), weff.view(np.uint32))


# ---------------------------------------------------------------- logits
def _check_decode(wl, requests=None, rows=None):
    g = GpuWorkload(wl)
    o = OracleWorkload(wl, requests=requests)
    nn = wl.next_n
    logits, row_len, row_req = sai.paged_mqa_logits(
        g.q_fp8.view(wl.batch, nn, 64, 128), g.w_eff, g.pool, g.block_table, g.ctx)
    torch.cuda.synchronize()
    lim, req = O.decode_limits(wl.ctx, nn)
    assert np.array_equal(row_len.cpu().numpy(), lim.clip(min=0))
    assert np.array_equal(row_req.cpu().numpy(), req)
    ref = O.paged_mqa_logits(o.q_codes.reshape(wl.batch, nn, 64, 128), o.w_eff, o.pool,
                             wl.block_table, wl.ctx, nn, wl.width, rows=rows)
    gl = logits.cpu().numpy()
    sel = slice(None) if rows is None else np.asarray(rows)
    worst = assert_logits_close(gl[sel], ref[sel], wl.name)
    _say(f"{wl.name}: worst err/tol {worst:.3g}")
    return g, logits, row_len, row_req


def test_paged_logits_tiny_decode():
    _say("paged_mqa_logits: tiny decode (batch 2, ctx 3000/5000)")
    _check_decode(synth.make(0))


@pytest.mark.parametrize("next_n", [1, 2, 3, 4])
def test_paged_logits_ragged_next_n(next_n):
    _say(f"paged_mqa_logits: ragged contexts, next_n={next_n}")
    ctx = [next_n, 63, 64, 65, 127, 129, 700, 1, 64 * 5 + 17][: 9 if next_n == 1 else 8]
    ctx = [max(c, next_n) for c in ctx]
    wl = synth.custom(len(ctx), next_n, ctx, num_blocks=64, bt_width=12, seed=100 + next_n)
    _check_decode(wl)


def test_paged_logits_width_not_multiple_of_64_and_empty_request():
    _say("paged_mqa_logits: stride 1000, an empty request")
    wl = synth.custom(3, 1, [900, 0, 257], num_blocks=40, bt_width=16, seed=7)
    g = GpuWorkload(wl)
    o = OracleWorkload(wl)
    logits = torch.full((3, 1000), 7.0, device=DEV)
    logits, row_len, _ = sai.paged_mqa_logits(g.q_fp8.view(3, 1, 64, 128), g.w_eff, g.pool,
                                              g.block_table, g.ctx, width=1000, logits=logits)
    ref = O.paged_mqa_logits(o.q_codes.reshape(3, 1, 64, 128), o.w_eff, o.pool, wl.block_table,
                             wl.ctx, 1, 1000)
    assert_logits_close(logits.cpu().numpy(), ref, "stride1000")
    assert row_len.cpu().tolist() == [900, 0, 257]


@pytest.mark.parametrize("width,offset", [(1001, 0), (1000, 1)])
def test_paged_logits_unaligned_rows(width, offset):
    """Rows that are not 16-byte aligned (an odd row pitch, or a base pointer
    4 bytes off) are written one float per lane instead of four."""
    _say(f"paged_mqa_logits: row pitch {width}, base offset {offset} floats")
    wl = synth.custom(3, 2, [700, 997, 2], num_blocks=40, bt_width=16, seed=11)
    g = GpuWorkload(wl)
    o = OracleWorkload(wl)
    buf = torch.full((6 * width + offset,), 7.0, device=DEV)
    logits = buf[offset:].view(6, width)
    sai.paged_mqa_logits(g.q_fp8.view(3, 2, 64, 128), g.w_eff, g.pool, g.block_table, g.ctx,
                         width=width, logits=logits)
    ref = O.paged_mqa_logits(o.q_codes.reshape(3, 2, 64, 128), o.w_eff, o.pool, wl.block_table,
                             wl.ctx, 2, width)
    assert_logits_close(logits.cpu().numpy(), ref, f"pitch{width}+{offset}")
    if offset:
        assert buf[0].item() == 7.0


def test_paged_logits_more_units_per_wave_than_stage():
    """next_n 4 over 16 long requests: each persistent wave scores about 12
    key blocks but stages at most 8 in LDS, so every wave writes out its
    results part-way through its share."""
    ctx = [98304 - 37 * i for i in range(16)]
    _say("paged_mqa_logits: 16 x ~98K keys, next_n=4")
    wl = synth.custom(16, 4, ctx, num_blocks=16 * 1536 + 8, bt_width=1536, seed=12)
    rows = [0, 3, 17, 30, 45, 62, 63]
    _check_decode(wl, requests=sorted({r // 4 for r in rows}), rows=rows)


def test_paged_logits_largest_batch():
    """4096 requests (the most the decode launch takes): the per-request
    prefix sums push the workgroup's LDS above 64 KB."""
    _say("paged_mqa_logits: batch 4096")
    rng = np.random.default_rng(13)
    ctx = rng.integers(1, 200, size=4096).tolist()
    wl = synth.custom(4096, 1, ctx, num_blocks=4096 * 4 + 8, bt_width=4, seed=13)
    props = torch.cuda.get_device_properties(0)
    lds = 4 * 2048 * 4 + (3 * 4097 + 8) * 4
    if getattr(props, "shared_memory_per_block", 1 << 30) < lds:
        with pytest.raises(RuntimeError, match="unsupported"):
            _check_decode(wl, requests=[0], rows=[0])
        return
    rows = [0, 1, 777, 2048, 4095]
    _check_decode(wl, requests=rows, rows=rows)


def test_paged_logits_deterministic_and_permutation_invariant():
    _say("paged_mqa_logits: determinism + block permutation")
    wl = synth.custom(4, 2, [1000, 333, 64, 2000], num_blocks=80, bt_width=40, seed=9)
    g = GpuWorkload(wl)
    args = (g.q_fp8.view(4, 2, 64, 128), g.w_eff)
    l1, _, _ = sai.paged_mqa_logits(*args, g.pool, g.block_table, g.ctx)
    l2, _, _ = sai.paged_mqa_logits(*args, g.pool, g.block_table, g.ctx)
    pi = torch.from_numpy(np.random.default_rng(1).permutation(80)).to(DEV)
    pool2 = torch.empty_like(g.pool)
    pool2[pi] = g.pool
    bt2 = torch.where(g.block_table >= 0, pi[g.block_table.clamp(min=0).long()].int(), g.block_table)
    l3, _, _ = sai.paged_mqa_logits(*args, pool2, bt2.contiguous(), g.ctx)
    assert torch.equal(l1, l2)
    assert torch.equal(l1, l3)


# ---------------------------------------------------------------- top-k / slots
def test_decode_topk_and_slots_bit_exact_tiny():
    _say("topk_rows + topk_to_global_slots: tiny decode")
    wl = synth.make(0)
    g, logits, row_len, row_req = _check_decode(wl)
    idx = sai.topk_rows(logits, row_len, 2048)
    slots = sai.topk_to_global_slots(idx, row_req, g.block_table)
    gl = logits.cpu().numpy()
    want = O.topk_rows(gl, row_len.cpu().numpy(), 2048)
    assert np.array_equal(idx.cpu().numpy(), want)
    want_s = O.topk_to_global_slots(want, row_req.cpu().numpy(), wl.block_table)
    assert np.array_equal(slots.cpu().numpy(), want_s)


def _adversarial_rows(W=9000):
    rng = np.random.default_rng(3)
    rows = []
    rows.append(rng.standard_normal(W))
    rows.append(np.zeros(W))                                   # all equal
    r = np.zeros(W); r[::2] = -0.0; rows.append(r)             # +-0 ties
    rows.append(np.arange(W, dtype=np.float64))                # increasing
    rows.append(-np.arange(W, dtype=np.float64))               # decreasing
    rows.append(np.round(rng.standard_normal(W) * 2))          # heavy ties
    r = rng.standard_normal(W); r[rng.random(W) < 0.3] = -np.inf; rows.append(r)
    rows.append(np.full(W, -np.inf))                           # all -inf
    r = rng.standard_normal(W) * 1e-38; rows.append(r)         # subnormals
    r = np.full(W, 1.0); r[5000:] = 2.0; rows.append(r)        # threshold inside a tie block
    L = np.stack(rows).astype(np.float32)
    lens = np.array([W, W, W, W, W, W, W, W, W, W, 2048, 2047, 1, 0, 5000, W - 1], np.int32)
    L = np.concatenate([L, L[:6]])
    return L, lens


@pytest.mark.parametrize("k", [2048, 1, 37, 1000])
def test_topk_adversarial_rows(k):
    _say(f"topk_rows: adversarial rows, k={k}")
    L, lens = _adversarial_rows()
    got = sai.topk_rows(torch.from_numpy(L).to(DEV), torch.from_numpy(lens).to(DEV), k)
    want = O.topk_rows(L, lens, k)
    assert np.array_equal(got.cpu().numpy(), want)


@pytest.mark.parametrize("k,width", [(2048, 40000), (37, 40000), (2048, 100000), (37, 100000)])
def test_topk_adversarial_wide_rows(k, width):
    """The same rows 40000 wide (one pass) and 100000 wide (seven segments
    whose winners are merged): ties and the exact fallbacks of every pass."""
    _say(f"topk_rows: adversarial rows {width} wide, k={k}")
    L, lens = _adversarial_rows(width)
    got = sai.topk_rows(torch.from_numpy(L).to(DEV), torch.from_numpy(lens).to(DEV), k)
    want = O.topk_rows(L, lens, k)
    assert np.array_equal(got.cpu().numpy(), want)


def _nan_rows(W):
    """Rows with NaNs of both signs and several payloads among numbers."""
    rng = np.random.default_rng(W + 1)
    nan_bits = np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFFFFFFFF, 0x7FFFFFFF], np.uint32)
    rows = []
    r = rng.standard_normal(W).astype(np.float32)
    m = rng.random(W) < 0.1
    r[m] = nan_bits[rng.integers(0, 5, m.sum())].view(np.float32)
    rows.append(r)                                             # 10 % NaN among numbers
    rows.append(np.full(W, np.nan, np.float32))                # all NaN
    r = np.full(W, np.nan, np.float32)
    r[rng.choice(W, 1500, replace=False)] = rng.standard_normal(1500)
    rows.append(r)                                             # fewer numbers than k: NaNs fill up
    r = np.full(W, -np.inf, np.float32)
    r[::3] = nan_bits[1].view(np.float32)
    r[1::97] = 0.5
    rows.append(r)                                             # NaN, -inf and a few numbers
    L = np.stack(rows)
    lens = np.array([W, W, W, W], np.int32)
    return L, lens


@pytest.mark.parametrize("width", [9000, 40000, 100000, 140000])
def test_topk_nan_ranks_last(width):
    """NaN ranks below -inf and NaNs tie by index on every selection path
    (one pass, segments + merge, streaming), as the oracle ranks them."""
    _say(f"topk_rows: NaN rows, width {width}")
    L, lens = _nan_rows(width)
    for k in (2048, 37):
        got = sai.topk_rows(torch.from_numpy(L).to(DEV), torch.from_numpy(lens).to(DEV), k)
        assert np.array_equal(got.cpu().numpy(), O.topk_rows(L, lens, k)), k


def test_decode_block_outside_pool_gives_nan_logits_ranked_last():
    """A block-table entry past the pool makes that block's visible columns
    NaN; the decode top-k ranks them last and the slot ids follow the table."""
    _say("decode pipeline: a block id outside the pool")
    wl = synth.custom(2, 1, [3000, 2500], num_blocks=100, bt_width=50, seed=31)
    g = GpuWorkload(wl)
    bt = wl.block_table.copy()
    bt[0, 7] = wl.num_blocks + 5
    bt[1, 10] = -3
    q = g.q_fp8.view(wl.batch, 1, 64, 128)
    logits, idx, slots = sai.decode_indexer(q, g.w_eff, g.pool, torch.from_numpy(bt).to(DEV), g.ctx)
    torch.cuda.synchronize()
    gl = logits.cpu().numpy()
    assert np.isnan(gl[0, 7 * 64:8 * 64]).all() and np.isnan(gl[1, 640:704]).all()
    o = OracleWorkload(wl)
    ref = O.paged_mqa_logits(o.q_codes.reshape(2, 1, 64, 128), o.w_eff, o.pool, wl.block_table,
                             wl.ctx, 1, wl.width)
    ok = np.ones(gl.shape, bool)
    ok[0, 7 * 64:8 * 64] = False
    ok[1, 640:704] = False
    assert_logits_close(np.where(ok, gl, 0.0), np.where(ok, ref, 0.0), "outside-pool decode")
    lim, req = O.decode_limits(wl.ctx, 1)
    want = O.topk_rows(gl, lim, 2048)
    assert np.array_equal(idx.cpu().numpy(), want)
    assert not np.isin(np.arange(448, 512), want[0]).any()
    assert not np.isin(np.arange(640, 704), want[1]).any()
    assert np.array_equal(slots.cpu().numpy(), O.topk_to_global_slots(want, req, bt))


@pytest.mark.parametrize("width,k", [(140000, 2048), (300000, 100)])
def test_topk_widest_rows(width, k):
    """Rows past the two-pass limit (streaming kernel) and a small k whose
    candidate lists still fit the merge."""
    _say(f"topk_rows: width {width}, k={k}")
    rng = np.random.default_rng(width + k)
    L = rng.standard_normal((4, width)).astype(np.float32)
    L[1, ::3] = 0.5
    lens = np.array([width, width - 7, k + 1, width // 2], np.int32)
    got = sai.topk_rows(torch.from_numpy(L).to(DEV), torch.from_numpy(lens).to(DEV), k)
    assert np.array_equal(got.cpu().numpy(), O.topk_rows(L, lens, k))


@pytest.mark.parametrize("rows,width", [(520, 1000), (600, 9000), (600, 40000)])
def test_topk_many_rows_small_workgroups(rows, width):
    """At least 512 workgroups switch to 256/512-thread shapes (one pass,
    segment pass and merge), with ties, short rows and tied thresholds."""
    _say(f"topk_rows_slots: {rows} rows x {width}")
    rng = np.random.default_rng(rows + width)
    L = rng.standard_normal((rows, width)).astype(np.float32)
    L[::7, ::3] = 0.25
    L[5] = 1.0
    lens = rng.integers(0, width + 1, size=rows).astype(np.int32)
    lens[:4] = [width, 2048, 2049, 0]
    nblk = -(-width // 64)
    bt = rng.permutation(2 * nblk)[:nblk].reshape(1, nblk).astype(np.int32)
    req = np.zeros(rows, np.int32)
    T = lambda a: torch.from_numpy(a).to(DEV)  # noqa: E731
    idx, slots = sai.topk_rows_slots(T(L), T(lens), T(req), T(bt), 2048)
    want = O.topk_rows(L, lens, 2048)
    assert np.array_equal(idx.cpu().numpy(), want)
    assert np.array_equal(slots.cpu().numpy(), O.topk_to_global_slots(want, req, bt))


@pytest.mark.parametrize("width", [4099, 40001])
def test_topk_unaligned_stride(width):
    _say(f"topk_rows: odd stride {width}")
    rng = np.random.default_rng(4)
    L = rng.standard_normal((5, width)).astype(np.float32)
    L[3] = np.round(L[3] * 2)                              # heavy ties: the exact fallbacks
    lens = np.array([width, 3000, 2049, width - 1, 100], np.int32)
    full = torch.from_numpy(L).to(DEV)
    got = sai.topk_rows(full, torch.from_numpy(lens).to(DEV), 2048)
    assert np.array_equal(got.cpu().numpy(), O.topk_rows(L, lens, 2048))


def test_slots_edge_cases():
    _say("topk_to_global_slots: -1, out-of-table, bad request")
    bt = np.array([[5, 9, -1], [2, 0, 7]], np.int32)
    idx = np.array([[0, 63, 64, 127, -1, 128, 191, 192],
                    [0, 1, 64, 130, 191, -1, -1, -1],
                    [0, 1, 2, 3, 4, 5, 6, 7]], np.int32)
    req = np.array([0, 1, 5], np.int32)
    got = sai.topk_to_global_slots(torch.from_numpy(idx).to(DEV), torch.from_numpy(req).to(DEV),
                                   torch.from_numpy(bt).to(DEV)).cpu().numpy()
    assert np.array_equal(got, O.topk_to_global_slots(idx, req, bt))
    assert got[0].tolist() == [320, 383, 576, 639, -1, -1, -1, -1]
    assert got[1].tolist() == [128, 129, 0, 450, 511, -1, -1, -1]
    assert got[2].tolist() == [-1] * 8


@pytest.mark.parametrize("width", [1000, 16384, 40000, 140000])
def test_topk_rows_slots_matches_the_two_calls(width):
    """The fused call on every selection path (one pass, one-segment rows,
    segments + merge, streaming): indices and slot ids against the oracle's
    top-k and slot map; then, with a request outside the batch and negative
    table entries, slot ids against the standalone topk_to_global_slots."""
    _say(f"topk_rows_slots: width {width}")
    rng = np.random.default_rng(width)
    rows, k = 7, 2048
    L = rng.standard_normal((rows, width)).astype(np.float32)
    L[3, ::5] = 1.5                                          # ties at the threshold
    L[1] = np.round(L[1] * 2)                                # heavy ties: the exact fallbacks
    lens = np.array([width, width - 1, 2048, min(width, 3000), 5, 0, width // 2], np.int32)
    nblk = -(-width // 64)
    bt = rng.permutation(4 * nblk)[: 3 * nblk].reshape(3, nblk).astype(np.int32)
    req = np.array([0, 1, 2, 1, 0, 2, 1], np.int32)
    T = lambda a: torch.from_numpy(a).to(DEV)  # noqa: E731
    idx, slots = sai.topk_rows_slots(T(L), T(lens), T(req), T(bt), k)
    want = O.topk_rows(L, lens, k)
    assert np.array_equal(idx.cpu().numpy(), want)
    assert np.array_equal(slots.cpu().numpy(), O.topk_to_global_slots(want, req, bt))
    # entries the library maps to -1: an unused table tail and a bad request
    bt[1, nblk // 2:] = -1
    req[6] = 7
    idx, slots = sai.topk_rows_slots(T(L), T(lens), T(req), T(bt), k)
    sep = sai.topk_to_global_slots(idx, T(req), T(bt))
    assert np.array_equal(idx.cpu().numpy(), want)
    assert np.array_equal(slots.cpu().numpy(), O.topk_to_global_slots(want, req, bt))
    assert torch.equal(slots, sep)
    assert (slots[6] == -1).all()


# ---------------------------------------------------------------- prefill
def test_gather_bit_exact():
    _say("gather_indexer_k: ragged requests incl. empty")
    wl = synth.custom(4, 0, [130, 0, 64, 301], num_blocks=24, bt_width=5, seed=21)
    g = GpuWorkload(wl)
    o = OracleWorkload(wl)
    total = wl.total_tokens
    kv, ks = sai.gather_indexer_k(g.pool, g.block_table, g.cu, total)
    rv, rs = O.gather_indexer_k(o.pool, wl.block_table, wl.cu_seq_lens, total)
    assert np.array_equal(kv.cpu().numpy(), rv)
    assert np.array_equal(ks.cpu().numpy().view(np.uint32), rs.view(np.uint32))


def test_prefill_logits_two_requests():
    _say("gather + mqa_logits: two requests 300 + 77 tokens")
    wl = synth.custom(2, 0, [300, 77], num_blocks=12, bt_width=5, seed=22)
    g = GpuWorkload(wl)
    o = OracleWorkload(wl)
    total = wl.total_tokens
    kv, ks = sai.gather_indexer_k(g.pool, g.block_table, g.cu, total)
    width = 320
    logits, row_len, row_req = sai.mqa_logits(g.q_fp8, g.w_eff, kv, ks, g.cu, width)
    rv, rs = O.gather_indexer_k(o.pool, wl.block_table, wl.cu_seq_lens, total)
    ref = O.mqa_logits(o.q_codes, o.w_eff, rv, rs, wl.cu_seq_lens, width)
    assert_logits_close(logits.cpu().numpy(), ref, "prefill")
    assert row_len.cpu().tolist() == list(range(1, 301)) + list(range(1, 78))
    assert row_req.cpu().tolist() == [0] * 300 + [1] * 77
    idx = sai.topk_rows(logits, row_len, 64)
    assert np.array_equal(idx.cpu().numpy(), O.topk_rows(logits.cpu().numpy(), row_len.cpu().numpy(), 64))


def test_prefill_matches_decode_next_n():
    """Same score on both paths: B=1, next_n=N=ctx on the paged cache equals
    prefill over the gathered K (bitwise: identical kernels' arithmetic order)."""
    _say("mqa_logits vs paged_mqa_logits (next_n=4, ctx=4)")
    wl = synth.custom(1, 4, [4], num_blocks=3, bt_width=1, seed=23)
    g = GpuWorkload(wl)
    ld, _, _ = sai.paged_mqa_logits(g.q_fp8.view(1, 4, 64, 128), g.w_eff, g.pool, g.block_table, g.ctx)
    cu = torch.tensor([0, 4], dtype=torch.int32, device=DEV)
    kv, ks = sai.gather_indexer_k(g.pool, g.block_table, cu, 4)
    lp, _, _ = sai.mqa_logits(g.q_fp8, g.w_eff, kv, ks, cu, 64)
    assert torch.equal(ld, lp)


def _chunked_case(ctx, n_q, width, seed, sentinel=None):
    """Gather each request's whole context, score a chunk of its last n_q
    tokens on the GPU and with the oracle."""
    wl = synth.custom(len(ctx), 0, ctx, num_blocks=sum(-(-c // 64) for c in ctx) + 3,
                      bt_width=max(-(-c // 64) for c in ctx) + 1, seed=seed)
    g = GpuWorkload(wl)
    o = OracleWorkload(wl)
    cu_k = np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32)
    cu_q = np.concatenate([[0], np.cumsum(n_q)]).astype(np.int32)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    rng = np.random.default_rng(seed + 1)
    qbits = synth.f32_to_bf16_bits(rng.standard_normal((tq, 64, 128)).astype(np.float32))
    w = (rng.standard_normal((tq, 64)) / 64).astype(np.float32)
    qf, weff, _ = sai.indexer_q_quant(bf16_tensor(qbits), torch.from_numpy(w).to(DEV))
    ck, cq = torch.from_numpy(cu_k).to(DEV), torch.from_numpy(cu_q).to(DEV)
    kv, ks = sai.gather_indexer_k(g.pool, g.block_table, ck, tk)
    logits = torch.full((tq, width), sentinel if sentinel is not None else 0.0, dtype=torch.float32, device=DEV)
    logits, row_len, row_req = sai.mqa_logits_chunked(qf, weff, kv, ks, cq, ck, width, logits=logits)
    rv, rs = O.gather_indexer_k(o.pool, wl.block_table, cu_k, tk)
    qc, ow, _ = O.quantize_q(synth.bf16_bits_to_f32(qbits), w)
    ref = O.mqa_logits_chunked(qc, ow, rv, rs, cu_q, cu_k, width)
    return wl, g, logits, row_len, row_req, ref, cu_q, cu_k


def test_chunked_prefill_ragged_batch():
    """Chunks of 200 (of 700), 130 (the whole request), 1 (of 64) and 5 (of a
    3-token context: two rows see nothing), scored against the gathered
    contexts; top-k and slot ids on the result."""
    ctx, n_q = [700, 130, 64, 3], [200, 130, 1, 5]
    _say(f"mqa_logits_chunked: contexts {ctx}, chunks {n_q}")
    wl, g, logits, row_len, row_req, ref, cu_q, cu_k = _chunked_case(ctx, n_q, 768, 41)
    got = logits.cpu().numpy()
    assert_logits_close(got, ref, "chunked prefill")
    want_len = [max(c - n + i + 1, 0) for c, n in zip(ctx, n_q) for i in range(n)]
    assert row_len.cpu().tolist() == want_len
    assert row_req.cpu().tolist() == [b for b, n in enumerate(n_q) for _ in range(n)]
    idx = sai.topk_rows(logits, row_len, 64)
    assert np.array_equal(idx.cpu().numpy(), O.topk_rows(got, row_len.cpu().numpy(), 64))
    slots = sai.topk_to_global_slots(idx, row_req, g.block_table)
    ref_slots = O.topk_to_global_slots(idx.cpu().numpy(), row_req.cpu().numpy(), wl.block_table)
    assert np.array_equal(slots.cpu().numpy(), ref_slots)


def test_chunked_prefill_width_clamp_leaves_rows_untouched():
    """Rows whose limit exceeds the width are not written (sentinel kept)."""
    ctx, n_q = [300, 90], [100, 90]
    _say(f"mqa_logits_chunked: width 256 under contexts {ctx}")
    _, _, logits, _, _, ref, _, _ = _chunked_case(ctx, n_q, 256, 43, sentinel=12345.0)
    got = logits.cpu().numpy()
    untouched = np.isnan(ref).all(axis=1)
    assert untouched.sum() == 44                     # request 0 rows with limit 257..300
    assert np.all(got[untouched] == 12345.0)
    assert_logits_close(got[~untouched], ref[~untouched], "chunked prefill, clamped width")


def test_chunked_prefill_matches_paged_decode_next_n():
    """Bitwise: chunks of 4 at the end of each context == paged decode with
    next_n = 4 on the same cache (the same arithmetic order in both kernels)."""
    ctx = [260, 65, 4]
    _say(f"mqa_logits_chunked vs paged_mqa_logits, next_n 4, contexts {ctx}")
    wl = synth.custom(3, 4, ctx, num_blocks=12, bt_width=5, seed=44)
    g = GpuWorkload(wl)
    ld, _, _ = sai.paged_mqa_logits(g.q_fp8.view(3, 4, 64, 128), g.w_eff, g.pool, g.block_table, g.ctx,
                                    width=320)
    cu_k = torch.tensor(np.concatenate([[0], np.cumsum(ctx)]), dtype=torch.int32, device=DEV)
    cu_q = torch.tensor([0, 4, 8, 12], dtype=torch.int32, device=DEV)
    kv, ks = sai.gather_indexer_k(g.pool, g.block_table, cu_k, sum(ctx))
    lc, _, _ = sai.mqa_logits_chunked(g.q_fp8, g.w_eff, kv, ks, cu_q, cu_k, 320)
    assert torch.equal(ld, lc)


@pytest.mark.parametrize("next_n", [1, 2])
def test_visible_logits_write_only_the_key_blocks(next_n):
    """paged_mqa_logits_visible: the request's key blocks exactly as the
    clean call writes them, everything after them untouched (sentinel), and
    the same top-k and slot ids downstream."""
    ctx = [1, 64, 65, 300, 2049]
    _say(f"paged_mqa_logits_visible: contexts {ctx}, next_n={next_n}")
    wl = synth.custom(len(ctx), next_n, ctx, num_blocks=60, bt_width=40, seed=51 + next_n)
    g = GpuWorkload(wl)
    q = g.q_fp8.view(len(ctx), next_n, 64, 128)
    lc, rl, rr = sai.paged_mqa_logits(q, g.w_eff, g.pool, g.block_table, g.ctx)
    sentinel = torch.full_like(lc, 777.0)
    lv, rlv, rrv = sai.paged_mqa_logits(q, g.w_eff, g.pool, g.block_table, g.ctx, logits=sentinel, clean=False)
    torch.cuda.synchronize()
    c, v = lc.cpu().numpy(), lv.cpu().numpy()
    for b, cb in enumerate(ctx):
        end = -(-cb // 64) * 64
        rows = slice(next_n * b, next_n * (b + 1))
        assert np.array_equal(v[rows, :end].view(np.uint32), c[rows, :end].view(np.uint32))
        assert np.all(v[rows, end:] == 777.0)
    assert torch.equal(rl, rlv) and torch.equal(rr, rrv)
    ic = sai.topk_rows(lc, rl, 2048)
    iv = sai.topk_rows(lv, rlv, 2048)
    assert torch.equal(ic, iv)


# ---------------------------------------------------------------- graph capture
def test_decode_pipeline_graph_capture_replays_match_eager():
    _say("hipGraph capture of the decode pipeline")
    wl = synth.custom(6, 2, [3000, 100, 2049, 5000, 64, 4000], num_blocks=300, bt_width=80, seed=31)
    g = GpuWorkload(wl)
    q = g.q_fp8.view(6, 2, 64, 128)
    eager = sai.decode_indexer(q, g.w_eff, g.pool, g.block_table, g.ctx)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sai.decode_indexer(q, g.w_eff, g.pool, g.block_table, g.ctx)   # warm-up on side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = sai.decode_indexer(q, g.w_eff, g.pool, g.block_table, g.ctx)
    for rep in range(3):
        for t in out:
            t.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(out, eager):
            assert torch.equal(a, b), f"replay {rep} differs"
        eager2 = sai.decode_indexer(q, g.w_eff, g.pool, g.block_table, g.ctx)
        torch.cuda.synchronize()
        for a, b in zip(eager2, eager):
            assert torch.equal(a, b)


@pytest.mark.parametrize("ctx,num_blocks,bt_width", [([40000, 20000, 3000, 17000], 1500, 640),
                                                     ([70000, 30000, 3000, 66000], 3000, 1100)])
def test_wide_row_pipeline_graph_capture_replays_match_eager(ctx, num_blocks, bt_width):
    """Rows wider than one top-k segment captured in a hipGraph: 40960
    columns (one pass of the wide-row kernel) and 70400 columns (segment
    pass, candidate lists in the workspace, merge pass).  Every replay
    equals the eager result, with eager work between replays."""
    _say(f"hipGraph capture of the decode pipeline, {bt_width * 64}-column rows")
    wl = synth.custom(4, 2, ctx, num_blocks=num_blocks, bt_width=bt_width, seed=47)
    g = GpuWorkload(wl)
    q = g.q_fp8.view(4, 2, 64, 128)
    eager = sai.decode_indexer(q, g.w_eff, g.pool, g.block_table, g.ctx)
    torch.cuda.synchronize()
    logits, idx, _ = eager
    rl = torch.from_numpy(np.repeat(wl.ctx, 2) - 2 + np.tile(np.arange(2), 4) + 1).to(torch.int32)
    assert np.array_equal(idx.cpu().numpy(), O.topk_rows(logits.cpu().numpy(), rl.numpy(), 2048))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sai.decode_indexer(q, g.w_eff, g.pool, g.block_table, g.ctx)   # warm-up on side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = sai.decode_indexer(q, g.w_eff, g.pool, g.block_table, g.ctx)
    for rep in range(3):
        for t in out:
            t.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(out, eager):
            assert torch.equal(a, b), f"replay {rep} differs"
        eager2 = sai.decode_indexer(q, g.w_eff, g.pool, g.block_table, g.ctx)
        torch.cuda.synchronize()
        for a, b in zip(eager2, eager):
            assert torch.equal(a, b)


def test_prefill_pipeline_graph_capture_replays_match_eager():
    """gather -> mqa_logits -> top-k with slot ids (3072 rows, so the top-k
    takes its many-row shapes) captured in a hipGraph: every replay equals
    the eager result, with eager work between replays."""
    _say("hipGraph capture of the prefill pipeline, 2000 + 1072 tokens")
    wl = synth.custom(2, 0, [2000, 1072], num_blocks=60, bt_width=32, seed=53)
    g = GpuWorkload(wl)
    total, width = wl.total_tokens, 2048

    def run():
        kv, ks = sai.gather_indexer_k(g.pool, g.block_table, g.cu, total)
        logits, row_len, row_req = sai.mqa_logits(g.q_fp8, g.w_eff, kv, ks, g.cu, width)
        idx, slots = sai.topk_rows_slots(logits, row_len, row_req, g.block_table, 2048)
        return kv, ks, logits, idx, slots

    eager = run()
    torch.cuda.synchronize()
    assert np.array_equal(eager[3].cpu().numpy(),
                          O.topk_rows(eager[2].cpu().numpy(), np.r_[1:2001, 1:1073].astype(np.int32), 2048))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()   # warm-up on side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = run()
    for rep in range(3):
        for t in out:
            t.fill_(0xA5 if t.dtype == torch.uint8 else -7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(out, eager):
            assert torch.equal(a, b), f"replay {rep} differs"
        eager2 = run()
        torch.cuda.synchronize()
        for a, b in zip(eager2, eager):
            assert torch.equal(a, b)


def test_producers_graph_capture_replays_match_eager():
    """The q quantiser, the indexer K-cache writer and the MLA cache writer
    captured in one hipGraph: every replay writes the bytes the eager calls
    wrote (skipped slots included), with eager work between replays."""
    _say("hipGraph capture of the producers: q quant, K-cache write, MLA cache write")
    rng = np.random.default_rng(59)
    n = 300
    q = bf16_tensor(synth.f32_to_bf16_bits(rng.standard_normal((n, 64, 128)).astype(np.float32)))
    wt = torch.from_numpy((rng.standard_normal((n, 64)) / 64).astype(np.float32)).to(DEV)
    k = bf16_tensor(synth.f32_to_bf16_bits(rng.standard_normal((n, 128)).astype(np.float32)))
    kv = bf16_tensor(synth.f32_to_bf16_bits(rng.standard_normal((n, 576)).astype(np.float32)))
    slot_np = rng.permutation(20 * 64)[:n].astype(np.int64)
    slot_np[::37] = -1
    slot = torch.from_numpy(slot_np).to(DEV)
    icache = torch.zeros((20, 8448), dtype=torch.uint8, device=DEV)
    mcache = torch.zeros((20, 64, 656), dtype=torch.uint8, device=DEV)
    qf = torch.empty((n, 64, 128), dtype=torch.uint8, device=DEV)
    weff = torch.empty((n, 64), dtype=torch.float32, device=DEV)
    qs = torch.empty((n,), dtype=torch.float32, device=DEV)
    outs = (qf, weff, qs, icache, mcache)

    def run():
        sai.indexer_q_quant(q, wt, qf, weff, qs)
        sai.indexer_k_cache_write(k, slot, icache)
        sai.mla_cache_write(kv[:, :512], kv[:, 512:], slot, mcache)

    def reset():
        qf.fill_(0xA5)
        weff.fill_(-7)
        qs.fill_(-7)
        icache.zero_()
        mcache.zero_()

    run()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()   # warm-up on side stream
    torch.cuda.current_stream().wait_stream(s)
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
            assert torch.equal(a, b), f"replay {rep} differs"
        reset()
        run()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert torch.equal(a, b)


@pytest.mark.parametrize("width", [1000, 4096, 4097, 8192, 16385, 32768, 32769, 40000, 65536, 65537,
                                   100000])
def test_topk_every_row_width_path(width):
    """Row widths on both sides of each register-resident size and the
    streaming kernel beyond them; rows of every length class."""
    _say(f"topk_rows: width {width}")
    rng = np.random.default_rng(width)
    rows = 6
    L = rng.standard_normal((rows, width)).astype(np.float32)
    L[1] = np.round(L[1] * 3)                              # heavy ties
    L[2, : width // 2] = -np.inf
    lens = np.array([width, width, width, min(width, 2049), max(width // 3, 1), 2048], np.int32)
    got = sai.topk_rows(torch.from_numpy(L).to(DEV), torch.from_numpy(lens).to(DEV), 2048)
    assert np.array_equal(got.cpu().numpy(), O.topk_rows(L, lens, 2048))


def test_slots_wide_table_elementwise_path():
    _say("topk_to_global_slots: block table wider than the LDS stage")
    rng = np.random.default_rng(8)
    bt = rng.integers(-1, 50000, (3, 9000)).astype(np.int32)
    idx = rng.integers(-1, 9000 * 64, (4, 300)).astype(np.int32)
    req = np.array([0, 2, 1, 7], np.int32)
    got = sai.topk_to_global_slots(torch.from_numpy(idx).to(DEV), torch.from_numpy(req).to(DEV),
                                   torch.from_numpy(bt).to(DEV)).cpu().numpy()
    assert np.array_equal(got, O.topk_to_global_slots(idx, req, bt))


# ---------------------------------------------------------------- past 4 GiB
def test_paged_pipeline_cache_past_4_gib():
    """A 520 000-block pool (4.39 GB): the requests' blocks sit past byte
    2^32, so every cache address needs 64-bit arithmetic.  Logits, top-k and
    slot ids against the oracle on a compact copy of the used blocks."""
    nb_big = 520_000
    ctx = [300, 1000, 65]
    _say(f"paged pipeline with a {nb_big}-block pool (blocks past 4 GiB), contexts {ctx}")
    wl = synth.custom(len(ctx), 2, ctx, num_blocks=40, bt_width=16, seed=61)
    used = np.unique(wl.block_table[wl.block_table >= 0])
    # big ids: the last len(used) blocks of the big pool (offsets > 2^32)
    big_of = {int(b): nb_big - len(used) + i for i, b in enumerate(used)}
    assert min(big_of.values()) * synth.BLOCK_BYTES > 2 ** 32
    bt_big = np.where(wl.block_table >= 0, np.vectorize(lambda b: big_of.get(int(b), -1))(wl.block_table), -1)
    bt_big = bt_big.astype(np.int32)
    pool = torch.empty((nb_big, synth.BLOCK_BYTES), dtype=torch.uint8, device=DEV)
    pool[nb_big - len(used):] = torch.from_numpy(np.tile(synth.poison_block(), (len(used), 1))).to(DEV)
    for b in range(wl.batch):
        c = int(wl.ctx[b])
        nblk = -(-c // 64)
        slots = (bt_big[b, :nblk].astype(np.int64)[:, None] * 64 + np.arange(64)[None, :]).reshape(-1)[:c]
        sai.indexer_k_cache_write(bf16_tensor(wl.k_request(b)), torch.from_numpy(slots).to(DEV), pool)
    q_fp8, w_eff, _ = sai.indexer_q_quant(bf16_tensor(wl.q()), torch.from_numpy(wl.w()).to(DEV))
    btg = torch.from_numpy(bt_big).to(DEV)
    ctxg = torch.from_numpy(wl.ctx).to(DEV)
    logits, row_len, row_req = sai.paged_mqa_logits(q_fp8.view(3, 2, 64, 128), w_eff, pool, btg, ctxg)
    idx, slots = sai.topk_rows_slots(logits, row_len, row_req, btg, 256)
    torch.cuda.synchronize()
    o = OracleWorkload(wl)  # the same tokens in the small pool under the original block ids
    ref = O.paged_mqa_logits(o.q_codes.reshape(3, 2, 64, 128), o.w_eff, o.pool, wl.block_table, wl.ctx, 2,
                             wl.width)
    got = logits.cpu().numpy()
    assert_logits_close(got, ref, "pool past 4 GiB")
    want = O.topk_rows(got, row_len.cpu().numpy(), 256)
    assert np.array_equal(idx.cpu().numpy(), want)
    assert np.array_equal(slots.cpu().numpy(), O.topk_to_global_slots(want, row_req.cpu().numpy(), bt_big))
    del pool
    torch.cuda.empty_cache()
