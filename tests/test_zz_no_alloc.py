"""The allocation-free entry point topk_rows_slots_noalloc (segment candidates
in the library's built-in device buffer) against topk_rows_slots with a
caller workspace, bit-exact, on consecutive calls whose sizes shrink (stale
candidates of a larger call must not leak into a smaller one), and against
the oracle's selection and slot map.  Outputs are preallocated, so the calls
under test allocate nothing."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_indexer_paged_amd import binding as sai

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCRATCH_BYTES = 16 << 20


def _say(msg):
    print(msg, flush=True)


def _case(rows, width, seed, batch=3):
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((rows, width)).astype(np.float32)
    L[0, ::7] = 0.25                                  # a block of ties
    L[1] = np.round(L[1] * 2)                         # heavy ties
    lens = rng.integers(1, width + 1, rows).astype(np.int32)
    lens[0], lens[-2] = width, min(width, 2048)
    lens[1] = min(width, 16384)                       # fits one segment
    nblk = -(-width // 64)
    bt = rng.permutation(batch * nblk + 50)[: batch * nblk].reshape(batch, nblk).astype(np.int32)
    bt[1, nblk // 2:] = -1                            # an unused table tail
    req = rng.integers(0, batch, rows).astype(np.int32)
    req[-1] = batch + 2                               # a request outside the batch
    return L, lens, req, bt


def _noalloc(lg, ln, rq, bt, k, idx, slots):
    lib = sai.load()
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.topk_rows_slots_noalloc(P(lg), lg.stride(0), P(ln), P(rq), P(bt), bt.stride(0),
                                       bt.shape[0], lg.shape[0], k, P(idx), P(slots), stream)


def _check(case, k, label):
    L, lens, req, bt = case
    rows, width = L.shape
    need = sai.topk_workspace_bytes(rows, width, k)
    _say(f"{label}: {rows} rows x {width} columns, k={k}, {need} scratch bytes")
    assert need <= SCRATCH_BYTES
    T = lambda a: torch.from_numpy(a).to(DEV)  # noqa: E731
    lg, ln, rq, b = T(L), T(lens), T(req), T(bt)
    ref_idx, ref_slots = sai.topk_rows_slots(lg, ln, rq, b, k)      # caller workspace
    idx = torch.full((rows, k), 7, dtype=torch.int32, device=DEV)
    slots = torch.full((rows, k), 7, dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    assert _noalloc(lg, ln, rq, b, k, idx, slots) == 0
    torch.cuda.synchronize()
    assert torch.equal(idx, ref_idx), label
    assert torch.equal(slots, ref_slots), label
    want = O.topk_rows(L, lens, k)
    assert np.array_equal(idx.cpu().numpy(), want), label
    assert np.array_equal(slots.cpu().numpy(), O.topk_to_global_slots(want, req, bt)), label


def test_noalloc_matches_workspace_entry_on_shrinking_calls():
    # 128 rows x 8 segments x 2048 candidates x 8 B fill the buffer exactly;
    # then fewer rows and segments, then a smaller k over the same buffer
    _check(_case(128, 131072, seed=1), 2048, "call 1 (whole buffer)")
    _check(_case(8, 100000, seed=2), 2048, "call 2 (smaller)")
    _check(_case(5, 70000, seed=3), 300, "call 3 (smaller k)")


def test_noalloc_one_pass_and_streaming_rows():
    # rows that need no scratch: one pass (<= 16384 columns, and <= 65536 in
    # launches of few rows) and rows past the segment-and-merge limit
    # (streaming kernel, slots mapped afterwards)
    _check(_case(64, 16384, seed=4), 2048, "one pass")
    _check(_case(16, 65536, seed=6), 2048, "one pass, wide rows")
    _check(_case(3, 140000, seed=5), 2048, "streaming")


def test_noalloc_rejects_problems_past_the_buffer():
    L = torch.zeros((129, 131072), dtype=torch.float32, device=DEV)
    ln = torch.full((129,), 131072, dtype=torch.int32, device=DEV)
    rq = torch.zeros((129,), dtype=torch.int32, device=DEV)
    bt = torch.zeros((1, 2048), dtype=torch.int32, device=DEV)
    idx = torch.full((129, 2048), 7, dtype=torch.int32, device=DEV)
    slots = torch.full((129, 2048), 7, dtype=torch.int32, device=DEV)
    assert _noalloc(L, ln, rq, bt, 2048, idx, slots) == -5      # SAI_ESCRATCH, nothing launched
    torch.cuda.synchronize()
    assert (idx == 7).all() and (slots == 7).all()
