"""Shared plumbing of the GPU parity tests: uploading a synthetic workload
through the library, building the same workload with the oracle, and the
comparison rules (logits within tolerance, integers bit-exact)."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle as O
from sparse_attention_indexer_paged_amd import binding as sai
from sparse_attention_indexer_paged_amd import synth

DEV = "cuda:0"

# Logit tolerance: |gpu - oracle| <= ATOL + RTOL * |oracle| on every column the
# oracle marks finite; masked columns must be exactly -inf.
RTOL = 1e-3
ATOL = 1e-4


def bf16_tensor(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


class GpuWorkload:
    """A synthetic workload built on the GPU by the library's own producers."""

    def __init__(self, wl, poison=True):
        self.wl = wl
        pool = wl.poisoned_pool() if poison else np.zeros((wl.num_blocks, synth.BLOCK_BYTES), np.uint8)
        self.pool = torch.from_numpy(pool).to(DEV)
        for b in range(wl.batch):
            k = bf16_tensor(wl.k_request(b))
            sm = torch.from_numpy(wl.slots_request(b)).to(DEV)
            sai.indexer_k_cache_write(k, sm, self.pool)
        self.q_bf16 = bf16_tensor(wl.q())
        self.w = torch.from_numpy(wl.w()).to(DEV)
        self.q_fp8, self.w_eff, self.q_scale = sai.indexer_q_quant(self.q_bf16, self.w)
        self.block_table = torch.from_numpy(wl.block_table).to(DEV)
        self.ctx = torch.from_numpy(wl.ctx).to(DEV)
        self.cu = torch.from_numpy(wl.cu_seq_lens).to(DEV)


# The oracle quantises one token row at a time, so its cache writes are cut
# into pieces of this many tokens and run on a thread pool (numpy releases
# the GIL inside its array loops); the bytes written are the same as one
# call per request.
WRITE_PIECE = 1024
WRITE_THREADS = 8


class OracleWorkload:
    """The same workload built on the CPU by the oracle (only the requests
    in ``requests`` get their K written; others stay poison).  With
    ``q_rows`` only those query rows are quantised (the quantiser works per
    token); other rows' codes and weights stay zero."""

    def __init__(self, wl, requests=None, poison=True, q_rows=None):
        self.wl = wl
        self.pool = wl.poisoned_pool() if poison else np.zeros((wl.num_blocks, synth.BLOCK_BYTES), np.uint8)
        reqs = list(range(wl.batch) if requests is None else requests)

        def write(b):
            k = synth.bf16_bits_to_f32(wl.k_request(b))
            sm = wl.slots_request(b)
            for a in range(0, len(sm), WRITE_PIECE):
                O.k_cache_write(k[a:a + WRITE_PIECE], sm[a:a + WRITE_PIECE], self.pool)

        with ThreadPoolExecutor(WRITE_THREADS) as ex:
            list(ex.map(write, reqs))
        q = synth.bf16_bits_to_f32(wl.q())
        w = wl.w()
        if q_rows is None:
            self.q_codes, self.w_eff, self.q_scale = O.quantize_q(q, w)
        else:
            r = np.asarray(q_rows, dtype=np.int64)
            self.q_codes = np.zeros(q.shape, np.uint8)
            self.w_eff = np.zeros(w.shape, np.float32)
            self.q_scale = np.zeros(q.shape[0], np.float32)
            self.q_codes[r], self.w_eff[r], self.q_scale[r] = O.quantize_q(q[r], w[r])


def oracle_topk(logits, row_len, k=2048, rows_per_task=64):
    """O.topk_rows over slices of rows on a thread pool (the selection is per
    row, so the result is the same as one call over all rows)."""
    R = logits.shape[0]
    parts = [slice(a, min(R, a + rows_per_task)) for a in range(0, R, rows_per_task)]
    row_len = np.asarray(row_len)
    with ThreadPoolExecutor(WRITE_THREADS) as ex:
        out = list(ex.map(lambda s: O.topk_rows(logits[s], row_len[s], k), parts))
    return np.concatenate(out) if out else np.full((0, k), -1, np.int32)


def assert_logits_close(gpu, ref, what=""):
    """gpu: float32 array, ref: float64 oracle array of the same shape."""
    gpu = np.asarray(gpu, dtype=np.float64)
    fin = np.isfinite(ref)
    assert not np.isnan(gpu).any(), f"{what}: NaN in GPU logits"
    assert np.all(np.isneginf(gpu[np.isneginf(ref)])), f"{what}: masked column not -inf"
    err = np.abs(gpu[fin] - ref[fin])
    tol = ATOL + RTOL * np.abs(ref[fin])
    bad = err > tol
    if bad.any():
        i = np.argmax(err / tol)
        raise AssertionError(f"{what}: {bad.sum()} of {fin.sum()} logits outside tolerance; "
                             f"worst gpu={gpu[fin][i]} ref={ref[fin][i]}")
    return float((err / tol).max()) if err.size else 0.0
