"""Shared plumbing of the GPU parity tests: uploading a synthetic workload
through the library, building the same workload with the oracle, and the
comparison rules (logits within tolerance, integers bit-exact)."""
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


class OracleWorkload:
    """The same workload built on the CPU by the oracle (only the requests
    in ``requests`` get their K written; others stay poison)."""

    def __init__(self, wl, requests=None, poison=True):
        self.wl = wl
        self.pool = wl.poisoned_pool() if poison else np.zeros((wl.num_blocks, synth.BLOCK_BYTES), np.uint8)
        reqs = range(wl.batch) if requests is None else requests
        for b in reqs:
            O.k_cache_write(synth.bf16_bits_to_f32(wl.k_request(b)), wl.slots_request(b), self.pool)
        q = synth.bf16_bits_to_f32(wl.q())
        self.q_codes, self.w_eff, self.q_scale = O.quantize_q(q, wl.w())


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
