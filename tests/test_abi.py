"""The C-ABI library loads, exports every symbol the headers under include/
declare, and its host-side validation rejects bad arguments without touching a
GPU."""
import ctypes
import glob
import os
import re
import subprocess

import pytest

from sparse_attention_indexer_paged_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

SAI_OK, SAI_EINVAL, SAI_EUNSUPPORTED, SAI_EWORKSPACE = 0, -1, -2, -3


def declared_functions():
    text = "\n".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libsai.so is not built (run __graft_entry__.build())")
    return binding.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    assert names == sorted([
        "sai_status_string", "sai_time_next_launch", "sai_time_span", "indexer_k_cache_write", "indexer_q_quant",
        "indexer_k_rope_cache_write", "indexer_q_rope_quant",
        "gather_indexer_k",
        "paged_mqa_logits", "paged_mqa_logits_visible", "mqa_logits", "mqa_logits_chunked", "topk_workspace_bytes", "topk_rows",
        "topk_to_global_slots", "topk_rows_slots", "topk_rows_slots_noalloc", "mla_cache_write",
        "sparse_mla_workspace_bytes",
        "sparse_mla_decode", "paged_mqa_topk_slots", "paged_mqa_topk_hist_bytes"])


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None
    assert set(binding.SIGNATURES) == set(declared_functions())


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, 7):
        assert binding.status_string(code).startswith("SAI")


def test_validation_needs_no_gpu(lib):
    nul = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(4096)        # never dereferenced: validation fails first
    # null pointers with a non-empty problem
    assert lib.paged_mqa_logits(nul, nul, nul, 10, nul, 4, nul, 2, 1, nul, 256, nul, nul, nul) == SAI_EINVAL
    # next_n outside 1..4, k outside 1..2048
    assert lib.paged_mqa_logits(fake, fake, fake, 10, fake, 4, fake, 2, 5, fake, 256, nul, nul, nul) == SAI_EUNSUPPORTED
    assert lib.paged_mqa_logits(fake, fake, fake, 10, fake, 4, fake, 2, 0, fake, 256, nul, nul, nul) == SAI_EUNSUPPORTED
    assert lib.topk_rows(fake, 256, fake, 3, 0, fake, nul, 0, nul) == SAI_EUNSUPPORTED
    assert lib.topk_rows(fake, 256, fake, 3, 2049, fake, nul, 0, nul) == SAI_EUNSUPPORTED
    # negative sizes
    assert lib.indexer_k_cache_write(fake, 128, fake, -1, fake, 4, nul) == SAI_EINVAL
    assert lib.indexer_k_cache_write(fake, 100, fake, 3, fake, 4, nul) == SAI_EINVAL   # stride < 128
    assert lib.gather_indexer_k(fake, 4, fake, 2, fake, -1, 10, fake, fake, nul) == SAI_EINVAL
    assert lib.mqa_logits(fake, fake, fake, fake, fake, 1, -5, fake, 64, nul, nul, nul) == SAI_EINVAL
    assert lib.topk_to_global_slots(fake, fake, fake, 4, 1, -1, 8, fake, nul) == SAI_EINVAL
    assert lib.indexer_q_quant(nul, nul, 3, nul, nul, nul, nul) == SAI_EINVAL
    # misaligned q
    assert lib.paged_mqa_logits(ctypes.c_void_p(4097), fake, fake, 10, fake, 4, fake, 2, 1, fake, 256, nul, nul, nul) == SAI_EINVAL
    # empty problems are no-ops
    assert lib.paged_mqa_logits(nul, nul, nul, 0, nul, 0, nul, 0, 1, nul, 0, nul, nul, nul) == SAI_OK
    assert lib.topk_rows(nul, 16, nul, 0, 8, nul, nul, 0, nul) == SAI_OK
    assert lib.indexer_k_cache_write(nul, 128, nul, 0, nul, 0, nul) == SAI_OK


def test_topk_workspace_query(lib):
    # rows up to 16384 wide need none, nor rows up to 65536 wide in
    # launches of fewer than 512 rows (one pass); other wider rows keep k
    # (key, column) candidates per 16384-column segment; past 8 segments
    # none again
    assert binding.topk_workspace_bytes(64, 16384, 2048) == 0
    assert binding.topk_workspace_bytes(256, 65536, 2048) == 0
    assert binding.topk_workspace_bytes(511, 65536, 2048) == 0
    assert binding.topk_workspace_bytes(512, 65536, 2048) == 512 * 4 * 2048 * 8
    assert binding.topk_workspace_bytes(64, 65537, 2048) == 64 * 5 * 2048 * 8
    assert binding.topk_workspace_bytes(32, 131072, 2048) == 32 * 8 * 2048 * 8
    assert binding.topk_workspace_bytes(32, 131073, 2048) == 0
    assert binding.topk_workspace_bytes(4, 300000, 100) == 4 * 19 * 100 * 8


def test_topk_rows_slots_host_validation(lib):
    fake = ctypes.c_void_p(4096)
    nul = ctypes.c_void_p(0)
    # null row_req / block_table / out_slots, negative sizes, bad k, no workspace
    assert lib.topk_rows_slots(fake, 256, fake, nul, fake, 4, 2, 3, 8, fake, fake, nul, 0, nul) == SAI_EINVAL
    assert lib.topk_rows_slots(fake, 256, fake, fake, nul, 4, 2, 3, 8, fake, fake, nul, 0, nul) == SAI_EINVAL
    assert lib.topk_rows_slots(fake, 256, fake, fake, fake, 4, 2, 3, 8, fake, nul, nul, 0, nul) == SAI_EINVAL
    assert lib.topk_rows_slots(fake, 256, fake, fake, fake, -1, 2, 3, 8, fake, fake, nul, 0, nul) == SAI_EINVAL
    assert lib.topk_rows_slots(fake, 256, fake, fake, fake, 4, 2, 3, 0, fake, fake, nul, 0, nul) == SAI_EUNSUPPORTED
    assert lib.topk_rows_slots(fake, 131072, fake, fake, fake, 4, 2, 3, 2048, fake, fake, nul, 0, nul) == SAI_EWORKSPACE
    assert lib.topk_rows_slots(nul, 16, nul, nul, nul, 0, 0, 0, 8, nul, nul, nul, 0, nul) == SAI_OK


def test_topk_rows_slots_noalloc_host_validation(lib):
    """The allocation-free entry rejects problems past its built-in buffer
    (16 MiB of segment candidates) and bad arguments before touching any
    device."""
    fake = ctypes.c_void_p(4096)
    nul = ctypes.c_void_p(0)
    f = lib.topk_rows_slots_noalloc
    assert binding.topk_workspace_bytes(128, 131072, 2048) == 16 << 20
    assert f(fake, 131072, fake, fake, fake, 2048, 32, 129, 2048, fake, fake, nul) == -5   # SAI_ESCRATCH
    assert f(fake, 65536, fake, fake, fake, 1024, 256, 512, 2048, fake, fake, nul) == -5   # 32 MiB
    assert binding.status_string(-5).startswith("SAI_ESCRATCH")
    assert f(fake, 65536, fake, fake, fake, 1024, 256, 3, 0, fake, fake, nul) == SAI_EUNSUPPORTED
    assert f(fake, 65536, fake, fake, fake, 1024, 256, 3, 2049, fake, fake, nul) == SAI_EUNSUPPORTED
    assert f(fake, 65536, fake, fake, fake, 1024, 256, -3, 2048, fake, fake, nul) == SAI_EINVAL
    assert f(fake, -1, fake, fake, fake, 1024, 256, 3, 2048, fake, fake, nul) == SAI_EINVAL
    assert f(nul, 16, nul, nul, nul, 0, 0, 0, 8, nul, nul, nul) == SAI_OK


def test_paged_mqa_topk_slots_host_checks(lib):
    """The fused decode step: which shapes take a histogram, its size, and
    argument errors returned before any launch."""
    assert binding.paged_mqa_topk_hist_bytes(128, 4096) == 128 * 1024 * 4
    assert binding.paged_mqa_topk_hist_bytes(511, 16384) == 511 * 1024 * 4
    assert binding.paged_mqa_topk_hist_bytes(512, 4096) == 0       # many rows: segmented path
    assert binding.paged_mqa_topk_hist_bytes(64, 16385) == 0       # wide rows: segmented path
    assert binding.paged_mqa_topk_hist_bytes(0, 4096) == 0
    assert binding.paged_mqa_topk_hist_bytes(64, 0) == 0
    nul, fake = ctypes.c_void_p(0), ctypes.c_void_p(4096)
    f = lib.paged_mqa_topk_slots

    def call(batch=2, next_n=1, stride=256, k=64, hist=fake, hist_bytes=2 * 4096, logits=fake,
             row_len=fake, row_req=fake, slots=fake, ws=nul, ws_bytes=0):
        return f(fake, fake, fake, 10, fake, 4, fake, batch, next_n, logits, stride, row_len, row_req, k,
                 fake, slots, hist, hist_bytes, ws, ws_bytes, nul)

    assert call(batch=0) == SAI_OK
    assert call(batch=-1) == SAI_EINVAL
    assert call(next_n=5) == SAI_EUNSUPPORTED
    assert call(k=0) == SAI_EUNSUPPORTED
    assert call(k=2049) == SAI_EUNSUPPORTED
    assert call(row_len=nul) == SAI_EINVAL          # both row outputs are required here
    assert call(row_req=nul) == SAI_EINVAL
    assert call(slots=nul) == SAI_EINVAL
    assert call(logits=nul) == SAI_EINVAL
    assert call(stride=0) == SAI_EINVAL
    assert call(hist_bytes=2 * 4096 - 4) == SAI_EWORKSPACE
    # rows cut into segments need workspace
    assert call(stride=131072, hist=nul, hist_bytes=0, k=2048) == SAI_EWORKSPACE


def test_fused_producer_host_checks(lib):
    """rope_dim must be even and at most 128, tables and positions present
    when rotating; no device work."""
    nul, fake = ctypes.c_void_p(0), ctypes.c_void_p(4096)
    k = lib.indexer_k_rope_cache_write
    assert k(fake, 128, fake, fake, fake, 10, 63, fake, 3, fake, 4, nul) == SAI_EINVAL    # odd
    assert k(fake, 128, fake, fake, fake, 10, 130, fake, 3, fake, 4, nul) == SAI_EINVAL   # > 128
    assert k(fake, 128, nul, fake, fake, 10, 64, fake, 3, fake, 4, nul) == SAI_EINVAL     # positions
    assert k(fake, 128, fake, nul, fake, 10, 64, fake, 3, fake, 4, nul) == SAI_EINVAL     # cos
    assert k(fake, 128, fake, fake, fake, -1, 64, fake, 3, fake, 4, nul) == SAI_EINVAL    # table rows
    assert k(fake, 100, fake, fake, fake, 10, 64, fake, 3, fake, 4, nul) == SAI_EINVAL    # stride
    assert k(fake, 128, fake, fake, fake, 10, 64, fake, 0, fake, 4, nul) == SAI_OK        # n == 0
    q = lib.indexer_q_rope_quant
    assert q(fake, fake, fake, fake, 10, 3, fake, 2, fake, fake, fake, nul) == SAI_EINVAL
    assert q(fake, fake, fake, nul, 10, 64, fake, 2, fake, fake, fake, nul) == SAI_EINVAL
    assert q(fake, fake, fake, fake, 10, 64, fake, 0, fake, fake, fake, nul) == SAI_OK


def test_topk_missing_workspace_is_rejected(lib):
    fake = ctypes.c_void_p(4096)
    nul = ctypes.c_void_p(0)
    assert lib.topk_rows(fake, 131072, fake, 8, 2048, fake, nul, 0, nul) == SAI_EWORKSPACE
    assert lib.topk_rows(fake, 131072, fake, 8, 2048, fake, fake, 100, nul) == SAI_EWORKSPACE


def test_time_next_launch_host_checks(lib):
    """Arming needs both events or neither; no device work happens here."""
    nul, fake = ctypes.c_void_p(0), ctypes.c_void_p(4096)
    assert lib.sai_time_next_launch(fake, nul) == SAI_EINVAL
    assert lib.sai_time_next_launch(nul, fake) == SAI_EINVAL
    assert lib.sai_time_next_launch(nul, nul) == SAI_OK
    assert lib.sai_time_span(fake, nul) == SAI_EINVAL
    assert lib.sai_time_span(nul, fake) == SAI_EINVAL
    assert lib.sai_time_span(nul, nul) == SAI_OK


def test_mla_cache_write_host_checks(lib):
    """Validation of host arguments; no device work."""
    nul, fake = ctypes.c_void_p(0), ctypes.c_void_p(4096)
    f = lib.mla_cache_write
    assert f(fake, 512, fake, 64, fake, 0, fake, 4, 64, nul) == SAI_OK           # n == 0
    assert f(fake, 512, fake, 64, fake, -1, fake, 4, 64, nul) == SAI_EINVAL      # n < 0
    assert f(fake, 511, fake, 64, fake, 3, fake, 4, 64, nul) == SAI_EINVAL       # kv stride
    assert f(fake, 516, fake, 64, fake, 3, fake, 4, 64, nul) == SAI_EINVAL       # kv stride % 8
    assert f(fake, 512, fake, 63, fake, 3, fake, 4, 64, nul) == SAI_EINVAL       # kpe stride
    assert f(fake, 512, fake, 64, fake, 3, fake, 4, 0, nul) == SAI_EINVAL        # block size
    assert f(nul, 512, fake, 64, fake, 3, fake, 4, 64, nul) == SAI_EINVAL        # null kv
    assert f(ctypes.c_void_p(4104), 512, fake, 64, fake, 3, fake, 4, 64, nul) == SAI_EINVAL  # unaligned


def test_sparse_mla_decode_host_checks(lib):
    """Workspace query and argument validation; no device work."""
    nul, fake = ctypes.c_void_p(0), ctypes.c_void_p(4096)
    ws = lib.sparse_mla_workspace_bytes
    assert ws(128, 128, 2048) == 0                         # 256 64-head workgroups: one pass
    assert ws(64, 128, 2048) == 64 * 128 * 2 * (512 + 2) * 4   # 2 splits fill the chip
    assert ws(2, 16, 2048) == 2 * 16 * 16 * (512 + 2) * 4  # 16-head groups, 16 splits
    assert ws(0, 16, 64) == 0 and ws(4, 24, 64) == 0 and ws(4, 16, 0) == 0
    f = lib.sparse_mla_decode

    def call(q=fake, rows=2, heads=16, nb=4, bs=64, k=64, scale=0.1, out=fake, w=nul, wb=0):
        return f(q, fake, rows, heads, fake, nb, bs, fake, k, scale, out, fake, w, wb, nul)

    assert call(rows=0) == SAI_OK
    assert call(rows=-1) == SAI_EINVAL
    assert call(heads=24) == SAI_EUNSUPPORTED
    assert call(heads=256) == SAI_EUNSUPPORTED
    assert call(bs=0) == SAI_EINVAL
    assert call(nb=0) == SAI_EINVAL
    assert call(k=-1) == SAI_EINVAL
    assert call(q=nul) == SAI_EINVAL
    assert call(out=ctypes.c_void_p(4100)) == SAI_EINVAL
    assert call(scale=float("nan")) == SAI_EINVAL
    assert call(k=2048) == SAI_EWORKSPACE                  # split path needs a workspace
    assert call(k=2048, w=fake, wb=ws(2, 16, 2048) - 1) == SAI_EWORKSPACE


def test_mqa_logits_chunked_host_checks(lib):
    """Argument validation of the chunked prefill call; no device work."""
    nul, fake = ctypes.c_void_p(0), ctypes.c_void_p(4096)
    f = lib.mqa_logits_chunked

    def call(q=fake, cq=fake, ck=fake, batch=2, tq=10, tk=30, stride=64, k=fake):
        return f(q, fake, k, fake, cq, ck, batch, tq, tk, fake, stride, nul, nul, nul)

    assert call(batch=0) == SAI_OK and call(tq=0) == SAI_OK
    assert call(batch=-1) == SAI_EINVAL and call(tk=-1) == SAI_EINVAL
    assert call(ck=nul) == SAI_EINVAL and call(cq=nul) == SAI_EINVAL and call(q=nul) == SAI_EINVAL
    assert call(k=nul) == SAI_EINVAL
    assert call(stride=0) == SAI_EINVAL
    assert call(batch=5000) == SAI_EUNSUPPORTED
