"""Host-side checks of the benchmark's command-line contract (no GPU)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=60)
    assert res.returncode == 2
    assert "one GPU only" in res.stderr
    assert res.stdout == ""


def test_entry_module_has_build_and_smoke():
    sys.path.insert(0, ROOT)
    try:
        import __graft_entry__ as entry
    finally:
        sys.path.pop(0)
    assert callable(entry.build) and callable(entry.smoke)
