"""Build libsai.so (the gfx950 indexer kernels behind the C ABI of include/sai.h).

Run as ``python -m sparse_attention_indexer_paged_amd.build``; the library is
written next to this file.  hipcc cross-compiles for gfx950, so no GPU is
needed to build.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libsai.so")

SOURCES = ["cache_ops.hip", "logits.hip", "prefill.hip", "topk.hip", "mla.hip"]
OBJDIR = os.path.join(HERE, "_build")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 VALU ops stay off: plain fp32 math only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]

# The logits kernels never rely on NaN semantics of fp operations (masks are
# integer selects): without NaN handling ReLU is one v_max_f32 instead of a
# canonicalise + max pair, and MFMA results go straight to VGPRs (no AGPR
# copies).
PER_FILE = {
    "logits.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"],
    "prefill.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the gfx950-only feature flag; that
    # warning is expected and harmless
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))


def build(verbose=False, defines=(), out=None):
    """Compile every source to an object, then link libsai.so.  ``defines``
    (e.g. ["SAI_DECODE_CHUNK=8"]) and ``out`` serve launch-shape sweeps."""
    os.makedirs(OBJDIR, exist_ok=True)
    dflags = ["-D" + d for d in defines]
    tag = "_".join(d.replace("=", "") for d in defines)
    objs = []
    for src in SOURCES:
        obj = os.path.join(OBJDIR, src.replace(".hip", (("_" + tag) if tag else "") + ".o"))
        _run([hipcc()] + FLAGS + PER_FILE.get(src, []) + dflags + ["-I", INCLUDE, "-I", CSRC, "-c",
             os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    lib = out or LIB
    tmp = lib + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
