"""Builds libq8attn.so in-tree with hipcc for gfx950 (cross-compiles without a GPU)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libq8attn.so")
# per-source extra flags.  The attention kernels never rely on NaN propagation (logits that could
# be NaN -- garbage bytes past a chunk end -- are replaced by the causal/range mask with a select
# before any arithmetic), so NaN-honouring canonicalisation is dropped there.
SOURCES = {"api.hip": [], "attn.hip": ["-fno-honor-nans"], "pack.hip": []}

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed FP32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only feature flag; that warning is expected
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if msgs and verbose:
        print("\n".join(msgs), file=sys.stderr)


def build(verbose: bool = False) -> str:
    tmpdir = tempfile.mkdtemp(prefix="q8attn_build_")
    try:
        objs = []
        for src, extra in SOURCES.items():
            obj = os.path.join(tmpdir, src + ".o")
            _run([HIPCC] + FLAGS + extra + ["-c", os.path.join(CSRC, src), "-o", obj], verbose)
            objs.append(obj)
        tmp = LIB + ".tmp%d" % os.getpid()
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
