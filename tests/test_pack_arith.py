"""CPU check (no GPU) of the binary32 arithmetic that the pack kernel's fast path rests on:
the scale division amax / 127 as a product and one FMA correction (correctly rounded for every
finite amax >= 0), and the fast quantiser (an FMA that rounds x times the reciprocal of the FP16
scale to an integer, and the window next to half-integers that it leaves to the exact path).
tests/arith/pack_arith_check.c runs both exhaustively over their domains; the GPU tests in
test_gpu_pack.py check the kernel itself against the oracle bit for bit."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "arith", "pack_arith_check.c")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_pack_arithmetic_exhaustive(tmp_path):
    exe = str(tmp_path / "pack_arith_check")
    r = subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-pthread", SRC, "-o", exe,
                        "-lm"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and r.stdout.strip() == "mismatches 0 0", r.stdout + r.stderr
