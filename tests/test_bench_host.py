"""Host-side logic of bench.py: the FLOP and byte counts the reported throughput and roofline
rest on, the key that ties the committed HBM traffic summary to the kernel's code, and the
single-GPU guard.  No GPU is needed."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import synthetic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_tokens_ignores_comments_and_layout():
    a = "int f(int x) {\n    return x + 1; // add one\n}\n/* block\n comment */\n"
    b = "int f(int x){return x+1;}  // other words\n"
    assert bench.code_tokens(a) == bench.code_tokens(b) == "intf(intx){returnx+1;}"


def test_code_tokens_keeps_literals_and_sees_code_changes():
    src = 'asm volatile("s_nop 0 // not a comment" ::: "memory"); char c = \'"\';'
    toks = bench.code_tokens(src)
    assert '"s_nop 0 // not a comment"' in toks
    assert "'\"'" in toks
    assert bench.code_tokens("x = a + 1;") != bench.code_tokens("x = a + 2;")
    assert bench.code_tokens('s = "a b";') != bench.code_tokens('s = "ab";')


def test_kernel_source_hash_is_stable():
    h = bench.kernel_source_hash()
    assert len(h) == 64 and h == bench.kernel_source_hash()


@pytest.mark.parametrize("wid", [0, 1, 2, 3])
def test_chunk_flops_sum_to_visible_pairs(wid):
    w = synthetic.WORKLOADS[wid]
    total = sum(bench.chunk_flops(w, p0, n) for p0, n in w.chunks())
    assert total == w.visible_pairs() * 4 * w.D


def test_chunk_flops_brute_force():
    w = synthetic.Workload(99, "t", 2, 3, 37, 53, 11, 16, None)
    for p0, n in w.chunks():
        pairs = sum(1 for i in range(w.M) for j in range(p0, p0 + n) if j <= w.q_pos0 + i)
        assert bench.chunk_flops(w, p0, n) == pairs * w.B * w.H * 4 * w.D


@pytest.mark.parametrize("form", ["plain", "fused", "lean"])
def test_algorithmic_bytes_row_by_row(form):
    """Per head and chunk: K and V rows (68 B each), and for every query row that sees a key of
    the chunk its FP16 Q row (128 B), its state read (m, 4 B, except in the lean form's first
    call; l and O, 260 B, unless the row has seen no key before) and written (264 B, except the
    lean form's completed rows); fused and lean, also out (128 B) and lse (4 B) of the rows
    whose position lies in the chunk."""
    w = synthetic.Workload(99, "t", 2, 3, 40, 40, 0, 16, None)
    got = bench.algorithmic_bytes(w, w.chunk, form=form)
    for c, (p0, n) in enumerate(w.chunks()):
        per_head = 2 * 68 * n
        for i in range(w.M):
            pos = w.q_pos0 + i
            if pos < p0:
                continue
            seen_before = p0 > 0
            completed = form != "plain" and pos < p0 + n
            per_head += 128
            per_head += 0 if (form == "lean" and p0 == 0) else 4
            per_head += 260 if seen_before else 0
            per_head += 0 if (form == "lean" and completed) else 264
            per_head += 128 + 4 if completed else 0
        assert got[c] == per_head * w.B * w.H


def test_traffic_summary_keyed_to_code():
    t = bench.read_summary(bench.TRAFFIC_FILE)
    assert len(t["kernel_source_sha256"]) == 64
    expect = float(t["hbm_bytes_per_launch"]) if \
        t["kernel_source_sha256"] == bench.kernel_source_hash() else None
    assert bench.traffic_per_launch() == expect


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv,
                       env={**os.environ, **env}, capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
