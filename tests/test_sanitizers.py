"""CPU sanitizer tier (no GPU): the host code under AddressSanitizer + UndefinedBehaviorSanitizer
and ThreadSanitizer.

* The C ABI's host code (chunked_flashattention_q8_amd/csrc/api.hip: argument checks, the state
  flags, the double-buffered streaming loop and the storage feed with its reader threads) is
  compiled as plain C++ with g++ and linked with tests/sanitize/host_harness.cpp, a fake
  in-process HIP runtime whose streams run copies as early as their events allow and whose
  stub kernel launches check, when they run, the bytes each chunk launch reads.  Built once
  with -fsanitize=address,undefined and once with -fsanitize=thread.
* The oracle (oracle/q8_oracle.c) is built with -fsanitize=address,undefined and the oracle's
  own pin tests run against that build in a child process (the ASan runtime preloaded).
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "chunked_flashattention_q8_amd", "csrc")
HARNESS = os.path.join(ROOT, "tests", "sanitize", "host_harness.cpp")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                                reason="needs gcc and g++")


def _gcc_runtime(name):
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _build_harness(tmp_path, sanitize):
    exe = str(tmp_path / ("harness_" + sanitize.replace(",", "_")))
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=" + sanitize,
           "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, os.path.join(CSRC, "api.hip"),
           "-x", "c++", HARNESS, "-pthread", "-o", exe]
    if "undefined" in sanitize:
        cmd.insert(5, "-fno-sanitize-recover=undefined")
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    return exe


@pytest.mark.skipif(not os.path.isdir("/opt/rocm/include/hip"), reason="needs the HIP headers")
@pytest.mark.parametrize("sanitize", ["address,undefined", "thread"])
def test_host_harness(tmp_path, sanitize):
    exe = _build_harness(tmp_path, sanitize)
    env = dict(os.environ, TMPDIR=str(tmp_path),
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and "ALL OK" in r.stdout, r.stdout[-2000:] + r.stderr[-6000:]


def test_oracle_tests_under_asan_ubsan(tmp_path):
    asan = _gcc_runtime("libasan.so")
    if asan is None:
        pytest.skip("no libasan")
    lib = str(tmp_path / "libq8oracle_asan.so")
    r = subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                        "-fPIC", "-shared", "-pthread", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=undefined",
                        os.path.join(ROOT, "oracle", "q8_oracle.c"), "-o", lib, "-lm"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    log = str(tmp_path / "asan")
    env = dict(os.environ, Q8_ORACLE_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:log_path=" + log,
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:log_path=" + log)
    tests = [os.path.join(ROOT, "tests", t) for t in
             ("test_oracle_f16.py", "test_oracle_pack.py", "test_oracle_attn.py",
              "test_oracle_sizes.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider"] +
                       tests, capture_output=True, text=True, timeout=600, env=env, cwd=ROOT)
    reports = ""
    for f in os.listdir(tmp_path):
        if f.startswith("asan"):
            reports += open(os.path.join(tmp_path, f)).read()[-4000:]
    assert r.returncode == 0 and not reports, r.stdout[-2000:] + reports
