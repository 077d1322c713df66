"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

Two randomised drivers, each built with gcc/g++ -fsanitize=address,undefined
and -fno-sanitize-recover, run to completion with no report:
  * tests/sanitize/plan_fuzz.cpp over the library's plan encoder and plan
    readers (quantized_momentum_newton_amd/csrc/plan.cpp, host-only C++);
  * tests/sanitize/oracle_fuzz.c over the CPU oracle's C part (oracle/q8.c).
The two are separate programs: the library and the oracle share no code.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1",
           OMP_NUM_THREADS="4")


def _build_and_run(cmd, exe, args, tmp_path):
    if shutil.which(cmd[0]) is None:
        pytest.skip(f"{cmd[0]} not available")
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([str(exe), *args], capture_output=True, text=True, env=ENV, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    return r.stdout


def test_plan_encoder_under_asan_ubsan(tmp_path):
    exe = tmp_path / "plan_fuzz"
    csrc = os.path.join(ROOT, "quantized_momentum_newton_amd", "csrc")
    cmd = ["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"), "-I", csrc,
           os.path.join(ROOT, "tests", "sanitize", "plan_fuzz.cpp"), os.path.join(csrc, "plan.cpp"), "-o", str(exe)]
    out = _build_and_run(cmd, exe, ["3000"], tmp_path)
    assert "0 failed checks" in out, out


def test_oracle_c_under_asan_ubsan(tmp_path):
    exe = tmp_path / "oracle_fuzz"
    cmd = ["gcc", "-std=c11", "-fopenmp", "-ffp-contract=off", *SAN,
           os.path.join(ROOT, "tests", "sanitize", "oracle_fuzz.c"), os.path.join(ROOT, "oracle", "q8.c"),
           "-o", str(exe), "-lm"]
    out = _build_and_run(cmd, exe, ["300"], tmp_path)
    assert "0 failed checks" in out, out
