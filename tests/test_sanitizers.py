"""Host-side sanitizer job: the planner and the oracle built with
AddressSanitizer and UndefinedBehaviorSanitizer (g++ / gcc, host code only;
no GPU code is involved) and driven by

  * tests/sanitize/plan_fuzz.cpp -- random problems and options through
    cbd_plan_ex (including degenerate, out-of-range and G > 256 ones): every
    call returns a status, every accepted plan keeps its invariants;
  * tests/sanitize/oracle_check.c -- the oracle's adjoint identity and the
    equality of its three forms on small integer-valued problems.

Any sanitizer report makes the program exit non-zero.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
       "-g", "-O1"]
ENV = {**os.environ, "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0:exitcode=3",
       "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1:exitcode=4", "OMP_NUM_THREADS": "2"}


def _build(tmp_path, out, cmd):
    exe = os.path.join(str(tmp_path), out)
    r = subprocess.run(cmd + ["-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_planner_fuzz_under_sanitizers(tmp_path):
    csrc = os.path.join(ROOT, "dnn_conv2d_bwd_amd", "csrc")
    exe = _build(tmp_path, "plan_fuzz", ["g++", "-std=c++17", *SAN, "-I", csrc,
                                         os.path.join(HERE, "plan_fuzz.cpp"),
                                         os.path.join(csrc, "cbd_plan.cpp")])
    r = subprocess.run([exe, "200000", "7"], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert "accepted" in r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_identities_under_sanitizers(tmp_path):
    exe = _build(tmp_path, "oracle_check", ["gcc", "-std=c11", *SAN, "-fopenmp", "-ffp-contract=off",
                                            os.path.join(HERE, "oracle_check.c"),
                                            os.path.join(ROOT, "oracle", "cbd_oracle.c"), "-lm"])
    r = subprocess.run([exe, "300"], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert "problems: 300" in r.stdout
