"""The C-only client (tests/c_client/cbd_client.c): hipMalloc, cbd_plan,
cbd_run on the default stream, hipMemcpy back, bit-exact comparison with the
oracle on integer-valued operands, for one problem of each kernel family --
the library as a plain C program uses it, with no torch in the process.

The program is built by __graft_entry__.build() (gcc against include/cbd.h,
libcbd.so and the HIP runtime)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_client", "cbd_client")


def test_c_client_builds_against_header_only():
    """CPU: the client is built (and so compiles as C against cbd.h alone)."""
    assert os.path.exists(EXE), "run __graft_entry__.build() first"


@pytest.mark.gpu
def test_c_client_end_to_end():
    assert os.path.exists(EXE), "the C client is not built (__graft_entry__.build())"
    print("[c-client] running", EXE, flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "CLIENT OK" in r.stdout
    assert r.stdout.count(" 0 mismatches") == 5
