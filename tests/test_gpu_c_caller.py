"""The ABI from a plain C program (tests/c/abi_from_c.c, built by
__graft_entry__.build()): device buffers from the HIP runtime's C API, a
workspace sized by os_softmax_workspace_bytes, os_softmax_fwd on shapes that
take the resident, stream and split paths, each checked against the fp64
oracle linked into the same program (fp32 y to 1e-6 + 1e-5 |y|, bf16 y to
one bf16 step, m bit-exact, lse to 1e-5 + 2 ulp).  The program runs as a
child process with its own HIP context."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "c", "abi_from_c")


def test_plain_c_caller_matches_the_oracle():
    assert os.path.exists(BIN), f"{BIN} missing: run __graft_entry__.build()"
    print("C caller: fp32 600x3001 (resident), bf16 520x40000 (stream), "
          "fp32 3x300001 (split)", flush=True)
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=300)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks hold" in r.stdout
