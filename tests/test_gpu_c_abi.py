"""The C ABI used from plain C (no PyTorch): tests/c/abi_forward.c, built by
__graft_entry__.build(), allocates with hipMalloc, runs dcn4_forward on a
problem whose exact output is a shifted copy of the input, then the backward
(dcn4_backward and dcn4_backward_ws) whose exact grad_x is grad_y shifted
back, and checks both."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c", "abi_forward")


def test_plain_c_client():
    if not os.path.exists(EXE):
        pytest.fail("tests/c/abi_forward is not built (run __graft_entry__.build())")
    print("running the plain C client", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=90)
    print(r.stdout, r.stderr)
    assert r.returncode == 0 and "OK" in r.stdout, r.stdout + r.stderr
