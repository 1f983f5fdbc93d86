"""The C ABI from a C++ caller with no Python in the loop: tests/c_abi/
gdn_c_demo.cpp (built with the library by __graft_entry__.build()) owns its
device memory through the HIP runtime and checks that the fused and two-pass
prefill paths agree bit for bit and that T decode steps equal one T-token
call.  It runs as a child process."""
import os
import subprocess

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEMO = os.path.join(ROOT, "tests", "c_abi", "gdn_c_demo")


def test_c_abi_caller():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(DEMO), "build the demo with __graft_entry__.build()"
    r = subprocess.run([DEMO], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0 and r.stdout.startswith("OK")
