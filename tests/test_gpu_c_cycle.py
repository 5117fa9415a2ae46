"""A whole cycle (selection, device-length draft steps, verify, acceptance)
driven through the C ABI from a HIP C++ program with no Python or torch in
it (tests/cycle_from_c.hip, built in-tree by the package build).  The
program checks the properties that need no oracle; the float64 parity of
every call is in the other GPU tests."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROGRAM = os.path.join(ROOT, "tests", "_build", "cycle_from_c")

pytestmark = pytest.mark.gpu


def test_cycle_driven_from_c():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(PROGRAM):
        pytest.skip(f"{PROGRAM} is not built (__graft_entry__.build() builds it)")
    res = subprocess.run([PROGRAM], capture_output=True, text=True, timeout=120)
    print(res.stdout, flush=True)
    sys.stdout.flush()
    assert res.returncode == 0, res.stdout + res.stderr
    assert "0 failure(s)" in res.stdout
