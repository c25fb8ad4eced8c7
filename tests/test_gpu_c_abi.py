"""The C ABI from plain C: ``tests/c_abi/ew_c_client`` (built by
``__graft_entry__.build()``) allocates with the HIP runtime's C API, calls the
library on its own stream, and compares every element with the CPU oracle.
It runs as a child process with no torch in it."""
import os
import subprocess

import pytest

from tests.conftest import ROOT

pytestmark = pytest.mark.gpu

EXE = os.path.join(ROOT, "tests", "c_abi", "ew_c_client")


def test_plain_c_client_matches_the_oracle():
    assert os.path.exists(EXE), "build the C client first: python __graft_entry__.py"
    print("[c-abi] running the plain C client", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "checks passed" in r.stdout and "FAIL" not in r.stderr, r.stdout + r.stderr
