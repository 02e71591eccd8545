"""The C ABI from a C++ program with no Python in it: tests/c_abi_check
(built by the package build from tests/c_abi_check.cpp) allocates device
memory with the HIP runtime, calls pararnn_solve_gru / pararnn_solve_lstm /
pararnn_adjoint with workspaces sized by pararnn_workspace_bytes, and
compares with the oracle's C library (fp64).  Bounds: 1e-5 max-abs for
states, 1e-5 relative to max(1, max|ref|) for gradients."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_check")


def test_c_abi_consumer_matches_oracle():
    if not os.path.exists(EXE):
        pytest.skip("tests/c_abi_check not built (python tests/build_c_abi_check.py)")
    res = subprocess.run([EXE], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                         timeout=120)
    print(res.stdout)
    assert res.returncode == 0, res.stdout
    assert "0 failure(s)" in res.stdout
