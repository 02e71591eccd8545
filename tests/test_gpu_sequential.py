"""GPU parity of the step-by-step application (pararnn_sequential) against
the fp64 sequential oracle, and its agreement with the Newton solve.
Tolerance 1e-5 max-abs (float32 states), as for the solve."""
import numpy as np
import pytest
import torch

from nonlinear_rnn_amd import pararnn as pr
from nonlinear_rnn_amd.inputs import make_inputs
from tests.gpu_util import dev_inputs, gpu_solve, max_err, oracle_states

pytestmark = pytest.mark.gpu

TOL32 = 1e-5


def run(inp, out=None):
    u, a, s0 = dev_inputs(inp)
    got = pr.sequential(inp.cell, u, a, s0, out=out)
    torch.cuda.synchronize()
    return [g.cpu().numpy() for g in got]


@pytest.mark.parametrize("cell", ["gru", "lstm"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 15, 16, 31, 32, 33, 1000, 4100])
def test_sequential_parity(cell, dtype, T):
    inp = make_inputs(cell, 2, T, 65, 2100 + T, u_dtype=dtype, s0_std=0.3, f_bias=1.0)
    assert max_err(run(inp), oracle_states(inp, rounded=True)) < TOL32


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_sequential_matches_newton_solve(cell):
    inp = make_inputs(cell, 3, 2048, 40, 2200, s0_std=0.2, f_bias=1.0)
    seq = run(inp)
    newton, info = gpu_solve(inp, 1e-6, 30)
    assert info["converged"]
    assert max_err(seq, [n.astype(np.float64) for n in newton]) < 2 * TOL32


def test_sequential_strided_planes():
    inp = make_inputs("lstm", 2, 301, 3, 2300, s0_std=0.1, f_bias=1.0)
    u, a, s0 = dev_inputs(inp)
    big = [torch.zeros((2, 3, 309), device="cuda") for _ in range(4)]
    for g in range(4):
        big[g][:, :, 3:304] = u[g]
    uv = [x[:, :, 3:304] for x in big]
    ob = [torch.zeros((2, 3, 305), device="cuda") for _ in range(2)]
    out = [x[:, :, 1:302] for x in ob]
    pr.sequential("lstm", uv, a, s0, out=out)
    torch.cuda.synchronize()
    assert max_err([o.cpu().numpy() for o in out], oracle_states(inp)) < TOL32
    for x in ob:
        assert float(x[:, :, 0].abs().max()) == 0.0 and float(x[:, :, 302:].abs().max()) == 0.0


def test_sequential_empty():
    for B, T, D in [(0, 10, 3), (2, 0, 3), (2, 10, 0)]:
        inp = make_inputs("gru", B, T, D, 1)
        got = run(inp)
        assert got[0].shape == (B, D, T)
