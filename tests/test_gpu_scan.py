"""GPU parity of the standalone linear-recurrence scan (pararnn_scan)
against the oracle's step-by-step recurrence (oracle.deer.linear_recurrence,
pinned by a dense block-bidiagonal solve).  Tolerance 1e-5 * max(1, max|x|)
(float32 scan of contracting maps, |A| < 1.1)."""
import numpy as np
import pytest
import torch

from nonlinear_rnn_amd import pararnn as pr
from oracle import deer
from tests.gpu_util import DEV

pytestmark = pytest.mark.gpu


def make(S, B, T, D, seed, with_x0=True):
    rng = np.random.default_rng(seed)
    A = rng.uniform(-1.05, 1.05, (S * S, B, D, T)).astype(np.float32)
    if S == 2:  # keep the 2x2 products contracting on average
        A *= np.float32(0.7)
    b = rng.standard_normal((S, B, D, T)).astype(np.float32)
    x0 = rng.standard_normal((S, B, D)).astype(np.float32) if with_x0 else None
    return A, b, x0


def reference(A, b, x0, reverse):
    SS, B, D, T = A.shape
    S = b.shape[0]
    An = np.moveaxis(A.reshape(S, S, B * D, T), (0, 1), (-2, -1)).astype(np.float64)
    bn = np.moveaxis(b.reshape(S, B * D, T), 0, -1).astype(np.float64)
    x0n = None if x0 is None else np.moveaxis(x0.reshape(S, B * D), 0, -1).astype(np.float64)
    x = deer.linear_recurrence(An, bn, x0n, reverse=reverse)
    return np.moveaxis(x, -1, 0).reshape(S, B, D, T)


def run(A, b, x0, reverse, KW=(0, 0)):
    At = [torch.from_numpy(a).to(DEV) for a in A]
    bt = [torch.from_numpy(v).to(DEV) for v in b]
    x0t = None if x0 is None else [torch.from_numpy(v).to(DEV) for v in x0]
    x = pr.scan(At, bt, x0t, reverse=reverse, steps_per_lane=KW[0], waves_per_block=KW[1])
    torch.cuda.synchronize()
    return np.stack([v.cpu().numpy() for v in x])


@pytest.mark.parametrize("S", [1, 2])
@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("T,KW", [(1, (0, 0)), (63, (1, 1)), (64, (1, 1)), (65, (1, 1)),
                                  (1000, (2, 2)), (1000, (0, 0)), (5000, (4, 4)),
                                  (5003, (1, 1)), (8192, (16, 4)), (777, (8, 2))])
def test_scan_parity(S, reverse, T, KW):
    A, b, x0 = make(S, 2, T, 3, 800 + T)
    got = run(A, b, x0, reverse, KW)
    ref = reference(A, b, x0, reverse)
    assert np.abs(got - ref).max() <= 1e-5 * max(1.0, np.abs(ref).max())


@pytest.mark.parametrize("S", [1, 2])
def test_scan_without_boundary_value(S):
    A, b, _ = make(S, 3, 2000, 4, 811, with_x0=False)
    got = run(A, b, None, False)
    ref = reference(A, b, None, False)
    assert np.abs(got - ref).max() <= 1e-5 * max(1.0, np.abs(ref).max())


@pytest.mark.parametrize("S", [1, 2])
def test_scan_empty(S):
    """No steps, no batch rows or no channels: nothing to do, no error."""
    for B, T, D in [(0, 10, 3), (2, 0, 3), (2, 10, 0)]:
        A, b, x0 = make(S, B, T, D, 812)
        got = run(A, b, x0, False)
        assert got.shape == (S, B, D, T)


def test_scan_is_the_newton_system():
    """One Newton update of the fused solve equals a scan of its own
    Jacobians and residuals: from s = 0 with one update, s^(1) = ds solves
    ds_t = A_t ds_{t-1} - r_t with A_t, r_t evaluated at s = 0."""
    from nonlinear_rnn_amd.inputs import make_inputs
    from tests.gpu_util import gpu_solve
    inp = make_inputs("gru", 1, 3000, 4, 812, s0_std=0.3)
    got, _ = gpu_solve(inp, 0.0, 1)
    u = deer.from_planes(inp.u)
    a = deer.a_per_channel(inp.a, 1)
    s0 = inp.s0[0].reshape(-1, 1).astype(np.float64)
    s = np.zeros((4, 3000, 1))
    J = deer.local_jacobians(deer.GRU, s, s0, u, a)
    r = deer.residual(deer.GRU, s, s0, u, a)
    Ab = J[..., 0, 0].reshape(1, 1, 4, 3000).astype(np.float32)
    bb = (-r[..., 0]).reshape(1, 1, 4, 3000).astype(np.float32)
    x = run(Ab, bb, None, False)
    assert np.abs(x[0] - got[0]).max() < 1e-5
