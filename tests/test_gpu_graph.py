"""The entry points under HIP graph capture: a solve (with its info record),
a multi-block solve (its init kernel), the adjoint, the scan and a staged
time-major solve are captured once with torch.cuda.graph and replayed
several times, with the program's own eager work and synchronisations
between the replays.  Every replay must reproduce the eager call bitwise,
also after the inputs are overwritten in place (the graph reads them
again).  The launches enqueue kernels only (no memset or copy nodes), so a
graph is a plain chain of kernel nodes.
"""
import pytest
import torch

from nonlinear_rnn_amd import pararnn as pr
from nonlinear_rnn_amd.inputs import make_inputs
from tests.gpu_util import DEV, dev_inputs

pytestmark = pytest.mark.gpu


def eager_noise():
    """Unrelated eager work between replays."""
    x = torch.randn((512, 512), device=DEV)
    y = (x @ x).sum()
    torch.cuda.synchronize()
    return float(y)


def capture(fn):
    """Warm up on a side stream (workspaces get allocated), then capture."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    return g, out


def flat(x):
    if isinstance(x, torch.Tensor):
        return [x]
    if isinstance(x, dict):
        return [t for k in sorted(x) for t in flat(x[k])]
    if isinstance(x, (list, tuple)):
        return [t for v in x for t in flat(v)]
    return []


def same(a, b):
    fa, fb = flat(a), flat(b)
    assert len(fa) == len(fb)
    for x, y in zip(fa, fb):
        assert torch.equal(x, y)


def check_replays(fn, perturb):
    g, out = capture(fn)
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        same(out, fn())
        eager_noise()
    perturb()
    g.replay()
    torch.cuda.synchronize()
    same(out, fn())


@pytest.mark.parametrize("cell", ["gru", "lstm"])
@pytest.mark.parametrize("KW", [(0, 0), (1, 1)])
def test_solve_replays(cell, KW):
    inp = make_inputs(cell, 2, 700, 12, 91, s0_std=0.3, f_bias=1.0)
    u, a, s0 = dev_inputs(inp)

    def fn():
        kw = dict(tol=1e-6, max_iters=20, steps_per_lane=KW[0], waves_per_block=KW[1])
        if cell == "gru":
            h, info = pr.solve_gru(u, a, s0[0], **kw)
            return [h, info]
        (c, h), info = pr.solve_lstm(u, a, s0[0], s0[1], **kw)
        return [c, h, info]

    def perturb():
        u[0].mul_(0.5)

    check_replays(fn, perturb)


def test_adjoint_and_scan_replay():
    inp = make_inputs("lstm", 2, 900, 8, 92, f_bias=1.0)
    u, a, s0 = dev_inputs(inp)
    (c, h), _ = pr.solve_lstm(u, a, s0[0], s0[1], tol=1e-6, max_iters=20)
    gh = torch.randn(h.shape, device=DEV)

    def adj():
        return pr.adjoint("lstm", u, a, s0, [c, h], [None, gh], steps_per_lane=1,
                          waves_per_block=1)

    check_replays(adj, lambda: gh.mul_(-1.0))

    A = torch.rand((2, 8, 900), device=DEV) * 0.9
    b = torch.randn((2, 8, 900), device=DEV)
    x0 = torch.randn((2, 8), device=DEV)

    def scan():
        return pr.scan([A], [b], [x0], steps_per_lane=1, waves_per_block=1)

    check_replays(scan, lambda: b.add_(1.0))


def test_time_major_solve_replays():
    """Staged route: transposes into the workspace, solve, transpose back."""
    inp = make_inputs("gru", 2, 640, 24, 93, s0_std=0.3)
    u, a, s0 = dev_inputs(inp)
    B, D, T = u[0].shape
    full = torch.empty((B, T, 3 * D), device=DEV)
    for g in range(3):
        full[:, :, g * D:(g + 1) * D] = u[g].transpose(1, 2)
    ut = [full[:, :, g * D:(g + 1) * D].transpose(1, 2) for g in range(3)]

    def fn():
        h, info = pr.solve_gru(ut, a, s0[0], tol=1e-6, max_iters=20)
        assert h.stride(1) == 1  # states follow the time-major projections
        return [h, info]

    check_replays(fn, lambda: full.mul_(0.75))
