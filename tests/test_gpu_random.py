"""Randomised parity sweeps: 48 solve configurations drawn from fixed seeds, each a
mix the hand-written cases do not cover together: cell, projection dtype,
batch, channels, a length that is rarely a tile multiple, forced or
automatic tiling, channel- or time-major planes, and a cold or warm
(init_from_output) Newton start.  Every solve is checked against the fp64
sequential oracle at the float32 tolerance (1e-5 max-abs; bf16 projections
against the oracle on the same rounded values), and must report
convergence with max|r| < tol.  The draw is deterministic, so a failing
case is named by its index.
"""
import numpy as np
import pytest
import torch

from nonlinear_rnn_amd import pararnn as pr
from nonlinear_rnn_amd.inputs import make_inputs
from tests.gpu_util import DEV, dev_inputs, max_err, oracle_states

pytestmark = pytest.mark.gpu

N_CASES = 48
TILINGS = [(0, 0), (1, 1), (2, 2), (4, 1), (4, 4), (8, 2), (16, 1), (16, 4), (1, 8), (2, 8)]


def draw(i):
    rng = np.random.default_rng(1000 + i)
    cell = ["gru", "lstm"][rng.integers(2)]
    B = int(rng.integers(1, 4))
    D = int(rng.integers(1, 40))
    T = int(rng.choice([1, 2, 3, 63, 65, 127, 129, 500, 1000, 2049, 4097, 5000]))
    if rng.random() < 0.25:
        T = int(rng.integers(1, 6000))
    KW = TILINGS[rng.integers(len(TILINGS))]
    return dict(cell=cell, B=B, D=D, T=T, K=KW[0], W=KW[1],
                bf16=bool(rng.random() < 0.3), time_major=bool(rng.random() < 0.3),
                warm=bool(rng.random() < 0.25), seed=2000 + i)


def time_major_views(planes):
    """The same values as views of one [B][T][G*D] tensor."""
    G = len(planes)
    B, D, T = planes[0].shape
    full = torch.empty((B, T, G * D), dtype=planes[0].dtype, device=DEV)
    for g, p in enumerate(planes):
        full[:, :, g * D:(g + 1) * D] = p.transpose(1, 2)
    return [full[:, :, g * D:(g + 1) * D].transpose(1, 2) for g in range(G)]


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_configuration(i):
    c = draw(i)
    print(f"\n[case {i}] {c}", flush=True)
    inp = make_inputs(c["cell"], c["B"], c["T"], c["D"], c["seed"], s0_std=0.3,
                      f_bias=1.0 if c["cell"] == "lstm" else 0.0,
                      u_dtype="bf16" if c["bf16"] else "f32")
    u, a, s0 = dev_inputs(inp)
    if c["time_major"]:
        u = time_major_views(u)
    ref = oracle_states(inp, rounded=True)
    S = len(ref)
    out = None
    if c["warm"]:
        # a perturbed oracle trajectory as the Newton start
        rng = np.random.default_rng(c["seed"])
        out = [torch.from_numpy((r + 0.05 * rng.standard_normal(r.shape)).astype(np.float32))
               .to(DEV) for r in ref]
        if c["time_major"]:
            out = [o.transpose(1, 2).contiguous().transpose(1, 2) for o in out]
    kw = dict(tol=1e-6, max_iters=40, steps_per_lane=c["K"], waves_per_block=c["W"],
              init_from_output=c["warm"])
    if c["cell"] == "gru":
        h, info = pr.solve_gru(u, a, s0[0], out=None if out is None else out[0], **kw)
        got = [h]
    else:
        (cc, h), info = pr.solve_lstm(u, a, s0[0], s0[1], out=out, **kw)
        got = [cc, h]
    info = pr.read_info(info)
    assert info["converged"] and info["max_abs_res"] < 1e-6, info
    assert len(got) == S
    err = max_err([g.cpu().numpy() for g in got], ref)
    assert err < 1e-5, err


@pytest.mark.parametrize("i", range(24))
def test_random_adjoint(i):
    """The adjoint on random configurations (time-major planes included),
    against the oracle's back-propagation through time on the same rounded
    projections; the device is fed the oracle trajectory, so the backward
    pass is compared alone.  Tolerance 1e-5 * max(1, max|ref|) per tensor."""
    from tests.test_gpu_adjoint import bptt, grad_close
    c = draw(100 + i)
    print(f"\n[adjoint case {i}] {c}", flush=True)
    inp = make_inputs(c["cell"], c["B"], c["T"], c["D"], c["seed"], s0_std=0.3,
                      f_bias=1.0 if c["cell"] == "lstm" else 0.0,
                      u_dtype="bf16" if c["bf16"] else "f32", with_grad=True)
    ref, states, ds0, lam = bptt(inp)
    u, a, s0 = dev_inputs(inp)
    s = [torch.from_numpy(x.astype(np.float32)).to(DEV) for x in states]
    dh = torch.from_numpy(inp.dh).to(DEV)
    if c["time_major"]:
        u = time_major_views(u)
        s = [x.transpose(1, 2).contiguous().transpose(1, 2) for x in s]
        dh = dh.transpose(1, 2).contiguous().transpose(1, 2)
    gs = [dh] if c["cell"] == "gru" else [None, dh]
    out = pr.adjoint(c["cell"], u, a, s0, s, gs, with_lambda=True,
                     steps_per_lane=c["K"], waves_per_block=c["W"])
    for g in range(len(inp.u)):
        grad_close(out["du"][g].cpu().numpy(), ref["du"][g])
    grad_close(out["da"].cpu().numpy(), ref["da"])
    for k in range(len(states)):
        grad_close(out["ds0"][k].cpu().numpy(), ds0[k])
        grad_close(out["lam"][k].cpu().numpy(), lam[k])


@pytest.mark.parametrize("i", range(24))
def test_random_scan(i):
    """The standalone scan on random configurations (state size, direction,
    boundary value or none, tiling, time-major planes) against the oracle's
    step-by-step recurrence; tolerance 1e-5 * max(1, max|x|)."""
    from tests.test_gpu_scan import make, reference
    c = draw(200 + i)
    rng = np.random.default_rng(c["seed"])
    S, reverse, with_x0 = int(rng.integers(1, 3)), bool(rng.random() < 0.5), bool(rng.random() < 0.7)
    print(f"\n[scan case {i}] {c} S={S} reverse={reverse} x0={with_x0}", flush=True)
    A, b, x0 = make(S, c["B"], c["T"], c["D"], c["seed"], with_x0)
    ref = reference(A, b, x0, reverse)
    At = [torch.from_numpy(v).to(DEV) for v in A]
    bt = [torch.from_numpy(v).to(DEV) for v in b]
    if c["time_major"]:
        At = [v.transpose(1, 2).contiguous().transpose(1, 2) for v in At]
        bt = [v.transpose(1, 2).contiguous().transpose(1, 2) for v in bt]
    x0t = None if x0 is None else [torch.from_numpy(v).to(DEV) for v in x0]
    x = pr.scan(At, bt, x0t, reverse=reverse, steps_per_lane=c["K"], waves_per_block=c["W"])
    got = np.stack([v.cpu().numpy() for v in x])
    scale = max(1.0, float(np.abs(ref).max()))
    assert float(np.abs(got - ref).max()) <= 1e-5 * scale
