"""GPU parity of every entry point on plane layouts other than channel-major
[B][D][T]: time-major [B][T][D] planes, and the gate blocks of one
[B][T][G*D] projection tensor passed as strided views (no copy).

Each case runs the same call on channel-major copies of the same inputs and
requires bitwise-equal results (the arithmetic is identical, only the loads
and stores differ), and checks the time-major result against the CPU oracle
at the usual tolerances (1e-5 max-abs for float32 states, 1e-5 * max(1,
|ref|) for gradients and scans).
"""
import ctypes

import numpy as np
import pytest
import torch

from nonlinear_rnn_amd import autograd as pag
from nonlinear_rnn_amd import pararnn as pr
from nonlinear_rnn_amd.inputs import make_inputs
from oracle import sequential as seq
from tests.gpu_util import DEV, dev_inputs, max_err, oracle_states

pytestmark = pytest.mark.gpu


def interleaved(planes):
    """Channel-major [B][D][T] planes -> one time-major [B][T][G*D] tensor
    and its gate blocks as [B][D][T]-indexed views."""
    G = len(planes)
    B, D, T = planes[0].shape
    full = torch.empty((B, T, G * D), dtype=planes[0].dtype, device=DEV)
    for g, p in enumerate(planes):
        full[:, :, g * D:(g + 1) * D] = p.transpose(1, 2)
    return full, [full[:, :, g * D:(g + 1) * D].transpose(1, 2) for g in range(G)]


def time_major(p):
    """A time-major copy of a [B][D][T] plane, as a [B][D][T]-indexed view."""
    return p.transpose(1, 2).contiguous().transpose(1, 2)


def tm_empty(B, D, T):
    return torch.empty((B, T, D), dtype=torch.float32, device=DEV).transpose(1, 2)


def solve(cell, u, a, s0, out=None, **kw):
    if cell == "gru":
        h, info = pr.solve_gru(u, a, s0[0], out=None if out is None else out[0], **kw)
        return [h], pr.read_info(info)
    (c, h), info = pr.solve_lstm(u, a, s0[0], s0[1], out=out, **kw)
    return [c, h], pr.read_info(info)


@pytest.mark.parametrize("cell", ["gru", "lstm"])
@pytest.mark.parametrize("udt", ["f32", "bf16"])
@pytest.mark.parametrize("T,KW", [(1, (0, 0)), (65, (1, 1)), (1000, (0, 0)), (1000, (2, 2)),
                                  (4100, (4, 4)), (4096, (16, 4))])
def test_solve_time_major(cell, udt, T, KW):
    inp = make_inputs(cell, 2, T, 5, 4000 + T, u_dtype=udt, s0_std=0.1, f_bias=1.0)
    u, a, s0 = dev_inputs(inp)
    ref, ref_info = solve(cell, u, a, s0, tol=1e-6, max_iters=40, steps_per_lane=KW[0],
                          waves_per_block=KW[1])
    _, ut = interleaved(u)
    got, info = solve(cell, ut, a, s0, tol=1e-6, max_iters=40, steps_per_lane=KW[0],
                      waves_per_block=KW[1])
    for g in got:  # default outputs follow the layout of u
        assert g.stride()[2] != 1 or T == 1
    for g, r in zip(got, ref):
        assert torch.equal(g, r)
    assert info == ref_info
    assert info["converged"]
    assert max_err([g.cpu().numpy() for g in got], oracle_states(inp, rounded=True)) < 1e-5


@pytest.mark.parametrize("cell", ["gru", "lstm"])
@pytest.mark.parametrize("KW", [(0, 0), (1, 2)])
def test_time_major_gather_route(cell, KW):
    """With a workspace too small to stage the planes channel-major, the solve
    gathers the time-major steps directly; same bits either way."""
    inp = make_inputs(cell, 2, 1000, 5, 4050, s0_std=0.1, f_bias=1.0)
    u, a, s0 = dev_inputs(inp)
    kw = dict(tol=1e-6, max_iters=40, steps_per_lane=KW[0], waves_per_block=KW[1])
    ref, ref_info = solve(cell, u, a, s0, **kw)
    _, ut = interleaved(u)
    nws = pr.workspace_bytes(cell, pr.make_shape(2, 1000, 5),
                             pr.make_newton(1e-6, 40, KW[0], KW[1]))
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=DEV)
    got, info = solve(cell, ut, a, s0, workspace=ws, **kw)
    for g, r in zip(got, ref):
        assert torch.equal(g, r)
    assert info == ref_info


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_solve_mixed_layouts(cell):
    """Time-major projections into channel-major states and the reverse."""
    inp = make_inputs(cell, 3, 777, 4, 4101, s0_std=0.2, f_bias=1.0)
    u, a, s0 = dev_inputs(inp)
    ref, _ = solve(cell, u, a, s0)
    _, ut = interleaved(u)
    S = len(s0)
    cm_out = [torch.empty((3, 4, 777), dtype=torch.float32, device=DEV) for _ in range(S)]
    got, _ = solve(cell, ut, a, s0, out=cm_out)
    for g, r in zip(got, ref):
        assert torch.equal(g, r)
    got, _ = solve(cell, u, a, s0, out=[tm_empty(3, 4, 777) for _ in range(S)])
    for g, r in zip(got, ref):
        assert torch.equal(g, r)


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_warm_start_time_major(cell):
    """init_from_output over several time blocks reads its start (and the
    states just before each block) from time-major planes."""
    inp = make_inputs(cell, 2, 700, 3, 4102, s0_std=0.1, f_bias=1.0)
    u, a, s0 = dev_inputs(inp)
    kw = dict(tol=1e-6, max_iters=40, steps_per_lane=1, waves_per_block=2)
    first, _ = solve(cell, u, a, s0, tol=0.0, max_iters=2, steps_per_lane=1, waves_per_block=2)
    cm = [x.clone() for x in first]
    ref, ref_info = solve(cell, u, a, s0, out=cm, init_from_output=True, **kw)
    tm = [time_major(x) for x in first]
    got, info = solve(cell, u, a, s0, out=tm, init_from_output=True, **kw)
    for g, r in zip(got, ref):
        assert torch.equal(g, r)
    assert info == ref_info and info["converged"]


@pytest.mark.parametrize("cell", ["gru", "lstm"])
@pytest.mark.parametrize("T,KW", [(300, (0, 0)), (1000, (1, 2)), (4100, (4, 4))])
def test_adjoint_time_major(cell, T, KW):
    inp = make_inputs(cell, 2, T, 5, 4200 + T, s0_std=0.3, f_bias=1.0, with_grad=True)
    u, a, s0 = dev_inputs(inp)
    if cell == "gru":
        r = seq.gru_bptt(inp.u_rounded, inp.a, inp.s0[0], inp.dh)
        states = [r["h"]]
    else:
        r = seq.lstm_bptt(inp.u_rounded, inp.a, inp.s0[0], inp.s0[1], inp.dh, None)
        states = [r["c"], r["h"]]
    s = [torch.from_numpy(x.astype(np.float32)).to(DEV) for x in states]
    dh = torch.from_numpy(inp.dh).to(DEV)
    gs = [dh] if cell == "gru" else [None, dh]
    kw = dict(with_lambda=True, steps_per_lane=KW[0], waves_per_block=KW[1])
    ref = pr.adjoint(cell, u, a, s0, s, gs, **kw)
    _, ut = interleaved(u)
    du_full, du = interleaved([torch.empty_like(x, dtype=torch.float32) for x in u])
    out = dict(du=du, da=torch.empty_like(ref["da"]), ds0=[torch.empty_like(x) for x in s0],
               lam=[tm_empty(*x.shape) for x in s])
    got = pr.adjoint(cell, ut, a, s0, [time_major(x) for x in s],
                     [None if g is None else time_major(g) for g in gs], out=out, **kw)
    torch.cuda.synchronize()
    for k in ("du", "ds0", "lam"):
        for g, x in zip(got[k], ref[k]):
            assert torch.equal(g, x), k
    assert torch.equal(got["da"], ref["da"])
    G = len(u)
    D = u[0].shape[1]
    for g in range(G):
        gd = du_full[:, :, g * D:(g + 1) * D].transpose(1, 2).cpu().numpy().astype(np.float64)
        assert np.abs(gd - r["du"][g]).max() <= 1e-5 * max(1.0, np.abs(r["du"][g]).max())


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_adjoint_time_major_gather_route(cell):
    """The adjoint with a base-size workspace gathers time-major steps
    directly; bitwise the result of the staged route."""
    inp = make_inputs(cell, 2, 900, 5, 4250, s0_std=0.3, f_bias=1.0, with_grad=True)
    u, a, s0 = dev_inputs(inp)
    h, _ = solve(cell, u, a, s0)
    _, ut = interleaved(u)
    st = [time_major(x) for x in h]
    gs = [None] * (len(h) - 1) + [time_major(torch.from_numpy(inp.dh).to(DEV))]

    def run(ws):
        _, du = interleaved([torch.empty_like(x, dtype=torch.float32) for x in u])
        out = dict(du=du, da=torch.empty((len(u), 5), device=DEV),
                   ds0=[torch.empty_like(x) for x in s0], lam=[tm_empty(2, 5, 900) for _ in h])
        return pr.adjoint(cell, ut, a, s0, st, gs, with_lambda=True, out=out, workspace=ws)

    staged = run(None)
    nws = pr.workspace_bytes(cell, pr.make_shape(2, 900, 5), pr.make_newton(0.0, 0),
                             adjoint=True)
    gathered = run(torch.empty(max(nws, 1), dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    for k in ("du", "ds0", "lam"):
        for x, y in zip(staged[k], gathered[k]):
            assert torch.equal(x, y), k
    assert torch.equal(staged["da"], gathered["da"])


@pytest.mark.parametrize("S", [1, 2])
@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("T,KW", [(63, (1, 1)), (1000, (0, 0)), (5003, (1, 1))])
def test_scan_time_major(S, reverse, T, KW):
    rng = np.random.default_rng(4300 + T)
    A = rng.uniform(-0.7, 0.7, (S * S, 2, 3, T)).astype(np.float32)
    b = rng.standard_normal((S, 2, 3, T)).astype(np.float32)
    x0 = rng.standard_normal((S, 2, 3)).astype(np.float32)
    At = [torch.from_numpy(x).to(DEV) for x in A]
    bt = [torch.from_numpy(x).to(DEV) for x in b]
    x0t = [torch.from_numpy(x).to(DEV) for x in x0]
    kw = dict(reverse=reverse, steps_per_lane=KW[0], waves_per_block=KW[1])
    ref = pr.scan(At, bt, x0t, **kw)
    _, tm = interleaved(At + bt)
    got = pr.scan(tm[:S * S], tm[S * S:], x0t, **kw)
    torch.cuda.synchronize()
    for g, r in zip(got, ref):
        assert g.stride()[1] == 1
        assert torch.equal(g, r)


@pytest.mark.parametrize("S", [1, 2])
def test_scan_time_major_gather_route(S):
    """The scan with a channel-major-size workspace gathers time-major steps;
    bitwise the staged result."""
    rng = np.random.default_rng(4350 + S)
    T = 3000
    A = rng.uniform(-0.7, 0.7, (S * S, 2, 3, T)).astype(np.float32)
    b = rng.standard_normal((S, 2, 3, T)).astype(np.float32)
    _, tm = interleaved([torch.from_numpy(x).to(DEV) for x in A] +
                        [torch.from_numpy(x).to(DEV) for x in b])
    kw = dict(steps_per_lane=1, waves_per_block=1)
    staged = pr.scan(tm[:S * S], tm[S * S:], None, **kw)
    nws = int(pr.load().pararnn_scan_workspace_bytes(
        S, ctypes.byref(pr.make_shape(2, T, 3)), ctypes.byref(pr.make_newton(0.0, 0, 1, 1))))
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=DEV)
    gathered = pr.scan(tm[:S * S], tm[S * S:], None, workspace=ws, **kw)
    torch.cuda.synchronize()
    for x, y in zip(staged, gathered):
        assert torch.equal(x, y)


@pytest.mark.parametrize("cell", ["gru", "lstm"])
@pytest.mark.parametrize("udt", ["f32", "bf16"])
def test_sequential_time_major(cell, udt):
    inp = make_inputs(cell, 2, 1001, 70, 4400, u_dtype=udt, s0_std=0.1, f_bias=1.0)
    u, a, s0 = dev_inputs(inp)
    ref = pr.sequential(cell, u, a, s0)
    _, ut = interleaved(u)
    got = pr.sequential(cell, ut, a, s0)
    torch.cuda.synchronize()
    for g, r in zip(got, ref):
        assert torch.equal(g, r)


@pytest.mark.parametrize("cell", ["gru", "lstm"])
@pytest.mark.parametrize("udt", [torch.float32, torch.bfloat16])
def test_autograd_time_major(cell, udt):
    """gru_time_major / lstm_time_major on a [B][T][G*D] tensor: states equal
    the per-gate solve's, gradients match the oracle's BPTT."""
    inp = make_inputs(cell, 2, 600, 5, 4500, s0_std=0.3, f_bias=1.0, with_grad=True)
    G, D, T = len(inp.u), 5, 600
    full = np.concatenate([p.transpose(0, 2, 1) for p in inp.u], axis=2)  # [B][T][G*D]
    u = torch.from_numpy(np.ascontiguousarray(full)).to(DEV).to(udt).requires_grad_(True)
    a = torch.from_numpy(inp.a).to(DEV).requires_grad_(True)
    s0 = [torch.from_numpy(x).to(DEV).requires_grad_(True) for x in inp.s0]
    dh = torch.from_numpy(inp.dh).to(DEV).transpose(1, 2)  # [B][T][D]
    if cell == "gru":
        h = pag.gru_time_major(u, a, s0[0], strict=True)
        u_seen = [p.astype(np.float64) for p in
                  np.split(u.detach().float().cpu().numpy(), G, axis=2)]
        u_seen = [x.transpose(0, 2, 1) for x in u_seen]
        ref = seq.gru_bptt(u_seen, inp.a, inp.s0[0], inp.dh)
        ref_s0 = [ref["dh0"]]
    else:
        c, h = pag.lstm_time_major(u, a, s0[0], s0[1], strict=True)
        u_seen = [x.transpose(0, 2, 1) for x in
                  np.split(u.detach().float().cpu().numpy().astype(np.float64), G, axis=2)]
        ref = seq.lstm_bptt(u_seen, inp.a, inp.s0[0], inp.s0[1], inp.dh, None)
        ref_s0 = [ref["dc0"], ref["dh0"]]
    assert tuple(h.shape) == (2, T, D)
    assert np.abs(h.detach().transpose(1, 2).cpu().numpy() - ref["h"]).max() < 1e-5
    (h * dh).sum().backward()
    gu = u.grad.float().cpu().numpy().astype(np.float64)
    # bf16 gradients are the float32 adjoint rounded once: compare at that
    # precision there, at 1e-5 relative for float32
    rel = 1e-5 if udt == torch.float32 else 2 ** -8
    for g in range(G):
        got = gu[:, :, g * D:(g + 1) * D].transpose(0, 2, 1)
        assert np.abs(got - ref["du"][g]).max() <= rel * max(1.0, np.abs(ref["du"][g]).max())
    assert np.abs(a.grad.cpu().numpy() - ref["da"]).max() <= 1e-5 * max(1.0, np.abs(ref["da"]).max())
    for x, r in zip(s0, ref_s0):
        assert np.abs(x.grad.cpu().numpy() - r).max() <= 1e-5 * max(1.0, np.abs(r).max())
