"""GPU parity of the adjoint (reverse scan with transposed Jacobians) against
back-propagation through time in the fp64 oracle.

The device adjoint is fed the oracle's trajectory rounded to float32, so
the comparison isolates the backward pass.  Tolerance per gradient tensor:
1e-5 * max(1, max|reference|).
"""
import numpy as np
import pytest
import torch

from nonlinear_rnn_amd import pararnn as pr
from nonlinear_rnn_amd.inputs import make_inputs
from oracle import sequential as seq
from tests.gpu_util import DEV, dev_inputs

pytestmark = pytest.mark.gpu


def grad_close(got, ref, rel=1e-5):
    got = np.asarray(got, np.float64)
    scale = max(1.0, float(np.abs(ref).max()) if ref.size else 1.0)
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    assert err <= rel * scale, (err, scale)


def bptt(inp, dc=None):
    if inp.cell == "gru":
        r = seq.gru_bptt(inp.u_rounded, inp.a, inp.s0[0], inp.dh)
        return r, [r["h"]], [r["dh0"]], [r["lam"]]
    r = seq.lstm_bptt(inp.u_rounded, inp.a, inp.s0[0], inp.s0[1], inp.dh, dc)
    return r, [r["c"], r["h"]], [r["dc0"], r["dh0"]], [r["lam_c"], r["lam_h"]]


def run_adjoint(inp, states, dc=None, KW=(0, 0)):
    u, a, s0 = dev_inputs(inp)
    s = [torch.from_numpy(x.astype(np.float32)).to(DEV) for x in states]
    dh = torch.from_numpy(inp.dh).to(DEV)
    if inp.cell == "gru":
        gs = [dh]
    else:
        gs = [None if dc is None else torch.from_numpy(dc).to(DEV), dh]
    out = pr.adjoint(inp.cell, u, a, s0, s, gs, with_lambda=True, steps_per_lane=KW[0],
                     waves_per_block=KW[1])
    torch.cuda.synchronize()
    return {k: (None if v is None else
                ([x.cpu().numpy() for x in v] if isinstance(v, list) else v.cpu().numpy()))
            for k, v in out.items()}


@pytest.mark.parametrize("cell", ["gru", "lstm"])
@pytest.mark.parametrize("T,KW", [(1, (0, 0)), (63, (1, 1)), (200, (0, 0)), (1000, (1, 1)),
                                  (1000, (2, 2)), (2049, (8, 4)), (4100, (0, 0)),
                                  (777, (4, 2)), (3000, (16, 1))])
def test_adjoint_parity(cell, T, KW):
    inp = make_inputs(cell, 2, T, 3, 500 + T, s0_std=0.3, f_bias=1.0, with_grad=True)
    ref, states, ds0, lam = bptt(inp)
    out = run_adjoint(inp, states, KW=KW)
    for g in range(len(inp.u)):
        grad_close(out["du"][g], ref["du"][g])
    grad_close(out["da"], ref["da"])
    for c in range(len(states)):
        grad_close(out["ds0"][c], ds0[c])
        grad_close(out["lam"][c], lam[c])


@pytest.mark.parametrize("KW", [(0, 0), (1, 1)])
def test_lstm_adjoint_with_cell_gradient(KW):
    inp = make_inputs("lstm", 2, 900, 4, 601, s0_std=0.3, f_bias=1.0, with_grad=True)
    dc = np.random.default_rng(602).standard_normal(inp.dh.shape).astype(np.float32)
    ref, states, ds0, lam = bptt(inp, dc)
    out = run_adjoint(inp, states, dc=dc, KW=KW)
    for g in range(4):
        grad_close(out["du"][g], ref["du"][g])
    grad_close(out["da"], ref["da"])
    for c in range(2):
        grad_close(out["ds0"][c], ds0[c])
        grad_close(out["lam"][c], lam[c])


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_adjoint_bf16_inputs(cell):
    inp = make_inputs(cell, 2, 1000, 3, 611, u_dtype="bf16", f_bias=1.0, with_grad=True)
    ref, states, ds0, lam = bptt(inp)
    out = run_adjoint(inp, states)
    for g in range(len(inp.u)):
        grad_close(out["du"][g], ref["du"][g])
    grad_close(out["da"], ref["da"])


def test_adjoint_deterministic():
    inp = make_inputs("lstm", 4, 3000, 8, 621, f_bias=1.0, with_grad=True)
    _, states, _, _ = bptt(inp)
    a = run_adjoint(inp, states, KW=(2, 2))
    b = run_adjoint(inp, states, KW=(2, 2))
    for k in ("du", "ds0", "lam"):
        for x, y in zip(a[k], b[k]):
            assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    assert np.array_equal(a["da"].view(np.uint32), b["da"].view(np.uint32))


def test_adjoint_empty_time():
    inp = make_inputs("gru", 2, 0, 3, 1, with_grad=True)
    u, a, s0 = dev_inputs(inp)
    s = [torch.empty((2, 3, 0), device=DEV)]
    gs = [torch.empty((2, 3, 0), device=DEV)]
    out = pr.adjoint("gru", u, a, s0, s, gs)
    torch.cuda.synchronize()
    assert float(out["da"].abs().max()) == 0.0
    assert float(out["ds0"][0].abs().max()) == 0.0


def test_adjoint_writes_into_given_buffers():
    """out= reuses the buffers of an earlier call (no allocation) and gives
    the same result bit for bit; buffers of the wrong shape are refused."""
    inp = make_inputs("lstm", 2, 700, 3, 631, f_bias=1.0, with_grad=True)
    _, states, _, _ = bptt(inp)
    u, a, s0 = dev_inputs(inp)
    s = [torch.from_numpy(x.astype(np.float32)).to(DEV) for x in states]
    gs = [None, torch.from_numpy(inp.dh).to(DEV)]
    first = pr.adjoint("lstm", u, a, s0, s, gs, with_lambda=True)
    ref = {k: [x.clone() for x in v] if isinstance(v, list) else v.clone()
           for k, v in first.items()}
    for v in first["du"] + first["ds0"] + first["lam"] + [first["da"]]:
        v.fill_(7.0)
    again = pr.adjoint("lstm", u, a, s0, s, gs, with_lambda=True, out=first)
    torch.cuda.synchronize()
    assert again["du"][0].data_ptr() == first["du"][0].data_ptr()
    for k in ("du", "ds0", "lam"):
        for x, y in zip(again[k], ref[k]):
            assert torch.equal(x, y)
    assert torch.equal(again["da"], ref["da"])
    bad = dict(first, da=torch.empty((3, 3), device=DEV))
    with pytest.raises(ValueError):
        pr.adjoint("lstm", u, a, s0, s, gs, out=bad)
