"""Pins of the CPU oracle against things other than itself.

Each test names what fixes the expected value: a library routine
(torch.nn.GRUCell / LSTMCell with diagonal recurrent weights, scipy's
lfilter), a closed form, finite differences, or the statements of
"Параллельность RNN?" (forpes.ru), section 1 (unique zero of the residual,
first piece of the forward substitution is free, associativity of the
linear recurrence, block-bidiagonal Jacobian).
"""
import os

import numpy as np
import pytest
import scipy.signal
import torch

from nonlinear_rnn_amd.inputs import make_inputs
from oracle import deer
from oracle import sequential as seq

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _chan(inp):
    """[B][D][T] planes -> deer layout [n, T, G] / [n, G] / [n, S]."""
    B = inp.u[0].shape[0]
    u = deer.from_planes(inp.u)
    a = deer.a_per_channel(inp.a, B)
    s0 = np.stack([np.asarray(p, np.float64).reshape(-1) for p in inp.s0], -1)
    return u, a, s0


def _oracle_states(inp):
    if inp.cell == "gru":
        h = seq.gru_forward(inp.u, inp.a, inp.s0[0])
        return deer.from_planes([h])
    c, h = seq.lstm_forward(inp.u, inp.a, inp.s0[0], inp.s0[1])
    return deer.from_planes([c, h])


# ------------------------------------------------ library-routine pins ----

def _torch_gru_loop(u, a, h0):
    """ParaGRU through torch.nn.GRUCell (float64).  torch's cell is
    r = sig(W_ir x + W_hr h), z_t = sig(W_iz x + W_hz h),
    n = tanh(W_in x + r * (W_hn h)), h' = (1 - z_t) n + z_t h.
    With x = [u_r, -u_z, u_c], W_ih = I, W_hh = [diag(a_r); diag(-a_z);
    diag(a_c)] and zero biases, z_t = 1 - z and n = c, i.e. exactly
    h' = (1 - z) h + z c."""
    uz, ur, uc = u          # torch [B, D, T] float64 leaves
    az, ar, ac = a          # [D]
    B, D, T = uz.shape
    cell = torch.nn.GRUCell(3 * D, D, bias=False).double()
    w_ih = torch.eye(3 * D, dtype=torch.float64)
    w_hh = torch.cat([torch.diag(ar), torch.diag(-az), torch.diag(ac)], 0)
    h = h0
    hs = []
    for t in range(T):
        x = torch.cat([ur[:, :, t], -uz[:, :, t], uc[:, :, t]], dim=1)
        h = torch.func.functional_call(cell, {"weight_ih": w_ih, "weight_hh": w_hh}, (x, h))
        hs.append(h)
    return torch.stack(hs, dim=2)


def _torch_lstm_loop(u, a, c0, h0):
    """ParaLSTM through torch.nn.LSTMCell (float64), gate order (i, f, g, o):
    x = [u_i, u_f, u_g, u_o], W_ih = I, W_hh = [diag(a_i); diag(a_f);
    diag(a_g); diag(a_o)], zero biases."""
    B, D, T = u[0].shape
    cell = torch.nn.LSTMCell(4 * D, D, bias=False).double()
    w_ih = torch.eye(4 * D, dtype=torch.float64)
    w_hh = torch.cat([torch.diag(x) for x in a], 0)
    h, c = h0, c0
    hs, cs = [], []
    for t in range(T):
        x = torch.cat([p[:, :, t] for p in u], dim=1)
        h, c = torch.func.functional_call(cell, {"weight_ih": w_ih, "weight_hh": w_hh},
                                          (x, (h, c)))
        hs.append(h)
        cs.append(c)
    return torch.stack(cs, 2), torch.stack(hs, 2)


def _t(x, grad=False):
    return torch.tensor(np.asarray(x, np.float64), dtype=torch.float64, requires_grad=grad)


@pytest.mark.parametrize("B,T,D,seed", [(2, 37, 5, 11), (1, 200, 3, 12)])
def test_gru_forward_matches_torch_grucell(B, T, D, seed):
    inp = make_inputs("gru", B, T, D, seed, s0_std=0.5, a_scale=2.0)
    h = seq.gru_forward(inp.u, inp.a, inp.s0[0])
    ref = _torch_gru_loop([_t(p) for p in inp.u], [_t(x) for x in inp.a],
                          _t(inp.s0[0])).numpy()
    np.testing.assert_allclose(h, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("B,T,D,seed", [(2, 41, 4, 13), (1, 150, 3, 14)])
def test_lstm_forward_matches_torch_lstmcell(B, T, D, seed):
    inp = make_inputs("lstm", B, T, D, seed, s0_std=0.5, f_bias=1.0, a_scale=2.0)
    c, h = seq.lstm_forward(inp.u, inp.a, inp.s0[0], inp.s0[1])
    rc, rh = _torch_lstm_loop([_t(p) for p in inp.u], [_t(x) for x in inp.a],
                              _t(inp.s0[0]), _t(inp.s0[1]))
    np.testing.assert_allclose(c, rc.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(h, rh.detach().numpy(), rtol=0, atol=1e-12)


def test_gru_bptt_matches_torch_autograd():
    inp = make_inputs("gru", 2, 29, 4, 21, s0_std=0.5, a_scale=1.5, with_grad=True)
    out = seq.gru_bptt(inp.u, inp.a, inp.s0[0], inp.dh)
    u = [_t(p, True) for p in inp.u]
    a = [_t(x, True) for x in inp.a]
    h0 = _t(inp.s0[0], True)
    hs = _torch_gru_loop(u, a, h0)
    L = (hs * _t(inp.dh)).sum()
    L.backward()
    np.testing.assert_allclose(out["h"], hs.detach().numpy(), atol=1e-12, rtol=0)
    for k in range(3):
        np.testing.assert_allclose(out["du"][k], u[k].grad.numpy(), atol=1e-11, rtol=0)
        np.testing.assert_allclose(out["da"][k], a[k].grad.numpy(), atol=1e-10, rtol=0)
    np.testing.assert_allclose(out["dh0"], h0.grad.numpy(), atol=1e-11, rtol=0)


@pytest.mark.parametrize("with_dc", [False, True])
def test_lstm_bptt_matches_torch_autograd(with_dc):
    inp = make_inputs("lstm", 2, 31, 3, 22, s0_std=0.5, f_bias=1.0, a_scale=1.5,
                      with_grad=True)
    dc = (np.random.default_rng(5).standard_normal(inp.dh.shape).astype(np.float32)
          if with_dc else None)
    out = seq.lstm_bptt(inp.u, inp.a, inp.s0[0], inp.s0[1], inp.dh, dc)
    u = [_t(p, True) for p in inp.u]
    a = [_t(x, True) for x in inp.a]
    c0, h0 = _t(inp.s0[0], True), _t(inp.s0[1], True)
    cs, hs = _torch_lstm_loop(u, a, c0, h0)
    L = (hs * _t(inp.dh)).sum()
    if with_dc:
        L = L + (cs * _t(dc)).sum()
    L.backward()
    for k in range(4):
        np.testing.assert_allclose(out["du"][k], u[k].grad.numpy(), atol=1e-11, rtol=0)
        np.testing.assert_allclose(out["da"][k], a[k].grad.numpy(), atol=1e-10, rtol=0)
    np.testing.assert_allclose(out["dc0"], c0.grad.numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(out["dh0"], h0.grad.numpy(), atol=1e-11, rtol=0)


def test_gru_linear_special_case_is_lfilter():
    """a = 0 and u_z constant in t: h_t = (1 - z) h_{t-1} + z tanh(u_c,t) is a
    first-order IIR filter, i.e. scipy.signal.lfilter([z], [1, -(1 - z)])."""
    T = 300
    inp = make_inputs("gru", 1, T, 3, 31, s0_std=1.0)
    inp.a[:] = 0.0
    uz_const = np.array([-0.7, 0.2, 1.9], np.float32)
    inp.u[0][0] = uz_const[:, None]
    h = seq.gru_forward(inp.u, inp.a, inp.s0[0])
    for d in range(3):
        z = 1.0 / (1.0 + np.exp(-np.float64(uz_const[d])))
        x = np.tanh(inp.u[2][0, d].astype(np.float64))
        h0 = np.float64(inp.s0[0][0, d])
        y, _ = scipy.signal.lfilter([z], [1.0, -(1.0 - z)], x, zi=[(1.0 - z) * h0])
        np.testing.assert_allclose(h[0, d], y, rtol=0, atol=1e-13)


# ---------------------------------------------------------- golden files ----

def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([float(x) for x in line.split()])
    return np.array(rows)


def test_golden_gru_halving():
    """tests/golden/gru_halving.txt: a = 0, u_z = u_c = 0 gives z = 1/2,
    c = 0, so h_t = h_0 / 2^t (closed form written out in the file)."""
    g = _read_golden("gru_halving.txt")
    T = g.shape[0]
    inp = make_inputs("gru", 1, T, 1, 0)
    inp.a[:] = 0
    inp.u[0][:] = 0
    inp.u[2][:] = 0
    inp.u[1][:] = 3.0  # r is irrelevant once a_c = 0
    inp.s0[0][:] = 1.0
    h = seq.gru_forward(inp.u, inp.a, inp.s0[0])
    np.testing.assert_allclose(h[0, 0], g[:, 1], rtol=0, atol=1e-15)
    # and the DEER solve reaches it
    u, a, s0 = _chan(inp)
    s, info = deer.newton("gru", u, a, s0, tol=1e-14, max_iters=T)
    np.testing.assert_allclose(s[0, :, 0], g[:, 1], rtol=0, atol=1e-15)


def test_golden_lstm_halving():
    """tests/golden/lstm_halving.txt: a = 0 and all projections 0 give
    i = f = o = 1/2, g = 0: c_t = c_{t-1} / 2, h_t = tanh(c_t) / 2."""
    g = _read_golden("lstm_halving.txt")
    T = g.shape[0]
    inp = make_inputs("lstm", 1, T, 1, 0)
    inp.a[:] = 0
    for p in inp.u:
        p[:] = 0
    inp.s0[0][:] = 1.0
    inp.s0[1][:] = 0.25
    c, h = seq.lstm_forward(inp.u, inp.a, inp.s0[0], inp.s0[1])
    np.testing.assert_allclose(c[0, 0], g[:, 1], rtol=0, atol=1e-15)
    np.testing.assert_allclose(h[0, 0], 0.5 * np.tanh(g[:, 1]), rtol=0, atol=1e-15)


# --------------------------------------------------- pins from the pages ----

@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_oracle_trajectory_is_zero_of_residual(cell):
    """§1.1: the sequential trajectory is the zero of r."""
    inp = make_inputs(cell, 2, 257, 5, 41, s0_std=0.3, f_bias=1.0)
    u, a, s0 = _chan(inp)
    s = _oracle_states(inp)
    r = deer.residual(deer.CELLS[cell], s, s0, u, a)
    assert np.abs(r).max() < 1e-14


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_local_jacobians_match_finite_differences(cell):
    C = deer.CELLS[cell]
    rng = np.random.default_rng(51)
    n = 40
    s = rng.standard_normal((n, C.S))
    u = rng.standard_normal((n, C.G)) * 1.5
    a = rng.uniform(-2, 2, (n, C.G))
    J = C.jac(s, u, a)
    eps = 1e-6
    for j in range(C.S):
        e = np.zeros(C.S)
        e[j] = eps
        fd = (C.step(s + e, u, a) - C.step(s - e, u, a)) / (2 * eps)
        np.testing.assert_allclose(J[:, :, j], fd, rtol=0, atol=1e-8)


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_dense_residual_jacobian_is_block_bidiagonal_fd(cell):
    """§1.3: dr/ds has identity diagonal blocks, -df/ds(s_{t-1}) below the
    diagonal and zeros elsewhere; checked against a brute-force central
    difference of the whole residual vector."""
    C = deer.CELLS[cell]
    inp = make_inputs(cell, 1, 6, 2, 52, s0_std=0.5, f_bias=1.0)
    u, a, s0 = _chan(inp)
    n, T = u.shape[0], u.shape[1]
    s = np.random.default_rng(53).standard_normal((n, T, C.S))
    J = deer.residual_jacobian_dense(C, s, s0, u, a)
    eps = 1e-6
    fd = np.zeros_like(J)
    for k in range(T * C.S):
        e = np.zeros(T * C.S)
        e[k] = eps
        e = e.reshape(T, C.S)
        rp = deer.residual(C, s + e, s0, u, a).reshape(n, -1)
        rm = deer.residual(C, s - e, s0, u, a).reshape(n, -1)
        fd[:, :, k] = (rp - rm) / (2 * eps)
    np.testing.assert_allclose(J, fd, rtol=0, atol=1e-8)


@pytest.mark.parametrize("S", [1, 2])
@pytest.mark.parametrize("T", [1, 2, 3, 5, 8, 17, 64])
def test_scans_agree_with_brute_force(S, T):
    """§1.3 levels 1 and 2: forward substitution, the pairwise tree and the
    closed-form sum of products all solve the same block-bidiagonal system,
    which a dense solve checks by brute force."""
    rng = np.random.default_rng(61 + T)
    n = 3
    A = rng.uniform(-1.2, 1.2, (n, T, S, S))
    b = rng.standard_normal((n, T, S))
    x1 = deer.solve_forward_substitution(A, b)
    x2 = deer.solve_tree_scan(A, b)
    x3 = deer.solve_closed_form(A, b)
    M = np.zeros((n, T * S, T * S))
    for t in range(T):
        M[:, t * S:(t + 1) * S, t * S:(t + 1) * S] = np.eye(S)
        if t:
            M[:, t * S:(t + 1) * S, (t - 1) * S:t * S] = -A[:, t]
    x4 = np.linalg.solve(M, b.reshape(n, -1)[..., None])[..., 0].reshape(n, T, S)
    for x in (x1, x2, x3):
        np.testing.assert_allclose(x, x4, rtol=0, atol=1e-10)


def test_linear_gru_one_newton_step_exact():
    """a = 0 makes f affine in h, so the linearisation is exact and a single
    Newton update from any start lands on the trajectory."""
    inp = make_inputs("gru", 2, 300, 4, 71, s0_std=0.5)
    inp.a[:] = 0
    u, a, s0 = _chan(inp)
    start = np.random.default_rng(72).standard_normal((u.shape[0], 300, 1)) * 3
    s, info = deer.newton("gru", u, a, s0, tol=0.0, max_iters=1, s_init=start)
    np.testing.assert_allclose(s, _oracle_states(inp), rtol=0, atol=1e-13)
    s, info = deer.newton("gru", u, a, s0, tol=1e-12, max_iters=5, s_init=start)
    assert (info["iters"] == 1).all() and info["converged"].all()


def test_linear_lstm_exact_after_two_steps():
    """a = 0: c' = f c + i g is affine in c (gates do not see the state), so
    c is exact after one update; h = o tanh(c) then needs a second one."""
    inp = make_inputs("lstm", 2, 200, 3, 73, s0_std=0.5, f_bias=1.0)
    inp.a[:] = 0
    u, a, s0 = _chan(inp)
    ref = _oracle_states(inp)
    s1, _ = deer.newton("lstm", u, a, s0, tol=0.0, max_iters=1)
    np.testing.assert_allclose(s1[..., 0], ref[..., 0], rtol=0, atol=1e-13)
    assert np.abs(s1[..., 1] - ref[..., 1]).max() > 1e-3
    s2, _ = deer.newton("lstm", u, a, s0, tol=0.0, max_iters=2)
    np.testing.assert_allclose(s2, ref, rtol=0, atol=1e-13)


@pytest.mark.parametrize("cell", ["gru", "lstm"])
@pytest.mark.parametrize("solver", ["serial", "tree"])
def test_prefix_exactness_stiff(cell, solver):
    """§1.3 level 1: ds_1 = -r_1 makes s_1 exact after one update, and by
    induction s_1..s_k are exact after k updates; so Newton from zero needs
    at most T updates even for a stiff cell (a ~ U(-4, 4))."""
    T = 24
    inp = make_inputs(cell, 1, T, 6, 81, f_bias=1.0, a_scale=4.0, u_scale=2.0)
    u, a, s0 = _chan(inp)
    ref = _oracle_states(inp)
    _, info = deer.newton(cell, u, a, s0, tol=0.0, max_iters=T, solver=solver,
                          history=True)
    for k, s in enumerate(info["history"]):
        if k:
            np.testing.assert_allclose(s[:, :k], ref[:, :k], rtol=0, atol=1e-12)
    s, info = deer.newton(cell, u, a, s0, tol=1e-11, max_iters=T, solver=solver)
    assert info["converged"].all() and (info["iters"] <= T).all()


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_t1_one_update_exact(cell):
    inp = make_inputs(cell, 3, 1, 4, 91, s0_std=1.0, f_bias=1.0)
    u, a, s0 = _chan(inp)
    start = np.random.default_rng(92).standard_normal((u.shape[0], 1, deer.CELLS[cell].S))
    s, _ = deer.newton(cell, u, a, s0, tol=0.0, max_iters=1, s_init=start)
    np.testing.assert_allclose(s, _oracle_states(inp), rtol=0, atol=1e-14)


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_newton_converges_to_oracle(cell):
    inp = make_inputs(cell, 2, 512, 8, 101, s0_std=0.1, f_bias=1.0)
    u, a, s0 = _chan(inp)
    s, info = deer.newton(cell, u, a, s0, tol=1e-12, max_iters=20)
    assert info["converged"].all()
    np.testing.assert_allclose(s, _oracle_states(inp), rtol=0, atol=1e-11)


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_bptt_adjoint_solves_transposed_system(cell):
    """The adjoint of the converged solve solves J(s*)^T lam = dL/ds for the
    §1.3 block-bidiagonal J; the BPTT oracle's total dL/ds_t must match a
    dense solve of that transposed system."""
    inp = make_inputs(cell, 1, 9, 3, 111, s0_std=0.5, f_bias=1.0, with_grad=True)
    u, a, s0 = _chan(inp)
    s = _oracle_states(inp)
    n, T = s.shape[:2]
    if cell == "gru":
        out = seq.gru_bptt(inp.u, inp.a, inp.s0[0], inp.dh)
        g = deer.from_planes([inp.dh])
        lam = deer.from_planes([out["lam"]])
    else:
        out = seq.lstm_bptt(inp.u, inp.a, inp.s0[0], inp.s0[1], inp.dh)
        g = np.stack([np.zeros((n, T)), deer.from_planes([inp.dh])[..., 0]], -1)
        lam = deer.from_planes([out["lam_c"], out["lam_h"]])
    ref = deer.adjoint_dense(deer.CELLS[cell], s, s0, u, a, g)
    np.testing.assert_allclose(lam, ref, rtol=0, atol=1e-11)


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_bptt_matches_finite_differences(cell):
    """Central differences of L = sum <dh, h> w.r.t. a few entries of u, a and
    the initial state; perturbations are powers of two so they are exact in
    float32."""
    inp = make_inputs(cell, 1, 16, 2, 121, s0_std=0.5, f_bias=1.0, with_grad=True)
    eps = np.float32(2.0 ** -10)

    def loss(i):
        if cell == "gru":
            h = seq.gru_forward(i.u, i.a, i.s0[0])
        else:
            _, h = seq.lstm_forward(i.u, i.a, i.s0[0], i.s0[1])
        return float((h * i.dh.astype(np.float64)).sum())

    if cell == "gru":
        out = seq.gru_bptt(inp.u, inp.a, inp.s0[0], inp.dh)
        ds0 = [out["dh0"]]
    else:
        out = seq.lstm_bptt(inp.u, inp.a, inp.s0[0], inp.s0[1], inp.dh)
        ds0 = [out["dc0"], out["dh0"]]

    def fd(arr, idx):
        old = arr[idx]
        arr[idx] = old + eps
        lp = loss(inp)
        arr[idx] = old - eps
        lm = loss(inp)
        arr[idx] = old
        return (lp - lm) / (2 * float(eps))

    for g in range(len(inp.u)):
        for idx in [(0, 0, 0), (0, 1, 7), (0, 0, 15)]:
            np.testing.assert_allclose(fd(inp.u[g], idx), out["du"][g][idx],
                                       rtol=2e-5, atol=2e-6)
        for d in range(2):
            np.testing.assert_allclose(fd(inp.a, (g, d)), out["da"][g, d],
                                       rtol=2e-5, atol=2e-6)
    for k, plane in enumerate(inp.s0):
        np.testing.assert_allclose(fd(plane, (0, 1)), ds0[k][0, 1], rtol=2e-5, atol=2e-6)


@pytest.mark.parametrize("S", [1, 2])
@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("T", [1, 2, 7, 33])
def test_linear_recurrence_is_dense_solve(S, reverse, T):
    """x_t - A_t x_{t-1} = b_t (x_0 given) as one block-bidiagonal system,
    solved densely; the reverse recurrence is the same system with time
    flipped."""
    rng = np.random.default_rng(131 + T)
    n = 3
    A = rng.uniform(-1.1, 1.1, (n, T, S, S))
    b = rng.standard_normal((n, T, S))
    x0 = rng.standard_normal((n, S))
    x = deer.linear_recurrence(A, b, x0, reverse=reverse)
    At, bt = (A[:, ::-1], b[:, ::-1]) if reverse else (A, b)
    M = np.zeros((n, T * S, T * S))
    rhs = bt.copy()
    rhs[:, 0] += np.einsum("nij,nj->ni", At[:, 0], x0)
    for t in range(T):
        M[:, t * S:(t + 1) * S, t * S:(t + 1) * S] = np.eye(S)
        if t:
            M[:, t * S:(t + 1) * S, (t - 1) * S:t * S] = -At[:, t]
    ref = np.linalg.solve(M, rhs.reshape(n, -1)[..., None])[..., 0].reshape(n, T, S)
    if reverse:
        ref = ref[:, ::-1]
    np.testing.assert_allclose(x, ref, rtol=0, atol=1e-10)
    if not reverse:
        np.testing.assert_allclose(deer.linear_recurrence(A, b), deer.solve_forward_substitution(A, b),
                                   rtol=0, atol=1e-12)


# ------------------------------------------------------------ projection ----

def test_projection_matches_brute_force_loops():
    from oracle import projection
    rng = np.random.default_rng(71)
    B, T, I, M = 2, 5, 4, 3
    x = rng.standard_normal((B, T, I))
    W = rng.standard_normal((M, I))
    bias = rng.standard_normal(M)
    u = projection.project(x, W, bias)
    for b in range(B):
        for m in range(M):
            for t in range(T):
                acc = bias[m]
                for k in range(I):
                    acc += W[m, k] * x[b, t, k]
                assert abs(u[b, m, t] - acc) < 1e-12


def test_projection_identity_weight_is_the_transpose():
    from oracle import projection
    rng = np.random.default_rng(72)
    x = rng.standard_normal((3, 7, 6))
    u = projection.project(x, np.eye(6))
    assert u.shape == (3, 6, 7)
    assert np.array_equal(u, np.transpose(x, (0, 2, 1)))


def test_projection_bias_only_and_abs_scale():
    from oracle import projection
    bias = np.array([1.5, -2.0])
    u = projection.project(np.zeros((1, 4, 3)), np.ones((2, 3)), bias)
    assert np.array_equal(u, np.broadcast_to(bias[None, :, None], (1, 2, 4)))
    x = np.array([[[1.0, -2.0]]])
    W = np.array([[3.0, 4.0]])
    assert projection.project(x, W)[0, 0, 0] == -5.0
    assert projection.project_abs(x, W, np.array([-1.0]))[0, 0, 0] == 12.0
