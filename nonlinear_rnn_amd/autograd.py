"""torch.autograd bindings of the fused solve and its adjoint.

``gru(u, a, h0)`` and ``lstm(u, a, c0, h0)`` return the converged states and
record a backward that runs the reverse-time adjoint scan
(``pararnn_adjoint``) — gradients for the projections u, the diagonal weights
a and the initial states.  Both directions run in the HIP kernels; this
module only wires them into autograd (the pages' ParaRNN framework derives
the backward pass by autodiff in its PyTorch tier; here it is the adjoint of
the converged Newton solve, the transposed block-bidiagonal system of
"Параллельность RNN?" (forpes.ru), §1.3).

Two layouts: ``gru``/``lstm`` take one [B][D][T]-indexed tensor per gate
(any strides; channel-major is the fast layout), ``gru_time_major`` /
``lstm_time_major`` take the [B][T][G*D] tensor a ``torch.nn.Linear`` over
[B][T][I] inputs produces and return [B][T][D] states; its gate planes are
passed to the kernels as strided views (no transpose copy), and the
gradient for u comes back as one [B][T][G*D] tensor written by the adjoint.

Non-convergence is not an error in the solve; pass ``strict=True`` to raise
when a solve stops at the iteration cap without reaching the tolerance (this
reads the device info record, i.e. synchronises).
"""
import torch

from . import pararnn as pr


def _check(info_t, strict):
    if strict:
        info = pr.read_info(info_t)
        if not info["converged"]:
            raise RuntimeError(f"ParaRNN Newton solve did not converge: {info}")


def _grad_like(g, ref):
    return g if g.dtype == ref.dtype else g.to(ref.dtype)


def _strided_like(g, ref):
    """`g` with the strides of `ref` (the adjoint reads upstream gradients in
    the layout of the states)."""
    if g.stride() == ref.stride():
        return g
    out = torch.empty_strided(ref.shape, ref.stride(), dtype=g.dtype, device=g.device)
    out.copy_(g)
    return out


def _gate_planes(u, G):
    """Gate planes of a time-major [B][T][G*D] tensor as [B][D][T]-indexed
    views (no copy)."""
    if u.dim() != 3 or u.shape[2] % G != 0:
        raise ValueError(f"u must be [B][T][{G}*D]")
    D = u.shape[2] // G
    return [u[:, :, g * D:(g + 1) * D].transpose(1, 2) for g in range(G)]


def _time_major_adjoint(cell, u, a, s0, s, gs):
    """Adjoint for time-major tensors: u [B][T][G*D], s and gs [B][T][D]
    (gs entries may be None).  Returns (du [B][T][G*D], da, ds0 list)."""
    G = pr.N_GATES[pr.CELLS[cell]]
    B, T, GD = u.shape
    D = GD // G
    du = torch.empty((B, T, GD), dtype=torch.float32, device=u.device)
    da = torch.empty((G, D), dtype=torch.float32, device=u.device)
    ds0 = [torch.empty((B, D), dtype=torch.float32, device=u.device) for _ in s0]
    gsv = [None if g is None else g.contiguous().transpose(1, 2) for g in gs]
    pr.adjoint(cell, _gate_planes(u, G), a, s0, [x.transpose(1, 2) for x in s], gsv,
               out=dict(du=_gate_planes(du, G), da=da, ds0=ds0, lam=None))
    return du, da, ds0


class _GruSolve(torch.autograd.Function):
    @staticmethod
    def forward(ctx, uz, ur, uc, a, h0, tol, max_iters, strict):
        u = [uz, ur, uc]
        h, info_t = pr.solve_gru(u, a, h0, tol=tol, max_iters=max_iters, info=strict)
        _check(info_t, strict)
        ctx.save_for_backward(uz, ur, uc, a, h0, h)
        return h

    @staticmethod
    def backward(ctx, gh):
        uz, ur, uc, a, h0, h = ctx.saved_tensors
        out = pr.adjoint("gru", [uz, ur, uc], a, [h0], [h], [_strided_like(gh, h)])
        du = out["du"]
        return (_grad_like(du[0], uz), _grad_like(du[1], ur), _grad_like(du[2], uc),
                out["da"], out["ds0"][0], None, None, None)


class _LstmSolve(torch.autograd.Function):
    @staticmethod
    def forward(ctx, ui, uf, ug, uo, a, c0, h0, tol, max_iters, strict):
        u = [ui, uf, ug, uo]
        (c, h), info_t = pr.solve_lstm(u, a, c0, h0, tol=tol, max_iters=max_iters, info=strict)
        _check(info_t, strict)
        ctx.save_for_backward(ui, uf, ug, uo, a, c0, h0, c, h)
        return c, h

    @staticmethod
    def backward(ctx, gc, gh):
        ui, uf, ug, uo, a, c0, h0, c, h = ctx.saved_tensors
        gs = [None if gc is None else _strided_like(gc, c),
              None if gh is None else _strided_like(gh, h)]
        out = pr.adjoint("lstm", [ui, uf, ug, uo], a, [c0, h0], [c, h], gs)
        du = out["du"]
        return (_grad_like(du[0], ui), _grad_like(du[1], uf), _grad_like(du[2], ug),
                _grad_like(du[3], uo), out["da"], out["ds0"][0], out["ds0"][1],
                None, None, None)


def gru(u, a, h0, *, tol=1e-6, max_iters=20, strict=False):
    """Differentiable ParaGRU solve.  u = (u_z, u_r, u_c) [B][D][T] device
    tensors; a [3][D]; h0 [B][D].  Returns h [B][D][T]."""
    uz, ur, uc = u
    return _GruSolve.apply(uz, ur, uc, a, h0, tol, max_iters, strict)


def lstm(u, a, c0, h0, *, tol=1e-6, max_iters=20, strict=False):
    """Differentiable ParaLSTM solve.  u = (u_i, u_f, u_g, u_o); a [4][D];
    c0, h0 [B][D].  Returns (c, h)."""
    ui, uf, ug, uo = u
    return _LstmSolve.apply(ui, uf, ug, uo, a, c0, h0, tol, max_iters, strict)


class _GruTimeMajor(torch.autograd.Function):
    @staticmethod
    def forward(ctx, u, a, h0, tol, max_iters, strict):
        B, T, _ = u.shape
        h = torch.empty((B, T, a.shape[1]), dtype=torch.float32, device=u.device)
        _, info_t = pr.solve_gru(_gate_planes(u, 3), a, h0, out=h.transpose(1, 2), tol=tol,
                                 max_iters=max_iters, info=strict)
        _check(info_t, strict)
        ctx.save_for_backward(u, a, h0, h)
        return h

    @staticmethod
    def backward(ctx, gh):
        u, a, h0, h = ctx.saved_tensors
        du, da, ds0 = _time_major_adjoint("gru", u, a, [h0], [h], [gh])
        return _grad_like(du, u), da, ds0[0], None, None, None


class _LstmTimeMajor(torch.autograd.Function):
    @staticmethod
    def forward(ctx, u, a, c0, h0, tol, max_iters, strict):
        B, T, _ = u.shape
        D = a.shape[1]
        c = torch.empty((B, T, D), dtype=torch.float32, device=u.device)
        h = torch.empty((B, T, D), dtype=torch.float32, device=u.device)
        _, info_t = pr.solve_lstm(_gate_planes(u, 4), a, c0, h0,
                                  out=[c.transpose(1, 2), h.transpose(1, 2)], tol=tol,
                                  max_iters=max_iters, info=strict)
        _check(info_t, strict)
        ctx.save_for_backward(u, a, c0, h0, c, h)
        return c, h

    @staticmethod
    def backward(ctx, gc, gh):
        u, a, c0, h0, c, h = ctx.saved_tensors
        du, da, ds0 = _time_major_adjoint("lstm", u, a, [c0, h0], [c, h], [gc, gh])
        return _grad_like(du, u), da, ds0[0], ds0[1], None, None, None


def gru_time_major(u, a, h0, *, tol=1e-6, max_iters=20, strict=False):
    """Differentiable ParaGRU solve on time-major tensors: u [B][T][3*D]
    (gate blocks z, r, c along the last dimension, float32 or bfloat16),
    a [3][D], h0 [B][D].  Returns h [B][T][D]."""
    return _GruTimeMajor.apply(u, a, h0, tol, max_iters, strict)


def lstm_time_major(u, a, c0, h0, *, tol=1e-6, max_iters=20, strict=False):
    """Differentiable ParaLSTM solve on time-major tensors: u [B][T][4*D]
    (gate blocks i, f, g, o), a [4][D], c0, h0 [B][D].  Returns (c, h), each
    [B][T][D]."""
    return _LstmTimeMajor.apply(u, a, c0, h0, tol, max_iters, strict)
