"""torch.autograd bindings of the fused solve and its adjoint.

``gru(u, a, h0)`` and ``lstm(u, a, c0, h0)`` return the converged states and
record a backward that runs the reverse-time adjoint scan
(``pararnn_adjoint``) — gradients for the projections u, the diagonal weights
a and the initial states.  Both directions run in the HIP kernels; this
module only wires them into autograd (the pages' ParaRNN framework derives
the backward pass by autodiff in its PyTorch tier; here it is the adjoint of
the converged Newton solve, the transposed block-bidiagonal system of
"Параллельность RNN?" (forpes.ru), §1.3).

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
        out = pr.adjoint("gru", [uz, ur, uc], a, [h0], [h], [gh.contiguous()])
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
        gs = [None if gc is None else gc.contiguous(), None if gh is None else gh.contiguous()]
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
