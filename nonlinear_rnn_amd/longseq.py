"""Long-sequence memory policy: chunked solves and checkpointed training.

Training keeps every hidden state of the sequence for the Newton iterations
and for the backward pass, which for very long sequences dominates memory
("ParaRNN：解锁非线性RNN并行训练的革命性框架", zhichai.net, section
"性能对比：与Transformer和Mamba2的较量", item "长序列处理").  Two policies, both running every step in the HIP kernels of
``pararnn``; this module only orders the calls:

* ``solve_chunked`` — the sequence is cut into time chunks solved one after
  another, chunk k starting from the last state of chunk k-1.  The converged
  trajectory is the unique zero of the residual ("Параллельность RNN?",
  forpes.ru, §1.1), so each chunk's solve reaches the exact trajectory of its
  span from the exact boundary state; the result equals the one-piece solve
  within the stopping tolerance.  Only one chunk's projections need to be
  resident if the caller streams them in.

* ``gru_checkpointed`` / ``lstm_checkpointed`` — differentiable solves that
  keep only the chunk-boundary states for the backward pass (S·B·D floats
  per chunk instead of S·B·D·T).  The backward walks the chunks from last to
  first: it re-solves the chunk from its boundary state, then runs the
  adjoint scan over the chunk with the gradient that flows into the chunk's
  last state from the next chunk (that chunk's initial-state gradient) as
  the adjoint's terminal gradient, which the kernel adds at the chunk's last
  step; the adjoint also adds the chunk's dL/da to the running sum.  The adjoint system is
  linear and block-bidiagonal (forpes.ru, §1.3), so the chunked sweep is the
  same reverse recurrence as the one-piece adjoint, cut at chunk boundaries.
  Cost: one more forward solve per chunk.
"""
import torch

from . import pararnn as pr


def _solve_span(cell, u, a, s0, out, tol, max_iters, info, stream):
    if cell == "gru":
        _, inf = pr.solve_gru(u, a, s0[0], out=out[0], tol=tol, max_iters=max_iters, info=info,
                              stream=stream)
    else:
        _, inf = pr.solve_lstm(u, a, s0[0], s0[1], out=out, tol=tol, max_iters=max_iters,
                               info=info, stream=stream)
    return inf


def _spans(T, chunk):
    if chunk <= 0:
        raise ValueError("chunk must be positive")
    return [(t0, min(T, t0 + chunk)) for t0 in range(0, T, chunk)]


def merge_info(infos):
    """One report for a chunked solve: worst chunk (synchronises)."""
    ds = [pr.read_info(i) for i in infos if i is not None]
    if not ds:
        return None
    units = sum(d["units"] for d in ds)
    isum = sum(d["iters_sum"] for d in ds)
    return dict(iters=max(d["iters"] for d in ds), converged=all(d["converged"] for d in ds),
                max_abs_res=max(d["max_abs_res"] for d in ds),
                nan_seen=any(d["nan_seen"] for d in ds), iters_sum=isum, units=units,
                iters_mean=isum / units if units else 0.0, chunks=len(ds))


def solve_chunked(cell, u, a, s0, *, chunk, out=None, tol=1e-6, max_iters=20, info=True,
                  stream=None):
    """Newton solve of the whole sequence as consecutive time chunks of at
    most `chunk` steps.  cell "gru" (s0 = [h0]) or "lstm" ([c0, h0]); u and
    out as for ``pararnn.solve_*`` (any plane layout).  Returns (states,
    info tensors, one per chunk; ``merge_info`` combines them)."""
    G, S = pr.N_GATES[pr.CELLS[cell]], pr.N_STATES[pr.CELLS[cell]]
    u, s0 = list(u), list(s0)
    if len(u) != G or len(s0) != S:
        raise ValueError("wrong number of gate or state planes")
    B, D, T = u[0].shape
    dev = u[0].device
    if out is None:
        out = pr._new_planes(S, B, T, D, pr._strides(u, "u"), dev)
    out = list(out)
    infos = []
    bnd = None
    for t0, t1 in _spans(T, chunk):
        start = s0
        if t0 > 0:
            if bnd is None:
                bnd = [torch.empty((B, D), dtype=torch.float32, device=dev) for _ in range(S)]
            for c in range(S):
                bnd[c].copy_(out[c][:, :, t0 - 1])
            start = bnd
        infos.append(_solve_span(cell, [p[:, :, t0:t1] for p in u], a, start,
                                 [o[:, :, t0:t1] for o in out], tol, max_iters, info, stream))
    return out, infos


class _Checkpointed(torch.autograd.Function):
    @staticmethod
    def forward(ctx, cell, chunk, tol, max_iters, strict, a, *planes):
        G, S = pr.N_GATES[pr.CELLS[cell]], pr.N_STATES[pr.CELLS[cell]]
        u, s0 = list(planes[:G]), list(planes[G:G + S])
        B, D, T = u[0].shape
        states, infos = solve_chunked(cell, u, a, s0, chunk=chunk, tol=tol,
                                      max_iters=max_iters, info=strict)
        if strict:
            rep = merge_info(infos)
            if not rep["converged"]:
                raise RuntimeError(f"ParaRNN Newton solve did not converge: {rep}")
        spans = _spans(T, chunk)
        # boundary states: the state before each chunk after the first
        bnd = torch.empty((max(len(spans) - 1, 0), S, B, D), dtype=torch.float32,
                          device=u[0].device)
        for k, (t0, _) in enumerate(spans[1:]):
            for c in range(S):
                bnd[k, c].copy_(states[c][:, :, t0 - 1])
        ctx.cell, ctx.chunk, ctx.tol, ctx.max_iters = cell, chunk, tol, max_iters
        ctx.set_materialize_grads(False)  # an unused output's gradient stays None
        ctx.save_for_backward(a, bnd, *u, *s0)
        return tuple(states) if S > 1 else states[0]

    @staticmethod
    def backward(ctx, *grads):
        cell, chunk = ctx.cell, ctx.chunk
        G, S = pr.N_GATES[pr.CELLS[cell]], pr.N_STATES[pr.CELLS[cell]]
        a, bnd, *rest = ctx.saved_tensors
        u, s0 = rest[:G], rest[G:G + S]
        B, D, T = u[0].shape
        dev = u[0].device
        spans = _spans(T, chunk)
        L = spans[0][1] - spans[0][0]
        # one chunk of recomputed states and of upstream gradients, in the
        # same (channel-major) layout so the adjoint reads both with one set
        # of strides
        s_buf = [torch.empty((B, D, L), dtype=torch.float32, device=dev) for _ in range(S)]
        g_buf = [torch.empty((B, D, L), dtype=torch.float32, device=dev) for _ in range(S)]
        du = [torch.empty_strided(p.shape, p.stride(), dtype=torch.float32, device=dev)
              for p in u]
        da = torch.empty((G, D), dtype=torch.float32, device=dev)
        carry = [[torch.empty((B, D), dtype=torch.float32, device=dev) for _ in range(S)]
                 for _ in range(2)]
        have_carry = False
        for k in range(len(spans) - 1, -1, -1):
            t0, t1 = spans[k]
            n = t1 - t0
            start = list(s0) if k == 0 else [bnd[k - 1, c] for c in range(S)]
            s_k = [x[:, :, :n] for x in s_buf]
            _solve_span(cell, [p[:, :, t0:t1] for p in u], a, start, s_k, ctx.tol,
                        ctx.max_iters, False, None)
            g_k = [None if grads[c] is None else g_buf[c][:, :, :n].copy_(grads[c][:, :, t0:t1])
                   for c in range(S)]
            # the next chunk's dL/ds_0 enters at this chunk's last step, and
            # dL/da accumulates over chunks, both inside the adjoint kernels
            pr.adjoint(cell, [p[:, :, t0:t1] for p in u], a, start, s_k, g_k,
                       gs_end=carry[(k + 1) % 2] if have_carry else None,
                       da_accumulate=have_carry,
                       out=dict(du=[x[:, :, t0:t1] for x in du], da=da, ds0=carry[k % 2],
                                lam=None))
            have_carry = True
        ds0 = carry[0]
        du = [g if g.dtype == p.dtype else g.to(p.dtype) for g, p in zip(du, u)]
        return (None, None, None, None, None, da, *du, *ds0)


def gru_checkpointed(u, a, h0, *, chunk, tol=1e-6, max_iters=20, strict=False):
    """Differentiable ParaGRU solve that keeps only chunk-boundary states
    for the backward pass.  u = (u_z, u_r, u_c) [B][D][T]-indexed planes;
    a [3][D]; h0 [B][D].  Returns h."""
    return _Checkpointed.apply("gru", int(chunk), tol, max_iters, strict, a, *u, h0)


def lstm_checkpointed(u, a, c0, h0, *, chunk, tol=1e-6, max_iters=20, strict=False):
    """Differentiable ParaLSTM solve that keeps only chunk-boundary states
    for the backward pass.  u = (u_i, u_f, u_g, u_o); a [4][D]; c0, h0
    [B][D].  Returns (c, h)."""
    return _Checkpointed.apply("lstm", int(chunk), tol, max_iters, strict, a, *u, c0, h0)
