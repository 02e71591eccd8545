"""Helpers shared by the GPU tests: move seeded inputs to the device, run the
HIP path through the binding, and compare with the CPU oracle."""
import numpy as np
import torch

from nonlinear_rnn_amd import pararnn as pr
from oracle import sequential as seq

DEV = "cuda:0"


def dev_inputs(inp):
    """Device tensors for the HIP path: the projections the device sees (bf16
    bits reinterpreted as torch.bfloat16 when the workload says so)."""
    if inp.u_bf16 is not None:
        u = [torch.from_numpy(p.view(np.int16)).view(torch.bfloat16).to(DEV) for p in inp.u_bf16]
    else:
        u = [torch.from_numpy(p).to(DEV) for p in inp.u]
    a = torch.from_numpy(inp.a).to(DEV)
    s0 = [torch.from_numpy(p).to(DEV) for p in inp.s0]
    return u, a, s0


def gpu_solve(inp, tol, cap, K=0, W=0, init=None, stream=None):
    """Returns (list of state planes as float32 numpy, info dict)."""
    u, a, s0 = dev_inputs(inp)
    if inp.cell == "gru":
        out = None if init is None else torch.from_numpy(np.ascontiguousarray(init[0])).to(DEV)
        h, info = pr.solve_gru(u, a, s0[0], out=out, tol=tol, max_iters=cap, steps_per_lane=K,
                               waves_per_block=W, init_from_output=init is not None,
                               stream=stream)
        states = [h]
    else:
        out = (None if init is None
               else [torch.from_numpy(np.ascontiguousarray(x)).to(DEV) for x in init])
        (c, h), info = pr.solve_lstm(u, a, s0[0], s0[1], out=out, tol=tol, max_iters=cap,
                                     steps_per_lane=K, waves_per_block=W,
                                     init_from_output=init is not None, stream=stream)
        states = [c, h]
    inf = pr.read_info(info)
    return [s.cpu().numpy() for s in states], inf


def oracle_states(inp, rounded=True, nthreads=0):
    u = inp.u_rounded if rounded else inp.u
    if inp.cell == "gru":
        return [seq.gru_forward(u, inp.a, inp.s0[0], nthreads)]
    c, h = seq.lstm_forward(u, inp.a, inp.s0[0], inp.s0[1], nthreads)
    return [c, h]


def max_err(got, ref):
    return max(float(np.max(np.abs(g.astype(np.float64) - r))) if g.size else 0.0
               for g, r in zip(got, ref))
