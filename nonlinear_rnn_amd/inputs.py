"""Seeded synthetic inputs for the ParaGRU / ParaLSTM Newton solves.

This module only draws random numbers and lays them out; it holds none of
the method's arithmetic.  Both the device path and the CPU oracle consume the
arrays it returns, so the two always see identical inputs.

Recipe (numpy PCG64 via ``numpy.random.default_rng(seed)``; draw order is
fixed): the gate planes of ``u`` in gate order, then the diagonal weights
``a`` ([G][D], gate order), then the initial states, then the upstream
gradients.

* ``u_*`` ~ N(0, 1) float32, one [B][D][T] plane per gate (time fastest);
  for the LSTM the forget-gate plane gets +1 (the forget-gate bias is part of
  the precomputed projection).
* ``a_*`` ~ U(-1, 1) float32, one value per gate and channel.
* initial states: zero, or N(0, std^2) for ``s0_std > 0``.
* upstream gradients dL/dh ~ N(0, 1) float32 [B][D][T].
* bf16 projections: the float32 draw rounded to nearest-even bfloat16; the
  unrounded float32 draw is kept too.

GRU gate order is (z, r, c); LSTM gate order is (i, f, g, o); LSTM states
are (c, h).
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

GATES = {"gru": ("z", "r", "c"), "lstm": ("i", "f", "g", "o")}
STATES = {"gru": ("h",), "lstm": ("c", "h")}


@dataclass
class Workload:
    name: str
    cell: str           # "gru" | "lstm"
    B: int
    T: int
    D: int
    u_dtype: str = "f32"  # "f32" | "bf16"
    s0_std: float = 0.0
    f_bias: float = 0.0
    tol: float = 1e-6
    max_iters: int = 20
    adjoint: bool = False
    seed: int = 0

    @property
    def N(self) -> int:
        return self.B * self.T * self.D

    @property
    def G(self) -> int:
        return len(GATES[self.cell])

    @property
    def S(self) -> int:
        return len(STATES[self.cell])


# The five workloads the parity tests and the bench use (seed = index + 1).
WORKLOADS = {
    "gru_small": Workload("ParaGRU f32 B=1 T=1024 D=64", "gru", 1, 1024, 64,
                          tol=1e-6, max_iters=20, seed=1),
    "gru_f32": Workload("ParaGRU f32 B=8 T=4096 D=1024", "gru", 8, 4096, 1024,
                        s0_std=0.1, tol=1e-6, max_iters=20, seed=2),
    "lstm_f32": Workload("ParaLSTM f32 B=8 T=4096 D=1024", "lstm", 8, 4096, 1024,
                         f_bias=1.0, tol=1e-6, max_iters=20, seed=3),
    "gru_bf16_long": Workload("ParaGRU bf16-u B=4 T=16384 D=4096", "gru", 4, 16384,
                              4096, u_dtype="bf16", tol=1e-5, max_iters=30, seed=4),
    "lstm_fwd_bwd": Workload("ParaLSTM f32 fwd+adjoint B=16 T=2048 D=4096", "lstm",
                             16, 2048, 4096, f_bias=1.0, tol=1e-6, max_iters=20,
                             adjoint=True, seed=5),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, nearest-even; returns the uint16 bit
    patterns.  (Finite inputs only, which is all this module draws.)"""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    return ((bits + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Inputs:
    cell: str
    u: list                       # G float32 planes [B][D][T] (unrounded draw)
    a: np.ndarray                 # [G][D] float32
    s0: list                      # S float32 planes [B][D]
    dh: Optional[np.ndarray] = None   # [B][D][T] float32 or None
    u_bf16: Optional[list] = None     # G uint16 planes (bf16 bits) or None
    meta: dict = field(default_factory=dict)

    @property
    def u_rounded(self) -> list:
        """The projections the device actually sees, as float32."""
        if self.u_bf16 is None:
            return self.u
        return [bf16_to_f32(p) for p in self.u_bf16]


def make_inputs(cell: str, B: int, T: int, D: int, seed: int, *,
                u_dtype: str = "f32", s0_std: float = 0.0, f_bias: float = 0.0,
                with_grad: bool = False, a_scale: float = 1.0,
                u_scale: float = 1.0) -> Inputs:
    """Draw one workload.  ``a_scale`` widens a ~ U(-a_scale, a_scale) (stiff
    cells); ``u_scale`` scales the N(0, 1) projections."""
    if cell not in GATES:
        raise ValueError(f"unknown cell {cell!r}")
    rng = np.random.default_rng(seed)
    G, S = len(GATES[cell]), len(STATES[cell])
    u = []
    for g in range(G):
        p = rng.standard_normal((B, D, T), dtype=np.float32)
        if u_scale != 1.0:
            p *= np.float32(u_scale)
        if cell == "lstm" and g == 1 and f_bias:
            p += np.float32(f_bias)
        u.append(p)
    a = (rng.random((G, D), dtype=np.float32) * np.float32(2.0) - np.float32(1.0))
    if a_scale != 1.0:
        a *= np.float32(a_scale)
    s0 = []
    for _ in range(S):
        if s0_std > 0:
            s0.append(rng.standard_normal((B, D), dtype=np.float32) * np.float32(s0_std))
        else:
            s0.append(np.zeros((B, D), np.float32))
    dh = rng.standard_normal((B, D, T), dtype=np.float32) if with_grad else None
    u_bf16 = [round_to_bf16(p) for p in u] if u_dtype == "bf16" else None
    meta = dict(seed=seed, rng="numpy PCG64 default_rng", u_dtype=u_dtype,
                s0_std=s0_std, f_bias=f_bias, a="U(-%g,%g)" % (a_scale, a_scale),
                u="N(0,%g)" % (u_scale ** 2))
    return Inputs(cell, u, a, s0, dh, u_bf16, meta)


def workload_inputs(w: Workload) -> Inputs:
    return make_inputs(w.cell, w.B, w.T, w.D, w.seed, u_dtype=w.u_dtype,
                       s0_std=w.s0_std, f_bias=w.f_bias, with_grad=w.adjoint)
