"""Input projection reference — test infrastructure only.

u[b][m][t] = sum_k W[m][k] x[b][t][k] + bias[m]: the dense product that
turns the inputs into the per-gate projections u_t = W x_t + b the cells
consume (voguetech.ru ParaRNN article, "Что именно сделали технически",
item 3).  Its plain definition in float64, one batch row at a time, with
numpy's matrix product as the only step; pinned in tests/test_oracle_pins.py
by a brute-force triple loop, an identity weight (the transpose of x) and a
bias-only case.
"""
import numpy as np


def project(x, W, bias=None):
    """x [B][T][I], W [M][I], bias [M] or None -> u [B][M][T], float64."""
    x = np.asarray(x, np.float64)
    W = np.asarray(W, np.float64)
    B, T, I = x.shape
    M = W.shape[0]
    u = np.empty((B, M, T))
    for b in range(B):
        u[b] = W @ x[b].T
    if bias is not None:
        u += np.asarray(bias, np.float64)[None, :, None]
    return u


def project_abs(x, W, bias=None):
    """sum_k |W[m][k] x[b][t][k]| + |bias[m]|: the scale of the rounding
    error of any summation order of the products."""
    return project(np.abs(np.asarray(x, np.float64)), np.abs(np.asarray(W, np.float64)),
                   None if bias is None else np.abs(np.asarray(bias, np.float64)))
