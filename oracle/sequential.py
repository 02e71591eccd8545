"""ORACLE — test infrastructure only: sequential fp64 cells and BPTT.

ctypes front end of ``oracle/oracle.c``.  The true trajectory is the unique
zero of the DEER residual and equals the step-by-step application of the
cell ("Параллельность RNN?" (forpes.ru), §1.1); these functions compute it
directly, channel by channel, in double precision.

All per-step arrays are numpy ``float32`` ``[B][D][T]`` (C-contiguous) on
input — exactly what the device path consumes — and ``float64`` on output.
Diagonal weights ``a`` are ``[G][D]``: GRU gates (z, r, c), LSTM gates
(i, f, g, o).  ``nthreads=0`` uses every OpenMP thread.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        lib.oracle_gru_forward.argtypes = [i64, i64, i64] + [vp] * 6 + [i32]
        lib.oracle_gru_bptt.argtypes = [i64, i64, i64] + [vp] * 13 + [i32]
        lib.oracle_lstm_forward.argtypes = [i64, i64, i64] + [vp] * 9 + [i32]
        lib.oracle_lstm_bptt.argtypes = [i64, i64, i64] + [vp] * 20 + [i32]
        for f in (lib.oracle_gru_forward, lib.oracle_gru_bptt,
                  lib.oracle_lstm_forward, lib.oracle_lstm_bptt):
            f.restype = ctypes.c_int
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _f32(x, shape):
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.shape != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {x.shape}")
    return x


def _p(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def _dims(u0):
    if u0.ndim != 3:
        raise ValueError("per-step planes must be [B][D][T]")
    return u0.shape


def gru_forward(u, a, h0, nthreads=0):
    """Sequential ParaGRU.  u = (u_z, u_r, u_c), each [B][D][T]; a [3][D];
    h0 [B][D].  Returns h [B][D][T] float64."""
    B, D, T = _dims(np.asarray(u[0]))
    uz, ur, uc = (_f32(x, (B, D, T)) for x in u)
    a = _f32(a, (3, D))
    h0 = _f32(h0, (B, D))
    h = np.empty((B, D, T), np.float64)
    rc = _load().oracle_gru_forward(B, T, D, _p(uz), _p(ur), _p(uc), _p(a),
                                    _p(h0), _p(h), nthreads)
    if rc:
        raise RuntimeError(f"oracle_gru_forward failed ({rc})")
    return h


def gru_bptt(u, a, h0, dh, nthreads=0):
    """Back-propagation through time of L = sum_t <dh_t, h_t> for ParaGRU.
    Returns dict(h, du=(du_z, du_r, du_c), da [3][D], dh0 [B][D],
    lam = total dL/dh_t [B][D][T])."""
    B, D, T = _dims(np.asarray(u[0]))
    uz, ur, uc = (_f32(x, (B, D, T)) for x in u)
    a = _f32(a, (3, D))
    h0 = _f32(h0, (B, D))
    dh = _f32(dh, (B, D, T))
    h = np.empty((B, D, T), np.float64)
    du = [np.empty((B, D, T), np.float64) for _ in range(3)]
    da = np.empty((3, D), np.float64)
    dh0 = np.empty((B, D), np.float64)
    lam = np.empty((B, D, T), np.float64)
    rc = _load().oracle_gru_bptt(B, T, D, _p(uz), _p(ur), _p(uc), _p(a), _p(h0),
                                 _p(dh), _p(h), _p(du[0]), _p(du[1]), _p(du[2]),
                                 _p(da), _p(dh0), _p(lam), nthreads)
    if rc:
        raise RuntimeError(f"oracle_gru_bptt failed ({rc})")
    return dict(h=h, du=tuple(du), da=da, dh0=dh0, lam=lam)


def lstm_forward(u, a, c0, h0, nthreads=0):
    """Sequential ParaLSTM.  u = (u_i, u_f, u_g, u_o), each [B][D][T];
    a [4][D]; c0, h0 [B][D].  Returns (c, h), each [B][D][T] float64."""
    B, D, T = _dims(np.asarray(u[0]))
    ui, uf, ug, uo = (_f32(x, (B, D, T)) for x in u)
    a = _f32(a, (4, D))
    c0 = _f32(c0, (B, D))
    h0 = _f32(h0, (B, D))
    c = np.empty((B, D, T), np.float64)
    h = np.empty((B, D, T), np.float64)
    rc = _load().oracle_lstm_forward(B, T, D, _p(ui), _p(uf), _p(ug), _p(uo),
                                     _p(a), _p(c0), _p(h0), _p(c), _p(h), nthreads)
    if rc:
        raise RuntimeError(f"oracle_lstm_forward failed ({rc})")
    return c, h


def lstm_bptt(u, a, c0, h0, dh, dc=None, nthreads=0):
    """Back-propagation through time of L = sum_t <dh_t, h_t> + <dc_t, c_t>
    for ParaLSTM (dc=None means zero).  Returns dict(c, h,
    du=(du_i, du_f, du_g, du_o), da [4][D], dc0, dh0, lam_c, lam_h), the last
    two being the total dL/dc_t and dL/dh_t."""
    B, D, T = _dims(np.asarray(u[0]))
    ui, uf, ug, uo = (_f32(x, (B, D, T)) for x in u)
    a = _f32(a, (4, D))
    c0 = _f32(c0, (B, D))
    h0 = _f32(h0, (B, D))
    dh = _f32(dh, (B, D, T))
    dc = None if dc is None else _f32(dc, (B, D, T))
    c = np.empty((B, D, T), np.float64)
    h = np.empty((B, D, T), np.float64)
    du = [np.empty((B, D, T), np.float64) for _ in range(4)]
    da = np.empty((4, D), np.float64)
    dc0 = np.empty((B, D), np.float64)
    dh0 = np.empty((B, D), np.float64)
    lam_c = np.empty((B, D, T), np.float64)
    lam_h = np.empty((B, D, T), np.float64)
    rc = _load().oracle_lstm_bptt(B, T, D, _p(ui), _p(uf), _p(ug), _p(uo), _p(a),
                                  _p(c0), _p(h0), _p(dh), _p(dc), _p(c), _p(h),
                                  _p(du[0]), _p(du[1]), _p(du[2]), _p(du[3]),
                                  _p(da), _p(dc0), _p(dh0), _p(lam_c), _p(lam_h),
                                  nthreads)
    if rc:
        raise RuntimeError(f"oracle_lstm_bptt failed ({rc})")
    return dict(c=c, h=h, du=tuple(du), da=da, dc0=dc0, dh0=dh0,
                lam_c=lam_c, lam_h=lam_h)


def gather_channels(planes, a, s0s, channels):
    """Pick channels [(b, d), ...] out of full-size inputs so that the
    oracle can run on a sample: returns (planes [1][n][T], a [G][n],
    initial states [1][n]) — the cells are per channel, so a channel's
    trajectory does not depend on any other channel."""
    bs = np.array([c[0] for c in channels], dtype=np.int64)
    ds = np.array([c[1] for c in channels], dtype=np.int64)
    sub = [np.ascontiguousarray(np.asarray(p)[bs, ds, :][None]) for p in planes]
    a_sub = np.ascontiguousarray(np.asarray(a)[:, ds])
    s0_sub = [np.ascontiguousarray(np.asarray(s)[bs, ds][None]) for s in s0s]
    return sub, a_sub, s0_sub
