"""Python binding of libpararnn.so (argument marshalling only).

Every computation runs in the HIP kernels behind the C ABI of
``include/pararnn.h``; this module only turns torch tensors (device memory)
and the current HIP stream into the pointers and sizes the ABI takes, and
raises on a non-OK status.  There is no fallback: if the library or a GPU
is missing, the calls raise.

Names follow the ABI: ``solve_gru``, ``solve_gru_noalloc``, ``solve_lstm``,
``adjoint``, ``scan``, ``sequential``, ``project``, ``workspace_bytes``,
``plan``.
"""
import ctypes
import os
import struct

import torch  # loads the HIP runtime the library then shares

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpararnn.so")

GRU, LSTM = 0, 1
F32, BF16 = 0, 1
CELLS = {"gru": GRU, "lstm": LSTM}
N_GATES = {GRU: 3, LSTM: 4}
N_STATES = {GRU: 1, LSTM: 2}


class PararnnError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"pararnn status {status}: {msg}")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("D", ctypes.c_int64),
                ("u_stride_b", ctypes.c_int64), ("u_stride_d", ctypes.c_int64),
                ("s_stride_b", ctypes.c_int64), ("s_stride_d", ctypes.c_int64),
                ("u_stride_t", ctypes.c_int64), ("s_stride_t", ctypes.c_int64)]


class ProjShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("I", ctypes.c_int64),
                ("M", ctypes.c_int64), ("x_stride_b", ctypes.c_int64),
                ("x_stride_t", ctypes.c_int64), ("w_stride_m", ctypes.c_int64),
                ("u_stride_b", ctypes.c_int64), ("u_stride_m", ctypes.c_int64)]


class Newton(ctypes.Structure):
    _fields_ = [("tol", ctypes.c_float), ("max_iters", ctypes.c_int32),
                ("steps_per_lane", ctypes.c_int32), ("waves_per_block", ctypes.c_int32),
                ("init_from_output", ctypes.c_int32)]


INFO_BYTES = 32
STATIC_SCRATCH_BYTES = 32 << 20  # PARARNN_STATIC_SCRATCH_BYTES
_INFO_FMT = "<iifiqq"

_lib = None


def load():
    """Load libpararnn.so (after torch, so both use one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m nonlinear_rnn_amd.build`")
    lib = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_GLOBAL)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    P = ctypes.POINTER
    lib.pararnn_status_string.restype = ctypes.c_char_p
    lib.pararnn_status_string.argtypes = [i32]
    lib.pararnn_workspace_bytes.restype = sz
    lib.pararnn_workspace_bytes.argtypes = [i32, P(Shape), P(Newton), i32]
    lib.pararnn_plan.restype = i32
    lib.pararnn_plan.argtypes = [i32, P(Shape), P(Newton), i32, P(ctypes.c_int32),
                                 P(ctypes.c_int32), P(ctypes.c_int64)]
    lib.pararnn_solve_gru.restype = i32
    lib.pararnn_solve_gru.argtypes = [P(Shape), vp, i32, vp, vp, vp, P(Newton), vp, vp, sz, vp]
    lib.pararnn_solve_gru_noalloc.restype = i32
    lib.pararnn_solve_gru_noalloc.argtypes = [P(Shape), vp, i32, vp, vp, vp, P(Newton), vp, vp]
    lib.pararnn_solve_lstm.restype = i32
    lib.pararnn_solve_lstm.argtypes = [P(Shape), vp, i32, vp, vp, vp, vp, vp, P(Newton), vp,
                                       vp, sz, vp]
    lib.pararnn_project.restype = i32
    lib.pararnn_project.argtypes = [P(ProjShape), vp, vp, vp, vp, i32, vp]
    lib.pararnn_sequential.restype = i32
    lib.pararnn_sequential.argtypes = [i32, P(Shape), vp, i32, vp, vp, vp, vp]
    lib.pararnn_scan_workspace_bytes.restype = sz
    lib.pararnn_scan_workspace_bytes.argtypes = [i32, P(Shape), P(Newton)]
    lib.pararnn_scan.restype = i32
    lib.pararnn_scan.argtypes = [i32, P(Shape), vp, vp, vp, vp, i32, P(Newton), vp, sz, vp]
    lib.pararnn_adjoint.restype = i32
    lib.pararnn_adjoint.argtypes = [i32, P(Shape), vp, i32, vp, vp, vp, vp, vp, vp, vp, i32,
                                    vp, vp, P(Newton), vp, sz, vp]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().pararnn_status_string(status).decode()


def _check(status):
    if status != 0:
        raise PararnnError(status, status_string(status))


def _ptr(t):
    # plain ints: ctypes converts them for c_void_p parameters
    return None if t is None else t.data_ptr()


def _ptr_array(ts):
    arr = (ctypes.c_void_p * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = None if t is None else t.data_ptr()
    return arr


# ------------------------------------------------------- argument checks ---
# Every check runs before the library is called: a tensor of the wrong
# dtype, shape, layout or device would otherwise hand the kernels a pointer
# they read or write out of bounds.  Shape and dtype are checked before the
# device, so each message names the first thing that is wrong.

def _require(cond, msg):
    """Raise ValueError(msg) if not cond; msg may be a callable, so that the
    message is only built on failure (these checks run on every call)."""
    if not cond:
        raise ValueError(msg() if callable(msg) else msg)


def _is_tensor(t):
    return isinstance(t, torch.Tensor)


def _plane_dims(planes, name):
    """(B, D, T) shared by every non-None plane (indexed [B][D][T])."""
    dims = None
    for p in planes:
        if p is None:
            continue
        if not _is_tensor(p) or p.dim() != 3:
            raise ValueError(f"{name}: planes must be 3-d tensors [B][D][T]")
        if dims is None:
            dims = p.shape
        elif p.shape != dims:
            raise ValueError(f"{name}: every plane must have the same shape")
    if dims is None:
        raise ValueError(f"{name}: no planes given")
    return tuple(dims)


_F32_ONLY = (torch.float32,)
_U_DTYPES = (torch.float32, torch.bfloat16)


def _gate_planes(u, G):
    """Checks the G projection planes (same shape [B][D][T], all float32 or
    all bfloat16); returns ((B, D, T), ABI dtype code).  One pass, since it
    runs on every solve."""
    if len(u) != G:
        raise ValueError(f"expected {G} gate planes, got {len(u)}")
    p0 = u[0]
    if not _is_tensor(p0) or p0.dim() != 3:
        raise ValueError("u: planes must be 3-d tensors [B][D][T]")
    dims, dt = p0.shape, p0.dtype
    if dt is torch.float32:
        code = F32
    elif dt is torch.bfloat16:
        code = BF16
    else:
        raise ValueError("u planes must be float32 or bfloat16")
    for p in u[1:]:
        if not _is_tensor(p) or p.shape != dims:
            raise ValueError("u: every plane must have the same shape [B][D][T]")
        if p.dtype is not dt:
            raise ValueError("u planes must all be float32 or all bfloat16")
    return tuple(dims), code


def _check_planes(planes, name, dims, dtypes=_F32_ONLY, allow_none=False):
    for p in planes:
        if p is None:
            if not allow_none:
                raise ValueError(f"{name}: a plane is missing")
            continue
        if not _is_tensor(p) or p.shape != dims:
            raise ValueError(f"{name}: planes must be [B][D][T] = {list(dims)}")
        if p.dtype not in dtypes:
            raise ValueError(f"{name}: planes must be {' or '.join(map(str, dtypes))}")


def _check_dense(t, name, dims):
    if not _is_tensor(t) or t.shape != dims:
        raise ValueError(f"{name}: expected a tensor of shape {list(dims)}")
    if t.dtype != torch.float32:
        raise ValueError(f"{name}: must be float32")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _check_devices(dev, tensors):
    """Every tensor on `dev`, and `dev` a GPU (checked last)."""
    for name, t in tensors:
        if t is not None and t.device != dev:
            raise ValueError(f"{name}: on {t.device}, expected {dev} (the device of u)")
    if dev.type != "cuda":
        raise ValueError(f"tensors are on {dev}: the kernels need GPU device memory")


def _record_on(stream, tensors):
    """Tensors allocated on the current stream but written on another one:
    tell torch's allocator, so it does not hand their memory out again
    before that stream's work is done."""
    if stream is None:
        return
    cur = torch.cuda.current_stream(stream.device)
    if stream.cuda_stream == cur.cuda_stream:
        return
    for t in tensors:
        if t is not None and t.numel():
            t.record_stream(stream)


def _strides(planes, name):
    """Shared (stride_b, stride_d, stride_t) of planes indexed [B][D][T], or
    None when every plane is empty.  Any layout is passed on (the library
    rejects overlapping ones): channel-major [B][D][T] is the fast one, a
    time-major [B][T][D] tensor is passed as its ``transpose(1, 2)`` view."""
    st = None
    for p in planes:
        if p is None:
            continue
        if p.dim() != 3:
            raise ValueError(f"{name}: planes must be indexed [B][D][T]")
        if p.numel() == 0:
            continue
        s = tuple(p.stride())
        if st is not None and s != st:
            raise ValueError(f"{name}: all planes must share strides")
        st = s
    return st


def _dense(B, T, D, like=None):
    """Strides of a new plane: time-major when `like` (strides) is not
    time-contiguous, channel-major otherwise."""
    if like is not None and like[2] != 1 and T > 1:
        return (T * D, 1, D)
    return (D * T, T, 1)


def _new_planes(n, B, T, D, like, dev):
    st = _dense(B, T, D, like)
    return [torch.empty_strided((B, D, T), st, dtype=torch.float32, device=dev)
            for _ in range(n)]


def make_shape(B, T, D, u_strides=None, s_strides=None):
    """Shape record; strides default to dense channel-major [B][D][T]."""
    us = u_strides or (D * T, T, 1)
    ss = s_strides or (D * T, T, 1)
    if len(us) == 2:
        us = (us[0], us[1], 1)
    if len(ss) == 2:
        ss = (ss[0], ss[1], 1)
    return Shape(B, T, D, us[0], us[1], ss[0], ss[1], us[2], ss[2])


def make_newton(tol=1e-6, max_iters=20, steps_per_lane=0, waves_per_block=0,
                init_from_output=False):
    return Newton(float(tol), int(max_iters), int(steps_per_lane), int(waves_per_block),
                  1 if init_from_output else 0)


def workspace_bytes(cell, shape, newton=None, adjoint=False):
    cell = CELLS.get(cell, cell)
    return int(load().pararnn_workspace_bytes(cell, ctypes.byref(shape),
                                              ctypes.byref(newton) if newton else None,
                                              1 if adjoint else 0))


def plan(cell, shape, newton=None, adjoint=False):
    """(steps per lane K, waves per block W, time blocks per channel)."""
    cell = CELLS.get(cell, cell)
    K, W, nb = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
    _check(load().pararnn_plan(cell, ctypes.byref(shape),
                               ctypes.byref(newton) if newton else None, 1 if adjoint else 0,
                               ctypes.byref(K), ctypes.byref(W), ctypes.byref(nb)))
    return K.value, W.value, nb.value


def decode_info(raw) -> dict:
    it, conv, mres, nan, isum, units = struct.unpack(_INFO_FMT, bytes(raw))
    return dict(iters=it, converged=bool(conv), max_abs_res=mres, nan_seen=bool(nan),
                iters_sum=isum, units=units, iters_mean=(isum / units) if units else 0.0)


class Workspace:
    """Grow-only device scratch buffers (torch-allocated), one per device
    and stream: the kernels' per-launch state (tickets, flags, records,
    partial sums) lives there, so launches on different streams must not
    share one.  Each buffer is allocated on its own stream, so torch's
    allocator orders its reuse after that stream's work."""

    MAX_STREAMS = 8  # buffers kept for the most recently used streams

    def __init__(self):
        self.buf = {}

    def get(self, nbytes, device, stream=None):
        if nbytes == 0:
            return None
        s = stream if stream is not None else torch.cuda.current_stream(device)
        key = (torch.device(device).index, s.cuda_stream)
        b = self.buf.pop(key, None)
        if b is None or b.numel() < nbytes:
            with torch.cuda.stream(s):
                b = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.buf[key] = b  # most recent last
        while len(self.buf) > self.MAX_STREAMS:
            # the oldest entry goes back to torch's allocator, which reuses it
            # only in its own stream's order
            self.buf.pop(next(iter(self.buf)))
        return b


_ws = Workspace()
_ws_sizes = {}  # (shape record, options record, workspace bytes) by solve arguments


def _stream_handle(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _u_dtype(planes):
    dts = {p.dtype for p in planes}
    if dts == {torch.float32}:
        return F32
    if dts == {torch.bfloat16}:
        return BF16
    raise ValueError("u planes must all be float32 or all bfloat16")


def _solve(cell, u, a, s0, out, tol, max_iters, steps_per_lane, waves_per_block,
           init_from_output, info, workspace, stream):
    lib = load()
    G, S = N_GATES[cell], N_STATES[cell]
    _require(len(s0) == S, "wrong number of state planes")
    (B, D, T), udt = _gate_planes(u, G)
    _check_dense(a, "a", (G, D))
    for i, x in enumerate(s0):
        _check_dense(x, f"initial state {i}", (B, D))
    dev = u[0].device
    allocated = []
    if out is None:
        _require(not init_from_output, "init_from_output needs the output planes")
        out = _new_planes(S, B, T, D, _strides(u, "u"), dev)
        allocated += out
    out = list(out)
    _require(len(out) == S, "wrong number of output planes")
    _check_planes(out, "states", (B, D, T))
    _check_devices(dev, [("u", p) for p in u] + [("a", a)] + [("initial state", x) for x in s0]
                   + [("states", x) for x in out] + [("workspace", workspace)])
    us, ss = _strides(u, "u"), _strides(out, "states")
    # the shape and option records and the workspace size depend on these
    # arguments only; cached so that small solves do not rebuild them (nor
    # pay a second library call) on every launch
    wkey = (cell, B, T, D, us, ss, tol, max_iters, steps_per_lane, waves_per_block,
            bool(init_from_output))
    hit = _ws_sizes.get(wkey)
    if hit is None:
        if len(_ws_sizes) >= 4096:
            _ws_sizes.clear()
        shape = make_shape(B, T, D, us, ss)
        newton = make_newton(tol, max_iters, steps_per_lane, waves_per_block, init_from_output)
        hit = _ws_sizes[wkey] = (shape, newton, workspace_bytes(cell, shape, newton))
    shape, newton, nws = hit
    ws = workspace if workspace is not None else _ws.get(nws, dev, stream)
    info_t = torch.empty(INFO_BYTES, dtype=torch.uint8, device=dev) if info else None
    _record_on(stream, allocated + [info_t])
    args = [ctypes.byref(shape), _ptr_array(u), udt, _ptr(a)]
    args += [_ptr(x) for x in s0] + [_ptr(x) for x in out]
    args += [ctypes.byref(newton), _ptr(info_t), _ptr(ws),
             0 if ws is None else ws.numel(), _stream_handle(stream)]
    fn = lib.pararnn_solve_gru if cell == GRU else lib.pararnn_solve_lstm
    _check(fn(*args))
    return out, info_t


def solve_gru(u, a, h0, *, out=None, tol=1e-6, max_iters=20, steps_per_lane=0,
              waves_per_block=0, init_from_output=False, info=True, workspace=None,
              stream=None):
    """ParaGRU Newton solve.  u = [u_z, u_r, u_c] device tensors [B][D][T]
    (float32 or bfloat16), a [3][D] float32, h0 [B][D] float32.  Returns
    (h, info_tensor) with info_tensor a 32-byte device buffer (or None);
    ``read_info(info_tensor)`` synchronises and decodes it."""
    out = None if out is None else [out]
    s, info_t = _solve(GRU, list(u), a, [h0], out, tol, max_iters, steps_per_lane,
                       waves_per_block, init_from_output, info, workspace, stream)
    return s[0], info_t


def solve_gru_noalloc(u, a, h0, out, *, tol=1e-6, max_iters=20, steps_per_lane=0,
                      waves_per_block=0, init_from_output=False, info=None, stream=None):
    """ParaGRU Newton solve that allocates nothing: ``out`` ([B][D][T]
    float32) and ``info`` (a 32-byte device buffer, or None) are the
    caller's, and the library's static per-GPU scratch array serves as the
    workspace (problems needing more than PARARNN_STATIC_SCRATCH_BYTES
    raise).  Calls whose executions overlap on one GPU share that array
    and must not overlap.  Returns ``out``."""
    lib = load()
    B, D, T = _plane_dims(list(u), "u")
    _require(len(u) == 3, "wrong number of gate planes")
    _check_planes(u, "u", (B, D, T), _U_DTYPES)
    _u_dtype(u)
    _check_dense(a, "a", (3, D))
    _check_dense(h0, "initial state", (B, D))
    _check_planes([out], "states", (B, D, T))
    if info is not None:
        _require(_is_tensor(info) and info.dtype == torch.uint8 and info.numel() == INFO_BYTES
                 and info.is_contiguous(), f"info must be a contiguous {INFO_BYTES}-byte uint8 buffer")
    dev = u[0].device
    _check_devices(dev, [("u", p) for p in u] + [("a", a), ("initial state", h0), ("states", out),
                         ("info", info)])
    us, ss = _strides(u, "u"), _strides([out], "states")
    shape = make_shape(B, T, D, us, ss)
    newton = make_newton(tol, max_iters, steps_per_lane, waves_per_block, init_from_output)
    _check(lib.pararnn_solve_gru_noalloc(ctypes.byref(shape), _ptr_array(u), _u_dtype(u), _ptr(a),
                                         _ptr(h0), _ptr(out), ctypes.byref(newton), _ptr(info),
                                         _stream_handle(stream)))
    return out


def solve_lstm(u, a, c0, h0, *, out=None, tol=1e-6, max_iters=20, steps_per_lane=0,
               waves_per_block=0, init_from_output=False, info=True, workspace=None,
               stream=None):
    """ParaLSTM Newton solve.  u = [u_i, u_f, u_g, u_o]; a [4][D]; c0, h0
    [B][D].  Returns ((c, h), info_tensor)."""
    s, info_t = _solve(LSTM, list(u), a, [c0, h0], out, tol, max_iters, steps_per_lane,
                       waves_per_block, init_from_output, info, workspace, stream)
    return (s[0], s[1]), info_t


def read_info(info_t) -> dict:
    torch.cuda.current_stream(info_t.device).synchronize()
    return decode_info(info_t.cpu().numpy().tobytes())


def adjoint(cell, u, a, s0, s, gs, *, gs_end=None, da_accumulate=False, with_lambda=False,
            steps_per_lane=0, waves_per_block=0, workspace=None, stream=None, out=None):
    """Backward pass of a converged solve for L = sum_t <gs_t, s_t>.
    cell "gru" (s0, s, gs: [h]) or "lstm" ([c, h]); an entry of gs may be
    None (zero).  ``gs_end`` (None, or S [B][D] tensors / None) is added to
    dL/ds_T: the ds0 a continuation of the sequence sends back.  With
    ``da_accumulate`` the new dL/da is added to ``out["da"]``.  Returns
    dict(du=[G planes], da [G][D], ds0=[S], lam=[S] or None), all float32
    device tensors; `out`, a dict of that form returned by an earlier call on
    the same shapes, is written in place instead of allocating."""
    lib = load()
    _require(cell in CELLS or cell in (GRU, LSTM), f"unknown cell {cell!r}")
    cell = CELLS.get(cell, cell)
    G, S = N_GATES[cell], N_STATES[cell]
    u, s0, s, gs = list(u), list(s0), list(s), list(gs)
    _require(len(u) == G and len(s0) == S and len(s) == S and len(gs) == S,
             "wrong number of gate or state planes")
    B, D, T = _plane_dims(u, "u")
    _check_planes(u, "u", (B, D, T), _U_DTYPES)
    _u_dtype(u)
    _check_dense(a, "a", (G, D))
    for i, x in enumerate(s0):
        _check_dense(x, f"initial state {i}", (B, D))
    _check_planes(s, "states", (B, D, T))
    _check_planes(gs, "upstream gradients", (B, D, T), allow_none=True)
    if gs_end is not None:
        gs_end = list(gs_end)
        _require(len(gs_end) == S, "gs_end: one [B][D] tensor (or None) per state component")
        for i, x in enumerate(gs_end):
            if x is not None:
                _check_dense(x, f"gs_end[{i}]", (B, D))
    _require(not da_accumulate or out is not None, "da_accumulate needs out['da'] to add to")
    dev = u[0].device
    us = _strides(u, "u") or (D * T, T, 1)
    ss = _strides(s + [g for g in gs if g is not None], "states") or (D * T, T, 1)
    allocated = []
    if out is not None:
        du, da, ds0, lam = list(out["du"]), out["da"], list(out["ds0"]), out.get("lam")
        lam = list(lam) if (lam is not None and with_lambda) else None
        dense = (D * T, T, 1)
        if (len(du) != G or len(ds0) != S or not _is_tensor(da) or tuple(da.shape) != (G, D)
                or any(tuple(x.shape) != (B, D, T) for x in du + (lam or []))
                or (_strides(du, "du") or dense) != us
                or any(tuple(x.shape) != (B, D) for x in ds0)
                or (with_lambda and (lam is None or len(lam) != S
                                     or (_strides(lam, "lam") or dense) != ss))):
            raise ValueError("out buffers do not match this problem")
        for x in du + [da] + ds0 + (lam or []):
            if x.dtype != torch.float32 or x.device != dev:
                raise ValueError("out buffers must be float32 on the device of u")
        for x in [da] + ds0:
            if not x.is_contiguous():
                raise ValueError("da and ds0 outputs must be contiguous")
    else:
        du = [torch.empty_strided((B, D, T), us, dtype=torch.float32, device=dev)
              for _ in range(G)]
        da = torch.empty((G, D), dtype=torch.float32, device=dev)
        ds0 = [torch.empty((B, D), dtype=torch.float32, device=dev) for _ in range(S)]
        lam = ([torch.empty_strided((B, D, T), ss, dtype=torch.float32, device=dev)
                for _ in range(S)] if with_lambda else None)
        allocated = du + [da] + ds0 + (lam or [])
    _check_devices(dev, [("u", p) for p in u] + [("a", a)]
                   + [("initial state", x) for x in s0] + [("states", x) for x in s]
                   + [("upstream gradient", x) for x in gs]
                   + [("gs_end", x) for x in (gs_end or [])] + [("workspace", workspace)])
    _record_on(stream, allocated)
    shape = make_shape(B, T, D, us, ss)
    newton = make_newton(0.0, 0, steps_per_lane, waves_per_block)
    nws = workspace_bytes(cell, shape, newton, adjoint=True)
    ws = workspace if workspace is not None else _ws.get(nws, dev, stream)
    _check(lib.pararnn_adjoint(cell, ctypes.byref(shape), _ptr_array(u), _u_dtype(u), _ptr(a),
                               _ptr_array(s0), _ptr_array(s), _ptr_array(gs),
                               _ptr_array(gs_end) if gs_end is not None else None,
                               _ptr_array(du), _ptr(da), 1 if da_accumulate else 0,
                               _ptr_array(ds0),
                               _ptr_array(lam) if lam is not None else None,
                               ctypes.byref(newton), _ptr(ws), 0 if ws is None else ws.numel(),
                               _stream_handle(stream)))
    return dict(du=du, da=da, ds0=ds0, lam=lam)


def project(x, w, bias=None, *, out=None, out_dtype=torch.float32, stream=None):
    """Input projection u[b][m][t] = sum_k w[m][k] x[b][t][k] + bias[m] on
    the matrix cores.  x [B][T][I] and w [M][I] bfloat16 with the last (k)
    dimension contiguous; bias float32 [M] or None.  Returns u [B][M][T]
    (float32 or bfloat16); for M = G*D, u[:, g*D:(g+1)*D] is gate g's plane
    for the solves."""
    lib = load()
    if x.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise ValueError("x and w must be bfloat16")
    if x.dim() != 3 or w.dim() != 2 or x.shape[2] != w.shape[1]:
        raise ValueError("x [B][T][I] and w [M][I] with matching I")
    if (x.numel() and x.stride(2) != 1) or (w.numel() and w.stride(1) != 1):
        raise ValueError("x and w must be contiguous along I")
    B, T, I = x.shape
    M = w.shape[0]
    if bias is not None and (bias.dtype != torch.float32 or tuple(bias.shape) != (M,)
                             or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous float32 [M]")
    allocated = []
    if out is None:
        out = torch.empty((B, M, T), dtype=out_dtype, device=x.device)
        allocated = [out]
    if tuple(out.shape) != (B, M, T) or out.dtype not in (torch.float32, torch.bfloat16) or (
            out.numel() and out.stride(2) != 1):
        raise ValueError("out must be [B][M][T] float32 or bfloat16, time contiguous")
    _check_devices(x.device, [("w", w), ("bias", bias), ("out", out)])
    _record_on(stream, allocated)
    # strides of size-1 dimensions are arbitrary in torch: use dense ones
    xst = x.stride(1) if T > 1 else I
    usm = out.stride(1) if M > 1 else T
    sh = ProjShape(B, T, I, M, x.stride(0) if B > 1 else xst * T, xst,
                   w.stride(0) if M > 1 else I, out.stride(0) if B > 1 else usm * M, usm)
    dt = BF16 if out.dtype == torch.bfloat16 else F32
    _check(lib.pararnn_project(ctypes.byref(sh), _ptr(x), _ptr(w), _ptr(bias), _ptr(out), dt,
                               _stream_handle(stream)))
    return out


def sequential(cell, u, a, s0, *, out=None, stream=None):
    """Step-by-step application s_t = f(s_{t-1}, u_t), one lane per channel
    (no Newton iteration).  cell "gru" (s0: [h0]) or "lstm" ([c0, h0]); u as
    for the solves.  Returns the S state planes [B][D][T] (float32)."""
    lib = load()
    _require(cell in CELLS or cell in (GRU, LSTM), f"unknown cell {cell!r}")
    cell = CELLS.get(cell, cell)
    G, S = N_GATES[cell], N_STATES[cell]
    u, s0 = list(u), list(s0)
    _require(len(u) == G and len(s0) == S, "wrong number of gate or state planes")
    B, D, T = _plane_dims(u, "u")
    _check_planes(u, "u", (B, D, T), _U_DTYPES)
    _u_dtype(u)
    _check_dense(a, "a", (G, D))
    for i, x in enumerate(s0):
        _check_dense(x, f"initial state {i}", (B, D))
    dev = u[0].device
    us = _strides(u, "u") or (D * T, T, 1)
    allocated = []
    if out is None:
        out = _new_planes(S, B, T, D, us, dev)
        allocated = out
    out = list(out)
    _require(len(out) == S, "out must be S float32 planes [B][D][T]")
    _check_planes(out, "out", (B, D, T))
    ss = _strides(out, "states") or (D * T, T, 1)
    _check_devices(dev, [("u", p) for p in u] + [("a", a)]
                   + [("initial state", x) for x in s0] + [("out", x) for x in out])
    _record_on(stream, allocated)
    shape = make_shape(B, T, D, us, ss)
    _check(lib.pararnn_sequential(cell, ctypes.byref(shape), _ptr_array(u), _u_dtype(u), _ptr(a),
                                  _ptr_array(s0), _ptr_array(out), _stream_handle(stream)))
    return out


def scan(A, b, x0=None, *, reverse=False, out=None, steps_per_lane=0, waves_per_block=0,
         workspace=None, stream=None):
    """Linear recurrence x_t = A_t x_{t-1} + b_t (or, reversed, x_t = A_t
    x_{t+1} + b_t) per channel.  A: S*S float32 planes [B][D][T] (2x2 blocks
    row-major), b: S planes, x0: None or S [B][D] boundary values.  Returns
    the S planes of x."""
    lib = load()
    A, b = list(A), list(b)
    S = len(b)
    _require(S in (1, 2) and len(A) == S * S,
             "state size must be 1 or 2 (A has S*S planes, b has S)")
    B, D, T = _plane_dims(A + b, "A/b")
    _check_planes(A + b, "A/b", (B, D, T))
    if x0 is not None:
        x0 = list(x0)
        _require(len(x0) == S, "x0: one [B][D] plane per state component")
        for i, x in enumerate(x0):
            _check_dense(x, f"x0[{i}]", (B, D))
    dev = b[0].device
    ins = _strides(A + b, "A/b") or (D * T, T, 1)
    allocated = []
    if out is None:
        out = _new_planes(S, B, T, D, ins, dev)
        allocated = out
    out = list(out)
    _require(len(out) == S, "out: one plane per state component")
    _check_planes(out, "x", (B, D, T))
    outs = _strides(out, "x") or (D * T, T, 1)
    _check_devices(dev, [("A/b", p) for p in A + b] + [("x0", x) for x in (x0 or [])]
                   + [("x", x) for x in out] + [("workspace", workspace)])
    _record_on(stream, allocated)
    shape = make_shape(B, T, D, ins, outs)
    newton = make_newton(0.0, 0, steps_per_lane, waves_per_block)
    nws = int(lib.pararnn_scan_workspace_bytes(S, ctypes.byref(shape), ctypes.byref(newton)))
    ws = workspace if workspace is not None else _ws.get(nws, dev, stream)
    _check(lib.pararnn_scan(S, ctypes.byref(shape), _ptr_array(A), _ptr_array(b),
                            _ptr_array(x0) if x0 is not None else None, _ptr_array(out),
                            1 if reverse else 0, ctypes.byref(newton), _ptr(ws),
                            0 if ws is None else ws.numel(), _stream_handle(stream)))
    return out
