"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/pararnn.h declares, plans tilings, sizes workspaces
and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

from nonlinear_rnn_amd import pararnn as pr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pararnn.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(pararnn_[a-z_0-9]+)\s*\(", txt)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ["pararnn_solve_gru", "pararnn_solve_lstm", "pararnn_adjoint",
              "pararnn_workspace_bytes", "pararnn_status_string", "pararnn_plan"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = pr.load()
    for n in _declared():
        assert hasattr(lib, n), n


def test_library_exports_no_undeclared_c_functions():
    """Every C-linkage function the library defines is one the header
    declares: internal helpers stay out of the exported name space."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--defined-only", pr.LIB_PATH], check=True,
                         stdout=subprocess.PIPE, text=True).stdout
    funcs = sorted({ln.split()[2] for ln in out.splitlines()
                    if len(ln.split()) == 3 and ln.split()[1] == "T"
                    and not ln.split()[2].startswith("_")})
    assert funcs == _declared()


def test_status_strings():
    assert pr.status_string(0) == "ok"
    for s in range(1, 6):
        assert pr.status_string(s) != "ok"
    assert "static" in pr.status_string(5)
    assert "unknown" in pr.status_string(99)


def test_plan_defaults():
    # one workgroup per channel up to 4096 steps, then time blocks
    assert pr.plan("gru", pr.make_shape(8, 4096, 1024)) == (16, 4, 1)
    assert pr.plan("gru", pr.make_shape(4, 16384, 4096)) == (16, 4, 4)
    # few channels: each spread over more waves at the same capacity
    assert pr.plan("gru", pr.make_shape(1, 1024, 64)) == (4, 4, 1)
    assert pr.plan("gru", pr.make_shape(1, 4096, 64)) == (8, 8, 1)
    assert pr.plan("gru", pr.make_shape(1, 4096, 64), adjoint=True) == (8, 4, 2)  # unchanged
    assert pr.plan("gru", pr.make_shape(1, 1, 64)) == (1, 1, 1)
    assert pr.plan("lstm", pr.make_shape(8, 4096, 1024)) == (16, 4, 1)
    assert pr.plan("lstm", pr.make_shape(16, 2048, 4096)) == (16, 2, 1)
    assert pr.plan("lstm", pr.make_shape(16, 2048, 4096), adjoint=True) == (8, 4, 1)
    # forced tiling, ragged T
    n = pr.make_newton(steps_per_lane=1, waves_per_block=1)
    assert pr.plan("gru", pr.make_shape(2, 3 * 64 + 7, 3), n) == (1, 1, 4)


@pytest.mark.parametrize("K,W", [(3, 1), (64, 1), (1, 16), (1, 3), (-1, 1), (32, 4)])
def test_plan_rejects_unsupported_tiling(K, W):
    n = pr.make_newton(steps_per_lane=K, waves_per_block=W)
    with pytest.raises(pr.PararnnError) as e:
        pr.plan("gru", pr.make_shape(1, 100, 1), n)
    assert e.value.status == 2


def test_wide_lane_tiling_is_gru_forward_only():
    n = pr.make_newton(steps_per_lane=32, waves_per_block=2)
    assert pr.plan("gru", pr.make_shape(1, 4096, 1), n) == (32, 2, 1)
    for cell, adj in [("lstm", False), ("gru", True), ("lstm", True)]:
        with pytest.raises(pr.PararnnError) as e:
            pr.plan(cell, pr.make_shape(1, 4096, 1), n, adjoint=adj)
        assert e.value.status == 2


def test_workspace_sizes():
    n = pr.make_newton(1e-6, 20)
    # one block per channel: only the per-unit convergence records
    assert pr.workspace_bytes("gru", pr.make_shape(8, 4096, 1024), n) == 8192 * 8
    # 16,384 channels of four 4096-step blocks, solved block-sequentially
    # inside one workgroup a channel: no hand-off, only the per-unit records
    units = 4 * 4096 * 4
    assert pr.plan("gru", pr.make_shape(4, 16384, 4096)) == (16, 4, 4)
    for cell in ("gru", "lstm"):
        for init in (False, True):
            assert pr.workspace_bytes(cell, pr.make_shape(4, 16384, 4096),
                                      pr.make_newton(1e-6, 20, init_from_output=init)) == units * 8
    # 64 channels: the blocks run side by side and exchange carries (flags,
    # per-iteration records of S + S^2 + 1 floats, boundary states of a warm
    # start)
    sh = pr.make_shape(1, 16384, 64)
    few = 64 * 4
    assert pr.plan("gru", sh) == (16, 4, 4)
    ws = pr.workspace_bytes("gru", sh, n)
    assert ws >= few * 4 + few * 21 * 3 * 4 + few * 8
    ws2 = pr.workspace_bytes("gru", sh, pr.make_newton(1e-6, 20, init_from_output=True))
    assert ws2 >= ws + few * 4
    assert pr.workspace_bytes("lstm", sh, n) > ws
    wa = pr.workspace_bytes("lstm", pr.make_shape(16, 2048, 4096), n, adjoint=True)
    assert wa >= 16 * 4096 * 4 * 4
    assert pr.workspace_bytes(7, pr.make_shape(1, 1, 1), n) == 0


def test_workspace_includes_staging_for_time_major_planes():
    """Planes that are not time-contiguous get room to be staged channel-major
    (projections at 4 bytes per element, states at 4); channel-major planes
    need none."""
    n = pr.make_newton(1e-6, 20)
    B, T, D = 8, 4096, 1024
    N = B * T * D
    dense = pr.workspace_bytes("gru", pr.make_shape(B, T, D), n)
    tm_u = pr.workspace_bytes("gru", pr.make_shape(B, T, D, (T * 3 * D, 1, 3 * D)), n)
    tm_both = pr.workspace_bytes("lstm", pr.make_shape(B, T, D, (T * 4 * D, 1, 4 * D),
                                                       (T * D, 1, D)), n)
    assert dense == B * D * 8  # the per-unit convergence records only
    assert dense + 3 * N * 4 <= tm_u < dense + 3 * N * 4 + 4096
    assert dense + 4 * N * 4 + 2 * N * 4 <= tm_both < dense + 6 * N * 4 + 4096
    assert pr.workspace_bytes("gru", pr.make_shape(B, 1, D, (3 * D, 1, 3 * D)), n) == B * D * 8
    # the adjoint stages u and dL/du (u-family), s, dL/ds and lambda (s-family)
    adj_dense = pr.workspace_bytes("lstm", pr.make_shape(B, T, D), n, adjoint=True)
    adj_tm = pr.workspace_bytes("lstm", pr.make_shape(B, T, D, (T * 4 * D, 1, 4 * D),
                                                      (T * D, 1, D)), n, adjoint=True)
    assert adj_dense + 14 * N * 4 <= adj_tm < adj_dense + 14 * N * 4 + 8192


def test_scan_keeps_channels_in_one_workgroup_up_to_8192_steps():
    """The standalone scan's default tiling: no time blocks (workspace 0) up
    to 8192 steps, then 8192-step blocks with records and flags."""
    lib = pr.load()
    n = pr.make_newton(0.0, 0)
    for S in (1, 2):
        for T in (1, 4096, 8192):
            sh = pr.make_shape(2, T, 3)
            assert lib.pararnn_scan_workspace_bytes(S, ctypes.byref(sh), ctypes.byref(n)) == 0
        sh = pr.make_shape(2, 8193, 3)
        assert lib.pararnn_scan_workspace_bytes(S, ctypes.byref(sh), ctypes.byref(n)) > 0
    assert lib.pararnn_scan_workspace_bytes(3, ctypes.byref(pr.make_shape(2, 9000, 3)),
                                            ctypes.byref(n)) == 0


def test_plane_layouts_accepted_and_rejected():
    """Any non-overlapping (stride_b, stride_d, stride_t) is a valid plane
    layout: channel-major, time-major [B][T][D], interleaved gate blocks of a
    [B][T][G*D] tensor, padded and permuted ones; overlapping ones are
    rejected before any device work."""
    def ok(us, ss=None, B=2, T=16, D=3):
        try:
            pr.plan("gru", pr.make_shape(B, T, D, us, ss))
            return True
        except pr.PararnnError as e:
            assert e.status == 1
            return False

    assert ok((48, 16, 1))                       # channel-major
    assert ok((48, 1, 3), (48, 1, 3))            # time-major [B][T][D]
    assert ok((144, 1, 9))                       # a gate block of [B][T][3*D]
    assert ok((100, 1, 5))                       # padded rows
    assert ok((1, 32, 2))                        # b fastest, then t, then d
    assert ok((0, 16, 1), B=1)                   # extent-1 dimensions are free
    assert ok((48, 1, 3), T=1, D=3)
    assert not ok((48, 1, 2))                    # steps overlap channels
    assert not ok((47, 1, 3))                    # batch rows overlap
    assert not ok((48, 16, 0))                   # every step at one address
    assert not ok((48, 1, 3), (48, 3, 1))        # the states' d and t overlap
    assert not ok((48, 16, -1))
    assert not ok((2 ** 62 + 16, 2 ** 61, 1))    # offsets past int64


def _call_gru(shape, newton, u=(1, 1, 1), a=1, h0=1, h=1, ws=None, nws=0, info=None):
    lib = pr.load()
    arr = (ctypes.c_void_p * 3)(*[x or None for x in u])
    return lib.pararnn_solve_gru(ctypes.byref(shape) if shape is not None else None, arr, 0,
                                 a, h0, h, ctypes.byref(newton) if newton else None, info,
                                 ws, nws, None)


def test_solve_rejects_bad_arguments_before_any_device_call():
    good = pr.make_shape(2, 16, 3)
    n = pr.make_newton(1e-6, 5)
    assert _call_gru(None, n) == 1
    assert _call_gru(good, None) == 1
    assert _call_gru(pr.make_shape(-1, 16, 3), n) == 1
    assert _call_gru(pr.make_shape(2, 16, 3, (48, 8)), n) == 1       # rows overlap
    assert _call_gru(pr.make_shape(2, 16, 3, None, (-48, 16)), n) == 1
    assert _call_gru(good, pr.make_newton(float("nan"), 5)) == 1
    assert _call_gru(good, pr.make_newton(-1.0, 5)) == 1
    assert _call_gru(good, pr.make_newton(float("inf"), 5)) == 1
    assert _call_gru(good, pr.make_newton(1e-6, -1)) == 1
    assert _call_gru(good, pr.make_newton(1e-6, 5, steps_per_lane=5)) == 2
    assert _call_gru(good, n, u=(1, 0, 1)) == 1
    assert _call_gru(good, n, a=None) == 1
    assert _call_gru(good, n, h=None) == 1
    # several time blocks need a workspace
    nb = pr.make_newton(1e-6, 5, steps_per_lane=1, waves_per_block=1)
    big = pr.make_shape(2, 200, 3)
    assert _call_gru(big, nb) == 3
    need = pr.workspace_bytes("gru", big, nb)
    assert _call_gru(big, nb, ws=16, nws=need - 1, info=16) == 3
    units_big = 2 * 3 * 4
    assert _call_gru(big, nb, ws=16, nws=need - 256 * ((units_big * 8 + 255) // 256) - 1) == 3
    assert _call_gru(big, nb, ws=8, nws=need) == 3                     # misaligned
    # an info record is folded from per-unit records kept in the workspace
    units = 2 * 3
    assert pr.workspace_bytes("gru", good, n) == 256 * ((units * 8 + 255) // 256)
    assert _call_gru(good, n, info=16) == 3
    assert _call_gru(good, n, info=16, ws=16, nws=units * 8 - 1) == 3


def test_lstm_and_adjoint_reject_bad_arguments():
    lib = pr.load()
    shape = pr.make_shape(1, 8, 2)
    n = pr.make_newton(1e-6, 5)
    u = (ctypes.c_void_p * 4)(1, 1, 1, 1)
    assert lib.pararnn_solve_lstm(ctypes.byref(shape), u, 0, 1, 1, None, 1, 1,
                                  ctypes.byref(n), None, None, 0, None) == 1
    assert lib.pararnn_solve_lstm(ctypes.byref(shape), u, 5, 1, 1, 1, 1, 1,
                                  ctypes.byref(n), None, None, 0, None) == 2
    s2 = (ctypes.c_void_p * 2)(1, 1)
    assert lib.pararnn_adjoint(3, ctypes.byref(shape), u, 0, 1, s2, s2, s2, None, u, 1, 0, s2,
                               None, None, None, 0, None) == 1
    assert lib.pararnn_adjoint(1, ctypes.byref(shape), u, 0, 1, s2, s2, s2, None, u, 1, 0, s2,
                               None, None, None, 0, None) == 3
    assert lib.pararnn_adjoint(1, ctypes.byref(shape), u, 0, None, s2, s2, s2, None, u, 1, 0, s2,
                               None, None, None, 0, None) == 1
    # da_accumulate is a 0/1 flag
    assert lib.pararnn_adjoint(1, ctypes.byref(shape), u, 0, 1, s2, s2, s2, s2, u, 1, 2, s2,
                               None, None, None, 0, None) == 1


def test_sequential_rejects_bad_arguments_before_any_device_call():
    lib = pr.load()
    sh = pr.make_shape(2, 16, 3)
    one = ctypes.c_void_p(16)
    u = (ctypes.c_void_p * 4)(one, one, one, one)
    s = (ctypes.c_void_p * 2)(one, one)
    assert lib.pararnn_sequential(7, ctypes.byref(sh), u, 0, one, s, s, None) == 1
    assert lib.pararnn_sequential(0, None, u, 0, one, s, s, None) == 1
    assert lib.pararnn_sequential(0, ctypes.byref(sh), u, 5, one, s, s, None) == 2
    assert lib.pararnn_sequential(0, ctypes.byref(sh), None, 0, one, s, s, None) == 1
    assert lib.pararnn_sequential(1, ctypes.byref(sh), u, 0, None, s, s, None) == 1
    nul = (ctypes.c_void_p * 2)(one, None)
    assert lib.pararnn_sequential(1, ctypes.byref(sh), u, 0, one, s, nul, None) == 1
    bad = pr.make_shape(2, 16, 3, (10, 16), (48, 16))  # overlapping rows
    assert lib.pararnn_sequential(0, ctypes.byref(bad), u, 0, one, s, s, None) == 1
    empty = pr.make_shape(0, 16, 3)
    assert lib.pararnn_sequential(0, ctypes.byref(empty), None, 0, None, None, None, None) == 0


def test_project_rejects_bad_arguments_before_any_device_call():
    lib = pr.load()
    one = ctypes.c_void_p(16)

    def call(sh, dt=0, x=one, w=one, u=one):
        return lib.pararnn_project(ctypes.byref(sh) if sh is not None else None, x, w, None, u,
                                   dt, None)

    good = pr.ProjShape(2, 8, 4, 6, 32, 4, 4, 48, 8)
    assert call(None) == 1
    assert call(pr.ProjShape(-1, 8, 4, 6, 32, 4, 4, 48, 8)) == 1
    assert call(good, dt=7) == 2
    assert call(pr.ProjShape(2, 8, 4, 6, 32, 3, 4, 48, 8)) == 1   # x rows overlap
    assert call(pr.ProjShape(2, 8, 4, 6, 31, 4, 4, 48, 8)) == 1   # x batches overlap
    assert call(pr.ProjShape(2, 8, 4, 6, 32, 4, 3, 48, 8)) == 1   # W rows overlap
    assert call(pr.ProjShape(2, 8, 4, 6, 32, 4, 4, 47, 8)) == 1   # u batches overlap
    assert call(good, x=None) == 1
    assert call(good, u=None) == 1
    assert call(pr.ProjShape(0, 8, 4, 6, 32, 4, 4, 48, 8), x=None, w=None, u=None) == 0


def test_workspace_cache_is_per_stream_and_bounded(monkeypatch):
    """Host logic of the binding's default workspace: one buffer per
    (device, stream), reused while large enough, regrown when not, and only
    the most recently used streams keep one."""
    import contextlib

    import torch
    monkeypatch.setattr(torch.cuda, "stream", lambda s: contextlib.nullcontext())

    class Stream:
        def __init__(self, handle):
            self.cuda_stream = handle

    ws = pr.Workspace()
    a = ws.get(64, "cpu", Stream(1))
    assert ws.get(32, "cpu", Stream(1)) is a          # reused
    assert ws.get(64, "cpu", Stream(2)) is not a      # another stream, another buffer
    bigger = ws.get(128, "cpu", Stream(1))
    assert bigger is not a and bigger.numel() == 128  # regrown
    assert ws.get(0, "cpu", Stream(1)) is None
    for h in range(100, 100 + 2 * pr.Workspace.MAX_STREAMS):
        ws.get(16, "cpu", Stream(h))
    assert len(ws.buf) == pr.Workspace.MAX_STREAMS
    assert (None, 1) not in ws.buf                    # oldest streams dropped


def test_kernel_digest_ignores_comments_and_layout():
    """Traffic records stay valid across documentation edits: the digest
    that ties them to the kernel sources hashes code only."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    a = bench._code_only("int f(int x) {  // add one\n    return x + 1; /* the\n result */\n}\n")
    b = bench._code_only("/* doc */\nint f(int x) {\n\n  return x + 1;\n}")
    assert a == b
    assert a != bench._code_only("int f(int x) { return x + 2; }")


def test_binding_rejects_bad_tensors_before_any_call():
    """The binding checks dtype, shape, layout and device of every tensor
    before calling the library (a float64 output or a 1-d weight vector
    would otherwise be written or read out of bounds by the kernels).  Here,
    on the CPU, every case must raise ValueError; the last one reaches the
    device check, since CPU memory is not device memory."""
    import torch

    B, D, T = 2, 3, 16
    f32 = dict(dtype=torch.float32)

    def planes(n, shape=(B, D, T), **kw):
        return [torch.zeros(shape, **(kw or f32)) for _ in range(n)]

    u, a, h0 = planes(3), torch.zeros(3, D), torch.zeros(B, D)
    out = torch.zeros(B, D, T)
    bad = [
        dict(u=planes(2)),                                          # gate count
        dict(u=planes(2) + [torch.zeros(B, D, T + 1)]),             # unequal planes
        dict(u=[torch.zeros(B * D * T)] * 3),                       # not [B][D][T]
        dict(u=planes(3, dtype=torch.float64)),                     # dtype
        dict(u=planes(2) + planes(1, dtype=torch.bfloat16)),        # mixed dtypes
        dict(a=torch.zeros(3 * D)),                                 # 1-d weights
        dict(a=torch.zeros(D, 3).t()),                              # non-contiguous
        dict(a=torch.zeros(3, D, dtype=torch.float64)),
        dict(h0=torch.zeros(D, B).t()),                             # transposed h0
        dict(h0=torch.zeros(B + 1, D)),
        dict(out=torch.zeros(B, D, T, dtype=torch.bfloat16)),       # output dtype
        dict(out=torch.zeros(B, D, T, dtype=torch.float64)),
        dict(out=torch.zeros(B, D, T - 1)),
        dict(),                                                     # CPU tensors
    ]
    for case in bad:
        kw = dict(u=u, a=a, h0=h0, out=out)
        kw.update(case)
        with pytest.raises(ValueError):
            pr.solve_gru(kw["u"], kw["a"], kw["h0"], out=kw["out"])
    with pytest.raises(ValueError):
        pr.solve_lstm(planes(4), torch.zeros(4, D), h0, torch.zeros(B, D, dtype=torch.float64))
    with pytest.raises(ValueError):
        pr.solve_gru(u, a, h0, init_from_output=True)
    # adjoint: states, upstream gradients, weights
    s, g = planes(1), planes(1)
    for case in [dict(s=planes(1, shape=(B, D, T - 1))), dict(gs=planes(1, dtype=torch.float64)),
                 dict(a=torch.zeros(3, D + 1)), dict(s0=[torch.zeros(B, D, 1)]), dict()]:
        kw = dict(u=u, a=a, s0=[h0], s=s, gs=g)
        kw.update(case)
        with pytest.raises(ValueError):
            pr.adjoint("gru", kw["u"], kw["a"], kw["s0"], kw["s"], kw["gs"])
    with pytest.raises(ValueError):
        pr.adjoint("tanh", u, a, [h0], s, g)
    # sequential and scan
    for case in [dict(a=torch.zeros(2, D)), dict(out=planes(1, dtype=torch.float64)), dict()]:
        kw = dict(a=a, out=planes(1))
        kw.update(case)
        with pytest.raises(ValueError):
            pr.sequential("gru", u, kw["a"], [h0], out=kw["out"])
    for case in [dict(A=planes(2)), dict(b=planes(1, dtype=torch.float64)),
                 dict(x0=[torch.zeros(B, D + 1)]), dict()]:
        kw = dict(A=planes(1), b=planes(1), x0=None)
        kw.update(case)
        with pytest.raises(ValueError):
            pr.scan(kw["A"], kw["b"], kw["x0"])


def test_static_scratch_solve_rejects_oversized_problems_before_any_device_call():
    """The allocation-free solve sizes its workspace on the host: a problem
    whose time-block records exceed the static array returns
    PARARNN_ERR_SCRATCH (5) before any HIP call, and so do bad arguments."""
    lib = pr.load()
    hdr = open(HEADER).read()
    assert re.search(r"#define PARARNN_STATIC_SCRATCH_BYTES \(32u << 20\)", hdr)
    assert pr.STATIC_SCRATCH_BYTES == 32 << 20
    one = ctypes.c_void_p(256)
    u = (ctypes.c_void_p * 3)(one, one, one)
    # 1024 channels x 1024 time blocks of 64 steps, 21 records each: 336 MB
    big = pr.make_shape(1, 65536, 1024)
    n = pr.make_newton(1e-6, 20, steps_per_lane=1, waves_per_block=1)
    assert pr.workspace_bytes("gru", big, n) > pr.STATIC_SCRATCH_BYTES
    assert lib.pararnn_solve_gru_noalloc(ctypes.byref(big), u, 0, one, one, one, ctypes.byref(n),
                                         None, None) == 5
    assert lib.pararnn_solve_gru_noalloc(None, u, 0, one, one, one, ctypes.byref(n),
                                         None, None) == 1
    assert lib.pararnn_solve_gru_noalloc(ctypes.byref(big), u, 0, one, one, one, None,
                                         None, None) == 1
    bad = pr.make_newton(1e-6, 20, steps_per_lane=3)
    assert lib.pararnn_solve_gru_noalloc(ctypes.byref(big), u, 0, one, one, one,
                                         ctypes.byref(bad), None, None) == 2
