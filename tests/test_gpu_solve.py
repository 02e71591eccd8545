"""GPU parity of the fused Newton solve (HIP path through the C ABI) against
the CPU oracle, plus the invariants the pages fix.

Tolerances: 1e-5 max-abs for float32 states; for bf16 projections the gate is
2e-2 against the oracle on the unrounded float32 draw, with a 1e-5
diagnostic against the oracle on the rounded values (what the device sees).
"""
import numpy as np
import pytest
import torch

from nonlinear_rnn_amd.inputs import make_inputs
from oracle import deer
from tests.gpu_util import gpu_solve, max_err, oracle_states

pytestmark = pytest.mark.gpu

TOL32 = 1e-5

TILINGS = [(0, 0), (1, 1), (2, 2), (4, 1), (16, 4), (8, 8)]


@pytest.mark.parametrize("cell", ["gru", "lstm"])
@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 200, 1000, 4100])
@pytest.mark.parametrize("KW", TILINGS)
def test_parity_small(cell, T, KW):
    K, W = KW
    inp = make_inputs(cell, 2, T, 3, 1000 + T, s0_std=0.1, f_bias=1.0)
    got, info = gpu_solve(inp, 1e-6, 40, K, W)
    ref = oracle_states(inp)
    assert info["converged"], info
    assert info["max_abs_res"] < 1e-6
    assert max_err(got, ref) < TOL32


@pytest.mark.parametrize("cell", ["gru", "lstm"])
@pytest.mark.parametrize("T,KW", [(96, (1, 1)), (1000, (1, 1)), (517, (2, 1)), (4100, (4, 4))])
def test_parity_bf16_inputs(cell, T, KW):
    inp = make_inputs(cell, 2, T, 5, 2000 + T, u_dtype="bf16", f_bias=1.0)
    got, info = gpu_solve(inp, 1e-6, 40, *KW)
    assert info["converged"]
    assert max_err(got, oracle_states(inp, rounded=True)) < TOL32
    assert max_err(got, oracle_states(inp, rounded=False)) < 2e-2


@pytest.mark.parametrize("cell", ["gru", "lstm"])
@pytest.mark.parametrize("KW", [(1, 1), (2, 2), (0, 0)])
@pytest.mark.parametrize("iters", [1, 2, 3])
def test_per_iteration_parity_with_deer(cell, KW, iters):
    """tol = 0 forces exactly `iters` updates everywhere; the iterate must be
    the DEER iterate of the numpy oracle (same start s = 0)."""
    inp = make_inputs(cell, 1, 300, 4, 3000 + iters, s0_std=0.3, f_bias=1.0)
    got, info = gpu_solve(inp, 0.0, iters, *KW)
    assert info["iters"] == iters and not info["converged"]
    u = deer.from_planes(inp.u)
    a = deer.a_per_channel(inp.a, 1)
    s0 = np.stack([p.reshape(-1).astype(np.float64) for p in inp.s0], -1)
    s, _ = deer.newton(cell, u, a, s0, tol=0.0, max_iters=iters)
    ref = [s[..., c].reshape(1, 4, 300) for c in range(s.shape[-1])]
    scale = max(1.0, max(float(np.abs(r).max()) for r in ref))
    assert max_err(got, ref) < 1e-4 * scale


@pytest.mark.parametrize("cell", ["gru", "lstm"])
@pytest.mark.parametrize("W", [1, 2, 4])
@pytest.mark.parametrize("iters", [1, 3])
def test_per_iteration_parity_full_single_blocks(cell, W, iters):
    """The same on full one-block-per-channel tiles (K = 16, T = 1024 W):
    the kernels that take the zero-start pass (ParaGRU) and keep three
    gates' projections in LDS (ParaLSTM)."""
    T = 64 * 16 * W
    inp = make_inputs(cell, 1, T, 4, 3100 + 10 * W + iters, s0_std=0.3, f_bias=1.0)
    got, info = gpu_solve(inp, 0.0, iters, 16, W)
    assert info["iters"] == iters and not info["converged"] and info["units"] == 4
    u = deer.from_planes(inp.u)
    a = deer.a_per_channel(inp.a, 1)
    s0 = np.stack([p.reshape(-1).astype(np.float64) for p in inp.s0], -1)
    s, _ = deer.newton(cell, u, a, s0, tol=0.0, max_iters=iters)
    ref = [s[..., c].reshape(1, 4, T) for c in range(s.shape[-1])]
    scale = max(1.0, max(float(np.abs(r).max()) for r in ref))
    assert max_err(got, ref) < 1e-4 * scale


def test_linear_gru_converges_in_one_update():
    inp = make_inputs("gru", 2, 3000, 8, 41, s0_std=0.5)
    inp.a[:] = 0
    got, info = gpu_solve(inp, 1e-6, 20)
    assert info["converged"] and info["iters"] == 1
    assert max_err(got, oracle_states(inp)) < TOL32


def test_linear_lstm_converges_in_two_updates():
    inp = make_inputs("lstm", 2, 3000, 8, 42, s0_std=0.5, f_bias=1.0)
    inp.a[:] = 0
    got, info = gpu_solve(inp, 1e-6, 20)
    assert info["converged"] and info["iters"] == 2
    assert max_err(got, oracle_states(inp)) < TOL32


@pytest.mark.parametrize("cell", ["gru", "lstm"])
@pytest.mark.parametrize("k", [1, 2, 3])
def test_prefix_exact_after_k_updates_stiff(cell, k):
    """After k updates from s = 0 the first k states are the exact ones, even
    for a stiff cell (a ~ U(-4, 4))."""
    inp = make_inputs(cell, 1, 256, 6, 50 + k, f_bias=1.0, a_scale=4.0, u_scale=2.0)
    got, info = gpu_solve(inp, 0.0, k, 1, 1)
    ref = oracle_states(inp)
    assert max_err([g[..., :k] for g in got], [r[..., :k] for r in ref]) < TOL32


@pytest.mark.parametrize("KW", [(0, 0), (1, 1)])
def test_tol_zero_runs_to_cap(KW):
    inp = make_inputs("gru", 1, 500, 4, 61)
    got, info = gpu_solve(inp, 0.0, 7, *KW)
    assert info["iters"] == 7 and not info["converged"] and not info["nan_seen"]
    assert info["iters_sum"] == 7 * info["units"]


@pytest.mark.parametrize("cell", ["gru", "lstm"])
@pytest.mark.parametrize("KW", [(0, 0), (1, 1)])
def test_nan_input_is_reported(cell, KW):
    inp = make_inputs(cell, 2, 400, 3, 71, f_bias=1.0)
    inp.u[0][1, 2, 123] = np.nan
    got, info = gpu_solve(inp, 1e-6, 10, *KW)
    assert info["nan_seen"] and not info["converged"]
    assert np.isnan(info["max_abs_res"])
    ref = oracle_states(inp)
    # every other channel is unaffected
    for g, r in zip(got, ref):
        g, r = g.copy(), r.copy()
        g[1, 2] = 0
        r[1, 2] = 0
        assert np.max(np.abs(g - r)) < TOL32
    assert np.isnan(got[-1][1, 2, 123:]).all()


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_bitwise_deterministic(cell):
    inp = make_inputs(cell, 2, 5000, 16, 81, f_bias=1.0)
    a, ia = gpu_solve(inp, 1e-6, 20, 2, 2)
    b, ib = gpu_solve(inp, 1e-6, 20, 2, 2)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    assert ia == ib


@pytest.mark.parametrize("cell", ["gru", "lstm"])
@pytest.mark.parametrize("KW", [(0, 0), (1, 1)])
def test_warm_start(cell, KW):
    inp = make_inputs(cell, 2, 700, 4, 91, s0_std=0.2, f_bias=1.0)
    ref = oracle_states(inp)
    start = [r.astype(np.float32) for r in ref]
    got, info = gpu_solve(inp, 1e-6, 20, *KW, init=start)
    assert info["iters"] == 0 and info["converged"]
    for g, s in zip(got, start):
        assert np.array_equal(g, s)
    # a perturbed start converges to the same trajectory
    rng = np.random.default_rng(5)
    pert = [s + rng.standard_normal(s.shape).astype(np.float32) * 0.05 for s in start]
    got, info = gpu_solve(inp, 1e-6, 20, *KW, init=pert)
    assert info["converged"] and info["iters"] >= 1
    assert max_err(got, ref) < TOL32


def test_empty_problems():
    for B, T, D in [(0, 10, 3), (2, 0, 3), (2, 10, 0)]:
        inp = make_inputs("gru", B, T, D, 1)
        got, info = gpu_solve(inp, 1e-6, 5)
        assert got[0].shape == (B, D, T)
        assert info["converged"] and info["iters"] == 0


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_channels_along_batch_only(cell):
    """D = 1: every channel is a batch row (257 of them, not a multiple of the
    8 XCDs, so some workgroups of the grid have no channel)."""
    inp = make_inputs(cell, 257, 300, 1, 4600, s0_std=0.2, f_bias=1.0)
    got, info = gpu_solve(inp, 1e-6, 30)
    assert info["converged"] and info["units"] == 257
    assert max_err(got, oracle_states(inp)) < TOL32


def test_strided_planes():
    """Planes that are views of larger buffers (row strides > T, not 16-byte
    multiples) take the scalar load path and give the same answer."""
    from nonlinear_rnn_amd import pararnn as pr
    inp = make_inputs("gru", 2, 301, 3, 97, s0_std=0.1)
    ref = oracle_states(inp)
    big = [torch.zeros((2, 3, 307), device="cuda") for _ in range(3)]
    for g in range(3):
        big[g][:, :, 2:303] = torch.from_numpy(inp.u[g]).cuda()
    u = [x[:, :, 2:303] for x in big]
    out_big = torch.zeros((2, 3, 305), device="cuda")
    out = out_big[:, :, 1:302]
    h, info = pr.solve_gru(u, torch.from_numpy(inp.a).cuda(), torch.from_numpy(inp.s0[0]).cuda(),
                           out=out, tol=1e-6, max_iters=20)
    assert pr.read_info(info)["converged"]
    assert max_err([out.cpu().numpy()], ref) < TOL32
    assert float(out_big[:, :, 0].abs().max()) == 0.0
    assert float(out_big[:, :, 302:].abs().max()) == 0.0


def test_runs_on_a_side_stream():
    inp = make_inputs("lstm", 2, 1500, 5, 99, f_bias=1.0)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        got, info = gpu_solve(inp, 1e-6, 20, stream=s)
    assert info["converged"]
    assert max_err(got, oracle_states(inp)) < TOL32


def test_concurrent_streams_keep_separate_workspaces():
    """Two multi-block solves (47 time blocks per channel, cross-block records
    in the workspace) in flight at once on two streams: the binding gives each
    stream its own workspace, and both match the oracle."""
    from nonlinear_rnn_amd import pararnn as pr
    from tests.gpu_util import dev_inputs
    inps = [make_inputs("gru", 2, 3000, 3, 4700 + i, s0_std=0.1) for i in range(2)]
    devs = [dev_inputs(inp) for inp in inps]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(2)]
    outs = []
    for (u, a, s0), st in zip(devs, streams):
        with torch.cuda.stream(st):
            h, info = pr.solve_gru(u, a, s0[0], tol=1e-6, max_iters=30, steps_per_lane=1,
                                   waves_per_block=1, stream=st)
        outs.append((h, info))
    torch.cuda.synchronize()
    for inp, (h, info) in zip(inps, outs):
        assert pr.read_info(info)["converged"]
        assert max_err([h.cpu().numpy()], oracle_states(inp)) < TOL32


@pytest.mark.parametrize("cell,dtype,T,KW", [
    ("gru", "f32", 512, (8, 1)), ("gru", "f32", 1024, (16, 1)), ("gru", "f32", 2048, (8, 4)),
    ("gru", "bf16", 1024, (16, 1)), ("gru", "bf16", 2048, (16, 2)),
    ("gru", "f32", 4096, (8, 8)),
    ("lstm", "f32", 512, (8, 1)), ("lstm", "f32", 1024, (16, 1)), ("lstm", "bf16", 1024, (16, 1)),
    ("lstm", "f32", 2048, (8, 4)),
])
def test_many_channels(cell, dtype, T, KW):
    """3000 channels: more workgroups than the device holds at once, so
    workgroups start as others retire; spot-checked against the sequential
    oracle on channels spread over the batch."""
    from oracle import sequential as seq
    inp = make_inputs(cell, 3, T, 1000, 1500 + T, u_dtype=dtype, s0_std=0.2, f_bias=1.0)
    got, info = gpu_solve(inp, 1e-6, 30, *KW)
    assert info["converged"] and info["units"] == 3000
    chans = [(0, 0), (2, 999), (1, 500), (0, 777), (2, 3), (1, 1)]
    u = inp.u_rounded
    sub_u, a_sub, s0_sub = seq.gather_channels(u, inp.a, inp.s0, chans)
    if cell == "gru":
        ref = [seq.gru_forward(sub_u, a_sub, s0_sub[0])[0]]
    else:
        ref = [x[0] for x in seq.lstm_forward(sub_u, a_sub, s0_sub[0], s0_sub[1])]
    bs = [c[0] for c in chans]
    ds = [c[1] for c in chans]
    assert max_err([g[bs, ds] for g in got], ref) < TOL32


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,W", [(2048, 2), (4096, 4)])
def test_vector_and_scalar_loads_agree(dtype, T, W):
    """ParaLSTM with one block per channel (T = 64 * 16 * W) and 2200
    channels: every channel matches the oracle, and the states are bitwise
    those of the same planes offset by one element, which the kernel reads
    step by step instead of in 16-byte vectors."""
    from nonlinear_rnn_amd import pararnn as pr
    from tests.gpu_util import dev_inputs
    B, D = 2, 1100
    assert pr.plan("lstm", pr.make_shape(B, T, D)) == (16, W, 1)
    inp = make_inputs("lstm", B, T, D, 5100 + T + len(dtype), u_dtype=dtype, s0_std=0.2,
                      f_bias=1.0)
    got, info = gpu_solve(inp, 1e-6, 30)
    assert info["converged"] and info["units"] == B * D
    assert max_err(got, oracle_states(inp, rounded=True)) < TOL32

    u, a, s0 = dev_inputs(inp)
    shifted = []
    for p in u:
        big = torch.zeros((B, D, T + 1), dtype=p.dtype, device=p.device)
        big[:, :, 1:] = p
        shifted.append(big[:, :, 1:])
    (c, h), info2 = pr.solve_lstm(shifted, a, s0[0], s0[1], tol=1e-6, max_iters=30)
    assert pr.read_info(info2)["iters_sum"] == info["iters_sum"]
    assert np.array_equal(c.cpu().numpy(), got[0]) and np.array_equal(h.cpu().numpy(), got[1])


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_long_sequence_default_tiling(cell):
    """Past 4096 steps: the default time blocks of 4096 steps, a ragged last
    block, bf16 and float32 projections."""
    from nonlinear_rnn_amd import pararnn as pr
    T = 17001
    K, W, nb = pr.plan(cell, pr.make_shape(2, T, 2))
    assert nb == -(-T // (64 * K * W)) and nb >= 3
    for dt in ("f32", "bf16"):
        inp = make_inputs(cell, 2, T, 2, 1700 + len(dt), u_dtype=dt, f_bias=1.0)
        got, info = gpu_solve(inp, 1e-6, 30)
        assert info["converged"] and info["units"] == 4 * nb
        assert max_err(got, oracle_states(inp, rounded=True)) < TOL32


def test_few_channels_long_sequence_default_tiling():
    """Few ParaGRU channels past 8 blocks of 4096 steps take 8192-step
    blocks (K = 16, W = 8), the last one ragged; float32 and bf16."""
    from nonlinear_rnn_amd import pararnn as pr
    T = 40000
    assert pr.plan("gru", pr.make_shape(1, T, 8)) == (16, 8, 5)
    for dt in ("f32", "bf16"):
        inp = make_inputs("gru", 1, T, 8, 4000 + len(dt), u_dtype=dt, s0_std=0.2)
        got, info = gpu_solve(inp, 1e-6, 30)
        assert info["converged"] and info["units"] == 8 * 5
        assert max_err(got, oracle_states(inp, rounded=True)) < TOL32


@pytest.mark.parametrize("cell", ["gru", "lstm"])
@pytest.mark.parametrize("cap", [2, 3, 4])
def test_time_blocks_stop_at_cap_after_a_guessed_last_pass(cell, cap):
    """Time blocks that reach the iteration cap on a residual-only pass (the
    guessed last evaluation: tol < max|r| < sqrt(tol)) still certify every
    record they stored, so successors reading carries iteration by iteration
    finish; the iterate is the oracle's DEER iterate after `cap` updates
    (blocks that stop earlier differ from it by less than tol)."""
    from nonlinear_rnn_amd import pararnn as pr
    T, D = 3000, 4
    inp = make_inputs(cell, 1, T, D, 900 + cap, s0_std=0.3, f_bias=1.0)
    K, W, nb = pr.plan(cell, pr.make_shape(1, T, D), pr.make_newton(1e-6, cap, 4, 1))
    assert nb == 12
    got, info = gpu_solve(inp, 1e-6, cap, 4, 1)
    assert info["iters"] == cap and info["units"] == D * nb
    u = deer.from_planes(inp.u)
    a = deer.a_per_channel(inp.a, 1)
    s0 = np.stack([p.reshape(-1).astype(np.float64) for p in inp.s0], -1)
    s, _ = deer.newton(cell, u, a, s0, tol=0.0, max_iters=cap)
    ref = [s[..., c].reshape(1, D, T) for c in range(s.shape[-1])]
    scale = max(1.0, max(float(np.abs(r).max()) for r in ref))
    assert max_err(got, ref) < 1e-4 * scale


def block_sequential_deer(cell, inp, P, cap):
    """The oracle's DEER iterates block by block: each time block of P steps
    is its own Newton solve (tol = 0, `cap` updates from zero), started from
    the previous block's final state."""
    B, D, T = inp.u[0].shape
    u = deer.from_planes(inp.u_rounded)
    a = deer.a_per_channel(inp.a, B)
    st = np.stack([p.reshape(-1).astype(np.float64) for p in inp.s0], -1)
    parts = []
    for t0 in range(0, T, P):
        s, _ = deer.newton(cell, u[:, t0:t0 + P], a, st, tol=0.0, max_iters=cap)
        parts.append(s)
        st = s[:, -1]
    s = np.concatenate(parts, axis=1)
    return [s[..., c].reshape(B, D, T) for c in range(s.shape[-1])]


@pytest.mark.parametrize("cell", ["gru", "lstm"])
@pytest.mark.parametrize("T", [8192, 9000])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_block_sequential_time_blocks(cell, T, dtype):
    """1024 channels (a full ticket group) past 4096 steps: blocks of 4096
    steps solved one after the other, each from its predecessor's converged
    last state, on float32 and bf16 projections, full blocks and a ragged
    last one.  Every channel matches the sequential oracle; results are
    bitwise repeatable; with tol = 0 and a cap the iterates are the
    block-by-block DEER iterates."""
    from nonlinear_rnn_amd import pararnn as pr
    B, D = 1, 1024
    K, W, nb = pr.plan(cell, pr.make_shape(B, T, D))
    assert (K, W, nb) == (16, 4, -(-T // 4096))
    inp = make_inputs(cell, B, T, D, 7100 + T + len(dtype), u_dtype=dtype, s0_std=0.2,
                      f_bias=1.0)
    got, info = gpu_solve(inp, 1e-6, 30)
    assert info["converged"] and info["units"] == D * nb and info["max_abs_res"] < 1e-6
    assert max_err(got, oracle_states(inp)) < TOL32
    again, info2 = gpu_solve(inp, 1e-6, 30)
    for x, y in zip(got, again):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    assert info2 == info
    cap = 3
    capped, info3 = gpu_solve(inp, 0.0, cap)
    assert info3["iters"] == cap and not info3["converged"]
    ref = block_sequential_deer(cell, inp, 4096, cap)
    scale = max(1.0, max(float(np.abs(r).max()) for r in ref))
    assert max_err(capped, ref) < 1e-4 * scale


@pytest.mark.parametrize("cell", ["gru", "lstm"])
@pytest.mark.parametrize("T", [8192, 9000])
def test_block_sequential_warm_start(cell, T):
    """Warm starts on the block-sequential path (1024 channels, blocks of
    4096 steps chained in one workgroup, full and ragged last block): a start
    at the oracle's trajectory stops with no update and returns it unchanged;
    a perturbed start converges to the same trajectory, the first step of
    every block after the first taken from its predecessor's converged state
    rather than from the perturbed start."""
    from nonlinear_rnn_amd import pararnn as pr
    B, D = 1, 1024
    assert pr.plan(cell, pr.make_shape(B, T, D))[2] == -(-T // 4096)
    inp = make_inputs(cell, B, T, D, 7300 + T, s0_std=0.2, f_bias=1.0)
    ref = oracle_states(inp)
    start = [r.astype(np.float32) for r in ref]
    got, info = gpu_solve(inp, 1e-5, 30, init=start)
    assert info["converged"] and info["iters"] == 0
    for g, s in zip(got, start):
        assert np.array_equal(g, s)
    rng = np.random.default_rng(6)
    pert = [s + rng.standard_normal(s.shape).astype(np.float32) * 0.05 for s in start]
    got, info = gpu_solve(inp, 1e-6, 30, init=pert)
    assert info["converged"] and info["iters"] >= 1
    assert max_err(got, ref) < TOL32


@pytest.mark.parametrize("cell", ["gru", "lstm"])
@pytest.mark.parametrize("T,W", [(4096, 4), (2048, 2)])
def test_warm_start_full_single_blocks(cell, T, W):
    """Warm starts on full one-block-per-channel tiles (K = 16), the kernels
    whose ParaLSTM form keeps three gates' projections in LDS: a start at
    the oracle's trajectory stops with no update and returns it unchanged;
    a perturbed start converges to the same trajectory."""
    from nonlinear_rnn_amd import pararnn as pr
    B, D = 2, 128
    assert pr.plan(cell, pr.make_shape(B, T, D)) == (16, W, 1)
    inp = make_inputs(cell, B, T, D, 7400 + T, s0_std=0.2, f_bias=1.0)
    ref = oracle_states(inp)
    start = [r.astype(np.float32) for r in ref]
    got, info = gpu_solve(inp, 1e-6, 20, init=start)
    assert info["converged"] and info["iters"] == 0
    for g, s in zip(got, start):
        assert np.array_equal(g, s)
    rng = np.random.default_rng(7)
    pert = [s + rng.standard_normal(s.shape).astype(np.float32) * 0.05 for s in start]
    got, info = gpu_solve(inp, 1e-6, 20, init=pert)
    assert info["converged"] and info["iters"] >= 1
    assert max_err(got, ref) < TOL32
