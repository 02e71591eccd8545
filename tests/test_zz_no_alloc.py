"""The allocation-free ParaGRU solve (pararnn_solve_gru_noalloc: workspace
from the library's static per-GPU array) against pararnn_solve_gru with a
caller workspace, through the C ABI: two calls in a row, the second on a
smaller problem (the array keeps the first call's flags and records, which
the solve must clear), each bitwise equal to the workspace entry point on
the same tiling and within 1e-5 of the fp64 oracle."""
import numpy as np
import pytest
import torch

from nonlinear_rnn_amd import pararnn as pr
from nonlinear_rnn_amd.inputs import make_inputs
from tests.gpu_util import DEV, dev_inputs, max_err, oracle_states

pytestmark = pytest.mark.gpu


def _both(inp, K, W, tol=1e-6, cap=20):
    u, a, s0 = dev_inputs(inp)
    B, D, T = u[0].shape
    ref, info_ref = pr.solve_gru(u, a, s0[0], tol=tol, max_iters=cap, steps_per_lane=K,
                                 waves_per_block=W)
    out = torch.full((B, D, T), float("nan"), dtype=torch.float32, device=DEV)
    info = torch.zeros(pr.INFO_BYTES, dtype=torch.uint8, device=DEV)
    pr.solve_gru_noalloc(u, a, s0[0], out, tol=tol, max_iters=cap, steps_per_lane=K,
                         waves_per_block=W, info=info)
    torch.cuda.synchronize()
    return ref, pr.read_info(info_ref), out, pr.read_info(info)


@pytest.mark.parametrize("first,second", [
    # (B, T, D, K, W): several ragged time blocks, then fewer and smaller
    ((2, 5000, 48, 16, 1), (1, 1500, 16, 16, 1)),
    # one block per channel (convergence records only), then multi-block
    ((1, 1024, 64, 0, 0), (1, 700, 8, 4, 1)),
])
def test_static_scratch_solve_matches_workspace_solve(first, second):
    for i, (B, T, D, K, W) in enumerate((first, second)):
        inp = make_inputs("gru", B, T, D, 40 + i, s0_std=0.1)
        ref, info_ref, got, info = _both(inp, K, W)
        assert torch.equal(got, ref), (B, T, D, K, W)
        assert info == info_ref
        assert info["converged"] and info["units"] > 0
        err = max_err([got.cpu().numpy()], oracle_states(inp))
        assert err < 1e-5, err


def test_static_scratch_solve_bf16_time_major():
    """Time-major bf16 planes: staged through the static array when they fit
    (here they do), bitwise equal to the workspace entry point."""
    B, T, D = 2, 2048, 32
    inp = make_inputs("gru", B, T, D, 44, u_dtype="bf16")
    u, a, s0 = dev_inputs(inp)
    full = torch.empty((B, T, 3 * D), dtype=torch.bfloat16, device=DEV)
    for g in range(3):
        full[:, :, g * D:(g + 1) * D] = u[g].transpose(1, 2)
    ut = [full[:, :, g * D:(g + 1) * D].transpose(1, 2) for g in range(3)]
    ref, _ = pr.solve_gru(u, a, s0[0], tol=1e-5, max_iters=30, info=False)
    out = torch.empty((B, T, D), dtype=torch.float32, device=DEV).transpose(1, 2)
    pr.solve_gru_noalloc(ut, a, s0[0], out, tol=1e-5, max_iters=30)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_static_scratch_solve_rejects_oversized_problem():
    B, T, D = 1, 65536, 1024
    u = [torch.zeros((B, D, T), dtype=torch.float32, device=DEV) for _ in range(3)]
    a = torch.zeros((3, D), dtype=torch.float32, device=DEV)
    h0 = torch.zeros((B, D), dtype=torch.float32, device=DEV)
    out = torch.zeros((B, D, T), dtype=torch.float32, device=DEV)
    with pytest.raises(pr.PararnnError) as e:
        pr.solve_gru_noalloc(u, a, h0, out, steps_per_lane=1, waves_per_block=1)
    assert e.value.status == 5
    assert float(out.abs().max()) == 0.0  # nothing ran
