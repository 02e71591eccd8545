"""GPU parity of the input projection (pararnn_project, MFMA) against the
float64 oracle on the same bf16 operands.

Bound: any order of summing the K exact products in float32 is within
K * 2^-24 * sum_k |w x| of the exact sum (plus the bias add); bfloat16
output adds one rounding, 2^-8 relative.
"""
import numpy as np
import pytest
import torch

from nonlinear_rnn_amd import pararnn as pr
from oracle import projection

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def bf16(a):
    """float32 array -> (torch bfloat16 on device, float64 numpy of the same values)."""
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)
    return t.to(DEV), t.to(torch.float64).numpy()


def check(got, x64, w64, bias, out_bf16=False):
    ref = projection.project(x64, w64, bias)
    scale = projection.project_abs(x64, w64, bias)
    K = x64.shape[2]
    bound = (K + 2) * 2.0 ** -24 * scale + 1e-30
    if out_bf16:
        bound = bound + 2.0 ** -8 * np.abs(ref)
    err = np.abs(got.to(torch.float64).cpu().numpy() - ref)
    assert np.all(err <= bound), (float(err.max()), float((err / bound).max()))


@pytest.mark.parametrize("B,T,I,M", [(2, 128, 64, 256), (1, 100, 40, 300), (3, 257, 1024, 288),
                                     (2, 384, 96, 768), (1, 1, 8, 1), (2, 130, 33, 257),
                                     (2, 700, 192, 600), (1, 2100, 128, 1100),
                                     # more tiles than compute units, ragged in m and t:
                                     # 408 tiles (a multiple of the 8 XCDs) with one k
                                     # step, 306 tiles (not a multiple) with two
                                     (4, 4100, 64, 1300), (3, 4100, 128, 1300)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_project_parity(B, T, I, M, out_dtype):
    rng = np.random.default_rng(B * 1000 + T + I + M)
    x, x64 = bf16(rng.standard_normal((B, T, I)))
    w, w64 = bf16(rng.standard_normal((M, I)) / np.sqrt(I))
    bias = rng.standard_normal(M).astype(np.float32)
    u = pr.project(x, w, torch.from_numpy(bias).to(DEV), out_dtype=out_dtype)
    torch.cuda.synchronize()
    check(u, x64, w64, bias.astype(np.float64), out_bf16=out_dtype == torch.bfloat16)


def test_project_no_bias_and_empty_inner_dimension():
    rng = np.random.default_rng(5)
    x, x64 = bf16(rng.standard_normal((2, 64, 48)))
    w, w64 = bf16(rng.standard_normal((256, 48)))
    u = pr.project(x, w)
    torch.cuda.synchronize()
    check(u, x64, w64, None)
    bias = torch.arange(5, dtype=torch.float32, device=DEV)
    u0 = pr.project(torch.empty((1, 3, 0), dtype=torch.bfloat16, device=DEV),
                    torch.empty((5, 0), dtype=torch.bfloat16, device=DEV), bias)
    torch.cuda.synchronize()
    assert torch.equal(u0, bias[None, :, None].expand(1, 5, 3))


def test_project_strided_views():
    """x and w as views into wider rows (k stride 1, row strides not 8-multiples
    or not 16-byte aligned), output as a view into a wider buffer."""
    rng = np.random.default_rng(6)
    xb, _ = bf16(rng.standard_normal((2, 70, 45)))
    wb, _ = bf16(rng.standard_normal((300, 41)))
    x = xb[:, 3:68, 1:41]
    w = wb[:, 1:41]
    x64 = x.to(torch.float64).cpu().numpy()
    w64 = w.to(torch.float64).cpu().numpy()
    big = torch.full((2, 310, 80), 7.0, device=DEV)
    out = big[:, 5:305, 2:67]
    pr.project(x, w, out=out)
    torch.cuda.synchronize()
    check(out, x64, w64, None)
    assert float(big[:, :5].sub(7).abs().max()) == 0.0
    assert float(big[:, :, :2].sub(7).abs().max()) == 0.0
    assert float(big[:, :, 67:].sub(7).abs().max()) == 0.0


def test_projection_feeds_the_solve():
    """x -> u (bf16 planes of one [B][3D][T] buffer) -> ParaGRU solve, against
    the oracle solve on the oracle projection rounded to bf16 the same way."""
    from oracle import sequential as seq
    B, T, I, D = 2, 512, 64, 32
    rng = np.random.default_rng(7)
    x, x64 = bf16(rng.standard_normal((B, T, I)))
    w, w64 = bf16(rng.standard_normal((3 * D, I)) / np.sqrt(I))
    u = pr.project(x, w, out_dtype=torch.bfloat16)
    planes = [u[:, g * D:(g + 1) * D] for g in range(3)]
    a = torch.from_numpy(rng.uniform(-1, 1, (3, D)).astype(np.float32)).to(DEV)
    h0 = torch.zeros((B, D), device=DEV)
    h, info = pr.solve_gru(planes, a, h0, tol=1e-6, max_iters=30)
    assert pr.read_info(info)["converged"]
    # oracle: the device's bf16 projections (checked above against the fp64
    # product), solved sequentially in fp64
    u_dev = [np.ascontiguousarray(p.to(torch.float32).cpu().numpy()) for p in planes]
    ref = seq.gru_forward(u_dev, a.cpu().numpy(), h0.cpu().numpy())
    assert np.max(np.abs(h.cpu().numpy() - ref)) < 1e-5
    check(u, x64, w64, None, out_bf16=True)


@pytest.mark.parametrize("key", ["gru_small", "gru_f32", "lstm_f32", "gru_bf16_long", "lstm_fwd_bwd"])
def test_project_workload_scale(key):
    """The projection of each workload at full size, in the launch the bench
    times (x [B][T][I=D] bf16, W [G*D][I] bf16, output [B][G*D][T] in the
    workload's projection dtype), checked against the oracle on every output
    row at sampled time steps (all column tiles) and on every time step of
    sampled rows (all row tiles), both including the tile edges."""
    from nonlinear_rnn_amd.inputs import WORKLOADS
    w = WORKLOADS[key]
    I, M = w.D, (3 if w.cell == "gru" else 4) * w.D
    gen = torch.Generator(device="cpu").manual_seed(w.seed + 200)
    x = torch.randn((w.B, w.T, I), generator=gen).to(torch.bfloat16).to(DEV)
    wt = (torch.randn((M, I), generator=gen) / I ** 0.5).to(torch.bfloat16)
    bias = torch.randn(M, generator=gen)
    w64, b64 = wt.to(torch.float64).numpy(), bias.to(torch.float64).numpy()
    out_dtype = torch.bfloat16 if w.u_dtype == "bf16" else torch.float32
    out = torch.empty((w.B, M, w.T), dtype=out_dtype, device=DEV)
    pr.project(x, wt.to(DEV), bias.to(DEV), out=out)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    rng = np.random.default_rng(w.seed + 200)

    def edges(n):
        ks = sorted({1, n // 512, n // 256} | set(rng.integers(1, n // 256 + 2, 4).tolist()))
        e = {0, n - 1} | {v for k in ks for v in (256 * k - 1, 256 * k) if 0 < v < n}
        return sorted(e | set(rng.integers(0, n, 16).tolist()))

    ts = edges(w.T)
    tsel = torch.tensor(ts, device=DEV)
    xs64 = x[:, tsel].to(torch.float64).cpu().numpy()
    check(out[:, :, tsel], xs64, w64, b64, out_bf16=out_dtype == torch.bfloat16)
    ms = edges(M)
    msel = torch.tensor(ms, device=DEV)
    for b in sorted({0, w.B - 1}):
        xb64 = x[b:b + 1].to(torch.float64).cpu().numpy()
        check(out[b:b + 1, msel], xb64, w64[ms], b64[ms], out_bf16=out_dtype == torch.bfloat16)
