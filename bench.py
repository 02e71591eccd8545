"""Bench: fused ParaGRU Newton solve, bf16 projections, B=4 T=16384 D=4096,
on one GPU, with the other four workloads measured in the same run.

One step = one whole Newton solve (residual + Jacobian + scan + update +
on-device convergence test, iterated to max|r| < tol or the iteration cap)
over the full batch, with the projections already resident in HBM.  For
the forward + backward workload (lstm_fwd_bwd) a step is the solve followed
by the adjoint pass for upstream gradients dL/dh_t.

Prints ONE JSON line for the headline workload (default gru_bf16_long, the
largest): throughput in hidden-state elements per second (B*T*D per solve)
from the wall clock of K back-to-back steps; the roofline of the dominant
kernel, algorithmic HBM bytes per launch over its HIP-event average (the
MALL evicted by a 512 MiB write before every launch) against the MI355X
8 TB/s, with the VALU issue fraction as a secondary key; every other
workload's figures under "configs"; and the CPU oracle timed on a bounded
sample of the headline workload on all host cores and on one.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gru_bf16_long]
                    [--configs all|none|key,key]
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
# The second roof: VALU issue.  On gfx950 a plain fp32 wave64 instruction
# (FMA, mul, add, max) occupies a SIMD for 2 cycles (32 lanes per clock:
# 256 CUs x 4 SIMDs x 32 lanes x 2 flops x 2.4 GHz is the published
# 157.3 TFLOP/s fp32 vector peak) and a transcendental (v_exp_f32,
# v_rcp_f32) for 8, a quarter of that rate; a probe of independent chains
# at 8 waves per SIMD measures 2.45 and 8.3 cycles, and exp interleaved
# with FMAs costs the sum of both (no overlap).  These kernels issue no
# packed fp32.
CYC_PLAIN, CYC_TRANS = 2.0, 8.0
SIMD_CYCLES_PER_S = 256 * 4 * 2.4e9
# Algorithmic operations per hidden-state element and Newton pass, from the
# cell formulas: gate pre-activations, exp2/rcp gates, residual, local
# Jacobian, one map composition, the update and the residual max, as
# (plain ops, transcendentals); a unit's last pass only evaluates the
# residual.  ParaGRU: 26 + 6 per update pass, 12 + 6 on the final one;
# ParaLSTM (2x2 maps): 52 + 10, and 18 + 10.
VALU_OPS = {"gru": ((26, 6), (12, 6)), "lstm": ((52, 10), (18, 10))}
# Plain ops that drop out of the first pass from the zero start, at every
# step but a lane's first (ParaGRU; the terms with h_{t-1} or h_t).
ZERO_PASS_SAVED = {"gru": 9, "lstm": 0}
HEADLINE = "gru_bf16_long"  # the largest workload
METRIC = "hidden-state elems/sec per Newton solve (B·T·D) + % of MI355X HBM peak"


def algorithmic_bytes(w):
    """Compulsory HBM traffic of one solve: read every projection once, the
    diagonal weights and the initial states, write every state once."""
    ub = 2 if w.u_dtype == "bf16" else 4
    return w.G * w.N * ub + w.G * w.D * 4 + w.S * w.B * w.D * 4 + w.S * w.N * 4


def adjoint_bytes(w):
    """Compulsory HBM traffic of one adjoint pass: read the projections, the
    converged states and the upstream gradients dL/dh_t, write dL/du; the
    [G][D] and [B][D] vectors (a, s0, da, ds0) are included."""
    ub = 2 if w.u_dtype == "bf16" else 4
    return (w.G * w.N * ub + w.S * w.N * 4 + w.N * 4 + w.G * w.N * 4
            + 2 * w.G * w.D * 4 + 2 * w.S * w.B * w.D * 4)


def data_recipe(w):
    parts = [f"u~N(0,1) {'rounded to bf16' if w.u_dtype == 'bf16' else 'f32'}", "a~U(-1,1)",
             f"s0~N(0,{w.s0_std}^2)" if w.s0_std else "s0=0"]
    if w.f_bias:
        parts.append(f"forget-gate bias +{w.f_bias:g}")
    if w.adjoint:
        parts.append("dL/dh_t~N(0,1)")
    return f"synthetic (seeded numpy PCG64, seed {w.seed}: " + ", ".join(parts) + ")"


# Sources whose code only the input projection uses; every other file under
# csrc/ (and the ABI header) builds the solve, adjoint and scan kernels.
PROJECTION_ONLY = ("project.hpp", "inst_project.hip")


def _code_only(text):
    """C/C++ source without comments, indentation and blank lines: edits
    to documentation do not change what is compiled."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(ln.strip() for ln in text.splitlines() if ln.strip())


def kernel_source_digest(family="solve"):
    """Hash of the code a kernel family is built from: "project" (the
    projection kernels and the ABI) or "solve" (everything else), plus the
    ABI header and the build script."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "nonlinear_rnn_amd", "csrc")
    names = sorted(os.listdir(csrc))
    if family == "project":
        names = [n for n in names if n in PROJECTION_ONLY or n == "pararnn.hip"]
    else:
        names = [n for n in names if n not in PROJECTION_ONLY]
    # the build script carries the compile flags (and per-unit scheduler choice)
    paths = [os.path.join(csrc, n) for n in names] + [os.path.join(ROOT, "include", "pararnn.h"),
                                                      os.path.join(ROOT, "nonlinear_rnn_amd",
                                                                   "build.py")]
    for path in paths:
        with open(path, encoding="utf-8") as f:
            h.update((os.path.basename(path) + _code_only(f.read())).encode())
    return h.hexdigest()[:16]


def measured_traffic(key):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{key}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    family = "project" if key.startswith("project_") else "solve"
    if rec.get("kernel_source_digest") != kernel_source_digest(family):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, inp, budget_s=10.0):
    """The fp64 sequential oracle on a sample of channels, timed on all host
    threads (OpenMP over channels) and on one thread."""
    from oracle import sequential as seq

    all_threads = seq.max_threads()

    def run(n, threads):
        chans = [(i % w.B, (i * 7919) % w.D) for i in range(n)]
        sub_u, a_sub, s0_sub = seq.gather_channels(inp.u, inp.a, inp.s0, chans)
        t = time.perf_counter()
        if w.cell == "gru":
            seq.gru_forward(sub_u, a_sub, s0_sub[0], threads)
        else:
            seq.lstm_forward(sub_u, a_sub, s0_sub[0], s0_sub[1], threads)
        return time.perf_counter() - t

    def timed(threads):
        n = min(w.B * w.D, 4 * threads)
        dt = run(n, threads)
        # a sample of about budget_s / 4 per run, repeated until about
        # budget_s of wall time is spent
        target = int(n * budget_s / 4 / max(dt, 1e-3))
        n = max(n, min(w.B * w.D, target))
        reps, total = 0, 0.0
        while reps == 0 or total < budget_s:
            total += run(n, threads)
            reps += 1
        dt = total / reps
        return n, reps, dt, n * w.T / dt

    n, reps, dt, rate = timed(all_threads)
    n1, reps1, dt1, rate1 = timed(1)
    return {"value": rate, "unit": "elem/s", "cores": all_threads, "kind": "oracle",
            "sample": f"{n} of {w.B * w.D} channels x T={w.T} (fp64 sequential step-by-step, "
                      f"OpenMP over channels), mean of {reps} runs, {dt:.3f} s each",
            "single_thread": {"value": rate1, "unit": "elem/s", "cores": 1,
                              "sample": f"{n1} channels x T={w.T}, mean of {reps1} runs, "
                                        f"{dt1:.3f} s each"}}


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak


def settle(fn, args):
    """Run `fn` back to back, untimed, for args.settle_ms of wall time: an
    idle MI355X needs some 20 ms of sustained load before its clocks reach
    their steady state (the B=8 T=4096 D=1024 ParaGRU solve takes 0.19 ms
    per call during the first ~100 calls, 0.172 ms after), and a few
    warm-up steps do not get there.  Returns the number of calls."""
    import torch

    n, t0 = 0, time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < args.settle_ms:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
        n += 8
    return n


def bench_project(w, args):
    """The input projection for the workload: x [B][T][I = D] and W [G*D][I]
    bf16 (seeded N(0,1), W scaled by 1/sqrt(I)), bias f32, output in the
    workload's projection dtype.  One step = one projection of the batch."""
    import numpy as np
    import torch
    from nonlinear_rnn_amd import pararnn as pr

    dev = "cuda:0"
    I, M = w.D, w.G * w.D
    rng = np.random.default_rng(w.seed + 100)
    gen = torch.Generator(device="cpu").manual_seed(w.seed + 100)
    x = torch.randn((w.B, w.T, I), generator=gen).to(torch.bfloat16).to(dev)
    wt = (torch.randn((M, I), generator=gen) / I ** 0.5).to(torch.bfloat16).to(dev)
    bias = torch.from_numpy(rng.standard_normal(M).astype(np.float32)).to(dev)
    out_dtype = torch.bfloat16 if w.u_dtype == "bf16" else torch.float32
    out = torch.empty((w.B, M, w.T), dtype=out_dtype, device=dev)
    stream = torch.cuda.current_stream()
    settle(lambda: pr.project(x, wt, bias, out=out, stream=stream), args)
    for _ in range(args.warmup):
        pr.project(x, wt, bias, out=out, stream=stream)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        pr.project(x, wt, bias, out=out, stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    kavg = sum(ms) / len(ms)
    flops = 2.0 * w.B * w.T * I * M
    tflops = flops / (kavg * 1e-3) / 1e12
    ob = 2 if out_dtype == torch.bfloat16 else 4
    nbytes = w.B * w.T * I * 2 + M * I * 2 + M * 4 + w.B * M * w.T * ob
    extra = {}
    # context: the library GEMM (hipBLASLt through torch.matmul) on the same
    # bf16 operands with bf16 output; the right operand is made contiguous
    # (x^T per batch row) outside the timed region
    xt = x.transpose(1, 2).contiguous()
    settle(lambda: torch.matmul(wt, xt), args)
    for _ in range(args.warmup):
        torch.matmul(wt, xt)
    lev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for e0, e1 in lev:
        e0.record(stream)
        torch.matmul(wt, xt)
        e1.record(stream)
    torch.cuda.synchronize()
    lms = sorted(e0.elapsed_time(e1) for e0, e1 in lev)[len(lev) // 2]
    extra["library_gemm"] = {"tflops": flops / (lms * 1e-3) / 1e12, "ms": lms,
                             "kind": "torch.matmul (hipBLASLt), same bf16 operands, bf16 "
                                     "output, no bias; context, not a baseline"}
    del xt
    if args.copy_mib:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        extra["copy_calibration_bytes"] = n * 4
    return dict({
        "metric": "input projection TFLOP/s (u = W x + b, bf16 in, fp32 accumulate)",
        "value": flops / (wall / args.steps) / 1e12, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": f"synthetic (torch.randn seed {w.seed + 100}: x~N(0,1), W~N(0,1/I), bias~N(0,1))",
        "config": {"workload": f"projection for {w.name}", "B": w.B, "T": w.T, "I": I, "M": M,
                   "out_dtype": "bf16" if ob == 2 else "f32"},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": measured_traffic("project_" + args.workload),
                     "algorithmic_bytes": nbytes, "kernel": "project_kernel",
                     "kernel_ms_avg": kavg, "kernel_ms_min": min(ms),
                     "hbm": {"achieved": nbytes / (kavg * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                             "unit": "GB/s",
                             "frac": nbytes / (kavg * 1e-3) / 1e9 / HBM_PEAK_GBS}},
    }, **extra)


def bench_scan(w, args):
    """The standalone linear-recurrence scan x_t = A_t x_{t-1} + b_t over the
    workload's channels and length, with the workload's state size (S = 1
    for ParaGRU, 2 for ParaLSTM): A ~ U(0, 0.9) (S*S planes, contracting), b
    ~ N(0, 1) (S planes), x0 = 0.  One step = one forward scan; a reverse
    scan is timed beside it.  HBM roof: A and b read once, x written once."""
    import torch
    from nonlinear_rnn_amd import pararnn as pr

    dev = "cuda:0"
    S = w.S
    gen = torch.Generator(device="cpu").manual_seed(w.seed + 300)
    A = [(torch.rand((w.B, w.D, w.T), generator=gen) * 0.9).to(dev) for _ in range(S * S)]
    b = [torch.randn((w.B, w.D, w.T), generator=gen).to(dev) for _ in range(S)]
    out = [torch.empty((w.B, w.D, w.T), device=dev) for _ in range(S)]
    stream = torch.cuda.current_stream()
    flush_buf = torch.empty(args.flush_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)

    def run(rev):
        pr.scan(A, b, reverse=rev, out=out, stream=stream)

    settle(lambda: run(False), args)
    for _ in range(args.warmup):
        run(False)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        run(False)
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    b2b = [e0.elapsed_time(e1) for e0, e1 in evs]

    def evicted(rev):
        ms = []
        for _ in range(args.steps):
            flush_mall(flush_buf)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run(rev)
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        return ms

    fwd, rev = evicted(False), evicted(True)
    extra = {}
    if args.copy_mib:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        extra["copy_calibration_bytes"] = n * 4
    nbytes = (S * S + 2 * S) * 4 * w.N
    kavg = sum(fwd) / len(fwd)
    ravg = sum(rev) / len(rev)
    gbs = nbytes / (kavg * 1e-3) / 1e9
    ms_per_step = wall * 1e3 / args.steps
    return {
        "metric": "linear-recurrence scan elems/sec (B·T·D) + % of MI355X HBM peak",
        "value": w.N / (ms_per_step * 1e-3), "unit": "elem/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": f"synthetic (torch seed {w.seed + 300}: A~U(0,0.9), b~N(0,1), x0=0)",
        "config": {"workload": f"scan, state size {S}, over the channels of {w.name}",
                   "B": w.B, "T": w.T, "D": w.D, "S": S},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic("scan_" + args.workload),
                     "algorithmic_bytes": nbytes, "kernel": "scan_kernel",
                     "kernel_ms_avg": kavg, "kernel_ms_min": min(fwd),
                     "kernel_ms_avg_back_to_back": sum(b2b) / len(b2b),
                     "timing": f"HIP events on the launch stream, {args.steps} launches, a "
                               f"{args.flush_mib} MiB write before each (outside the event pair)"},
        "reverse": {"kernel_ms_avg": ravg, "achieved": nbytes / (ravg * 1e-3) / 1e9,
                    "frac": nbytes / (ravg * 1e-3) / 1e9 / HBM_PEAK_GBS},
        **extra,
    }


def bench_checkpoint(w, args):
    """Training step (forward solve + backward through torch.autograd) on
    the workload, one-piece vs checkpointed in time chunks of --chunk steps:
    time per step and the peak device memory each holds beyond the inputs."""
    import numpy as np
    import torch
    from nonlinear_rnn_amd import autograd as pag
    from nonlinear_rnn_amd import longseq
    from nonlinear_rnn_amd.inputs import workload_inputs

    dev = "cuda:0"
    inp = workload_inputs(w)
    if inp.u_bf16 is not None:
        u = [torch.from_numpy(p.view(np.int16)).view(torch.bfloat16).to(dev)
             for p in inp.u_bf16]
    else:
        u = [torch.from_numpy(p).to(dev) for p in inp.u]
    for p in u:
        p.requires_grad_(True)
    a = torch.from_numpy(inp.a).to(dev).requires_grad_(True)
    s0 = [torch.from_numpy(p).to(dev).requires_grad_(True) for p in inp.s0]
    rng = np.random.default_rng(w.seed + 7)
    gh = torch.from_numpy(rng.standard_normal((w.B, w.D, w.T)).astype(np.float32)).to(dev)
    del inp

    def step(kind, held=None):
        # the loss consumes the states and drops them, as a next layer would:
        # what stays allocated until the backward is what the solve keeps
        kw = dict(tol=w.tol, max_iters=w.max_iters)
        if kind == "full":
            out = pag.gru(u, a, s0[0], **kw) if w.cell == "gru" else pag.lstm(u, a, *s0, **kw)
        elif w.cell == "gru":
            out = longseq.gru_checkpointed(u, a, s0[0], chunk=args.chunk, **kw)
        else:
            out = longseq.lstm_checkpointed(u, a, *s0, chunk=args.chunk, **kw)
        h = out if w.cell == "gru" else out[1]
        loss = (h * gh).sum()
        del out, h
        if held is not None:
            torch.cuda.synchronize()
            held.append(torch.cuda.memory_allocated())
        loss.backward()
        for t in u + [a] + s0:
            t.grad = None

    res = {}
    for kind in ("full", "checkpointed"):
        settle(lambda: step(kind), args)
        for _ in range(args.warmup):
            step(kind)
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        held = []
        step(kind, held)
        torch.cuda.reset_peak_memory_stats()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step(kind)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        res[kind] = {"ms_per_step": ms, "held_for_backward_bytes": held[0] - base,
                     "peak_extra_bytes": torch.cuda.max_memory_allocated() - base}
    return {
        "metric": "training step (solve + adjoint) time and peak memory, one-piece vs "
                  "checkpointed",
        "value": w.N / (res["checkpointed"]["ms_per_step"] * 1e-3), "unit": "elem/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": res["checkpointed"]["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": data_recipe(w),
        "config": {"workload": w.name, "B": w.B, "T": w.T, "D": w.D, "chunk": args.chunk},
        "full": res["full"], "checkpointed": res["checkpointed"],
        "state_bytes": w.S * w.B * w.D * w.T * 4,
    }


def bench_speedup(args):
    """Parallel (Newton) vs sequential application on the same GPU, the
    comparison behind the pages' speed-up figures: ParaGRU f32 with 64
    channels (B=1, D=64, the small workload's width) and growing T, inputs
    drawn as for that workload (seed 1).  Both kernels produce the same
    trajectory (to the Newton tolerance); times are HIP-event medians."""
    import numpy as np
    import torch
    from nonlinear_rnn_amd import pararnn as pr
    from nonlinear_rnn_amd.inputs import make_inputs

    dev = "cuda:0"
    stream = torch.cuda.current_stream()
    points = []
    for T in (1024, 4096, 16384, 65536, 262144):
        inp = make_inputs("gru", 1, T, 64, 1)
        u = [torch.from_numpy(p).to(dev) for p in inp.u]
        a = torch.from_numpy(inp.a).to(dev)
        h0 = torch.from_numpy(inp.s0[0]).to(dev)
        h = torch.empty((1, 64, T), dtype=torch.float32, device=dev)
        hs = [torch.empty_like(h)]

        def newton():
            pr.solve_gru(u, a, h0, out=h, tol=1e-6, max_iters=20, info=False, stream=stream)

        def seq():
            pr.sequential("gru", u, a, [h0], out=hs, stream=stream)

        res = {}
        for name, fn in (("newton", newton), ("sequential", seq)):
            settle(fn, args)
            for _ in range(max(1, args.warmup)):
                fn()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(7)]
            for e0, e1 in ev:
                e0.record(stream)
                fn()
                e1.record(stream)
            torch.cuda.synchronize()
            res[name] = sorted(e0.elapsed_time(e1) for e0, e1 in ev)[3]
        info = pr.read_info(pr.solve_gru(u, a, h0, out=h, tol=1e-6, max_iters=20)[1])
        err = float((h - hs[0]).abs().max())
        points.append({"T": T, "newton_ms": res["newton"], "sequential_ms": res["sequential"],
                       "speedup": res["sequential"] / res["newton"],
                       "newton_updates": info["iters"], "max_abs_diff": err})
    best = max(points, key=lambda q: q["speedup"])
    return {"metric": "parallel (Newton) vs sequential application, same GPU",
            "value": best["speedup"], "unit": "x", "n_gpus": 1, "steps": 7,
            "warmup": args.warmup, "ms_per_step": best["newton_ms"], "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic (seeded numpy PCG64, seed 1: u~N(0,1), a~U(-1,1), h0=0)",
            "config": {"workload": "ParaGRU f32 B=1 D=64, T from 1024 to 262144"},
            "points": points}


def flush_mall(buf):
    """Write the whole eviction buffer (>= 512 MB, twice the 256 MB MALL), so
    that the next launch finds none of its inputs in the last-level cache."""
    buf.fill_(1.0)


def measure_solve(w, key, args, flush_buf, headline):
    """One workload: convergence report, then the contract's timed region
    (K back-to-back steps, wall clock, HIP events around every launch on its
    stream), then K more steps with a MALL-evicting write before each one
    (outside the event pair) for the roofline."""
    import numpy as np
    import torch
    from nonlinear_rnn_amd import pararnn as pr
    from nonlinear_rnn_amd.inputs import workload_inputs

    inp = workload_inputs(w)
    dev = "cuda:0"
    if inp.u_bf16 is not None:
        u = [torch.from_numpy(p.view(np.int16)).view(torch.bfloat16).to(dev) for p in inp.u_bf16]
    else:
        u = [torch.from_numpy(p).to(dev) for p in inp.u]
    a = torch.from_numpy(inp.a).to(dev)
    s0 = [torch.from_numpy(p).to(dev) for p in inp.s0]
    out = [torch.empty((w.B, w.D, w.T), dtype=torch.float32, device=dev) for _ in range(w.S)]
    time_major = headline and args.layout == "time"
    if time_major:
        # one [B][T][G*D] tensor (what a Linear over [B][T][I] inputs gives),
        # passed per gate as strided views; states [B][T][D]
        G, D = w.G, w.D
        full = torch.empty((w.B, w.T, G * D), dtype=u[0].dtype, device=dev)
        for g, p in enumerate(u):
            full[:, :, g * D:(g + 1) * D] = p.transpose(1, 2)
        u = [full[:, :, g * D:(g + 1) * D].transpose(1, 2) for g in range(G)]
        out = [torch.empty((w.B, w.T, D), dtype=torch.float32, device=dev).transpose(1, 2)
               for _ in range(w.S)]
    stream = torch.cuda.current_stream()
    ws_solve = ws_adj = None
    if time_major and args.route == "gather":
        # workspaces of the channel-major size: no room to stage, so the
        # kernels gather the time-major steps directly
        dense = pr.make_shape(w.B, w.T, w.D)
        nwt = pr.make_newton(w.tol, w.max_iters)
        ws_solve = torch.empty(max(1, pr.workspace_bytes(w.cell, dense, nwt)),
                               dtype=torch.uint8, device=dev)
        ws_adj = torch.empty(max(1, pr.workspace_bytes(w.cell, dense, nwt, adjoint=True)),
                             dtype=torch.uint8, device=dev)

    def solve(info):
        if w.cell == "gru":
            return pr.solve_gru(u, a, s0[0], out=out[0], tol=w.tol, max_iters=w.max_iters,
                                info=info, workspace=ws_solve, stream=stream)[1]
        return pr.solve_lstm(u, a, s0[0], s0[1], out=out, tol=w.tol, max_iters=w.max_iters,
                             info=info, workspace=ws_solve, stream=stream)[1]

    adj_out = None
    gs = None
    if w.adjoint:
        gh = torch.from_numpy(inp.dh).to(dev)
        if time_major:
            gh = gh.transpose(1, 2).contiguous().transpose(1, 2)
            du_full = torch.empty((w.B, w.T, w.G * w.D), dtype=torch.float32, device=dev)
            adj_out = dict(du=[du_full[:, :, g * w.D:(g + 1) * w.D].transpose(1, 2)
                               for g in range(w.G)],
                           da=torch.empty((w.G, w.D), dtype=torch.float32, device=dev),
                           ds0=[torch.empty((w.B, w.D), dtype=torch.float32, device=dev)
                                for _ in range(w.S)], lam=None)
        gs = [None, gh] if w.cell == "lstm" else [gh]

    def backward():
        nonlocal adj_out
        adj_out = pr.adjoint(w.cell, u, a, s0, out, gs, stream=stream, out=adj_out,
                             workspace=ws_adj)

    # convergence report (untimed; the solve is deterministic)
    info = pr.read_info(solve(True))

    def step():
        solve(False)
        if w.adjoint:
            backward()

    n_settle = settle(step, args)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    nev = 3 if w.adjoint else 2

    def events():
        return [[torch.cuda.Event(enable_timing=True) for _ in range(nev)]
                for _ in range(args.steps)]

    def run(evs, flush):
        for ev in evs:
            if flush:
                flush_mall(flush_buf)
            ev[0].record(stream)
            solve(False)
            ev[1].record(stream)
            if w.adjoint:
                backward()
                ev[2].record(stream)

    # the timed region: K back-to-back steps
    evs = events()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(evs, False)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    # the roofline region: K steps, the MALL evicted before each one (the
    # eviction buffer written once beforehand, so that no first touch of
    # its pages falls inside the region)
    cold = events()
    flush_mall(flush_buf)
    torch.cuda.synchronize()
    run(cold, True)
    torch.cuda.synchronize()

    def kernel_stats(i, name, nbytes):
        warm = [ev[i].elapsed_time(ev[i + 1]) for ev in evs]
        ms = [ev[i].elapsed_time(ev[i + 1]) for ev in cold]
        avg = sum(ms) / len(ms)
        return {"kernel": name, "ms_avg": avg, "ms_min": min(ms),
                "ms_median": sorted(ms)[len(ms) // 2],
                "ms_avg_back_to_back": sum(warm) / len(warm), "bytes": nbytes,
                "achieved": nbytes / (avg * 1e-3) / 1e9,
                "hbm_frac": nbytes / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS}

    kernels = [kernel_stats(0, "newton_kernel", algorithmic_bytes(w))]
    # VALU issue cycles of the solve: every unit runs its updates plus one
    # final residual pass (iters_mean = updates per unit)
    (pu, tu), (pf, tf) = VALU_OPS[w.cell]
    n = info["iters_mean"]
    K, W, nb = pr.plan(w.cell, pr.make_shape(w.B, w.T, w.D))
    # the first pass is an update pass unless a unit stops at once
    saved = ZERO_PASS_SAVED[w.cell] * CYC_PLAIN * (K - 1) / K * min(1.0, n)
    cyc_per_elem = (n * (pu * CYC_PLAIN + tu * CYC_TRANS) + pf * CYC_PLAIN + tf * CYC_TRANS
                    - saved) / 64
    t_alu_ms = w.N * cyc_per_elem / SIMD_CYCLES_PER_S * 1e3
    kernels[0]["valu"] = {"bound": "alu", "min_ms": t_alu_ms,
                          "frac": t_alu_ms / kernels[0]["ms_avg"],
                          "simd_cycles_per_elem": cyc_per_elem,
                          "ops": "algorithmic wave64 VALU issue cycles per SIMD (plain fp32 op 2, "
                                 "exp/rcp 8) over 1024 SIMDs at 2.4 GHz"}
    if w.adjoint:
        kernels.append(kernel_stats(1, "adjoint_kernel", adjoint_bytes(w)))
    res = {
        "workload": w.name, "B": w.B, "T": w.T, "D": w.D, "N": w.N,
        "ms_per_step": ms_per_step, "elem_per_s": w.N / (ms_per_step * 1e-3),
        "tol": w.tol, "max_iters": w.max_iters, "seed": w.seed,
        "tiling": {"K": K, "W": W, "time_blocks": nb},
        "newton_updates": info["iters"], "newton_updates_mean": info["iters_mean"],
        "converged": info["converged"], "max_abs_res": info["max_abs_res"],
        "settle": {"ms": args.settle_ms, "steps": n_settle},
        "kernels": kernels,
    }
    # context: the same trajectory by step-by-step application on the GPU
    # (one lane per channel), the baseline of the pages' parallel speed-up
    seq_out = [torch.empty_like(x) for x in out]
    for _ in range(2):
        pr.sequential(w.cell, u, a, s0, out=seq_out, stream=stream)
    sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(5)]
    for e0, e1 in sev:
        e0.record(stream)
        pr.sequential(w.cell, u, a, s0, out=seq_out, stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    seq_ms = sorted(e0.elapsed_time(e1) for e0, e1 in sev)[len(sev) // 2]
    res["gpu_sequential"] = {"ms": seq_ms, "elem_per_s": w.N / (seq_ms * 1e-3),
                             "newton_kernel_speedup": seq_ms / kernels[0]["ms_avg"],
                             "kind": "step-by-step application, one lane per channel"}
    del seq_out
    if headline and args.copy_mib:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = n * 4
    if headline and not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, inp)
    del u, a, s0, out, adj_out, gs, inp
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE,
                    help="the workload the line's value and roofline are quoted on "
                         f"(default {HEADLINE}, the largest)")
    ap.add_argument("--configs", default="all",
                    help="other workloads measured in the same run and nested under "
                         "'configs': all (default), none, or a comma list of keys")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed back-to-back steps before the warm-up steps, for this long "
                         "(ms of wall time), so that the GPU clocks reach their steady state")
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="size of the buffer written before every step of the roofline "
                         "region (evicts the 256 MB MALL); at least 512")
    ap.add_argument("--op", choices=["solve", "project", "scan", "checkpoint", "speedup"],
                    default="solve",
                    help="solve: the Newton solve (default); project: the input projection "
                         "u = W x + b for the workload's shapes with I = D inputs; scan: the "
                         "standalone linear-recurrence scan over the workload's channels; "
                         "checkpoint: a training step one-piece vs checkpointed in time "
                         "chunks (--chunk); speedup: Newton vs sequential application on "
                         "the same GPU, 64 channels, growing T")
    ap.add_argument("--chunk", type=int, default=512,
                    help="time chunk of --op checkpoint")
    ap.add_argument("--layout", choices=["channel", "time"], default="channel",
                    help="channel: [B][D][T] planes (default); time: the gate blocks of one "
                         "[B][T][G*D] projection tensor and [B][T][D] states (the headline "
                         "workload only)")
    ap.add_argument("--route", choices=["staged", "gather"], default="staged",
                    help="with --layout time: staged (planes copied channel-major through "
                         "the workspace, the default) or gather (a channel-major-size "
                         "workspace, every step loaded on its own)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the timed region, copy a buffer of this many MiB three "
                         "times (plain device copy used to calibrate HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on exactly one GPU (asked for {args.gpus}); "
              "channels are independent, so the path shards over B*D with no exchange, "
              "but no multi-GPU run is part of it.", file=sys.stderr)
        sys.exit(2)
    if args.flush_mib < 512:
        ap.error("--flush-mib must be at least 512 (twice the MALL)")

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    from nonlinear_rnn_amd import pararnn as pr  # noqa: F401  (fails loudly if not built)
    from nonlinear_rnn_amd.inputs import WORKLOADS

    w = WORKLOADS[args.workload]
    if args.op == "project":
        print(json.dumps(bench_project(w, args)), flush=True)
        return
    if args.op == "scan":
        print(json.dumps(bench_scan(w, args)), flush=True)
        return
    if args.op == "checkpoint":
        print(json.dumps(bench_checkpoint(w, args)), flush=True)
        return
    if args.op == "speedup":
        print(json.dumps(bench_speedup(args)), flush=True)
        return
    if args.configs == "all":
        others = [k for k in WORKLOADS if k != args.workload]
    elif args.configs == "none":
        others = []
    else:
        others = [k for k in args.configs.split(",") if k and k != args.workload]
        for k in others:
            if k not in WORKLOADS:
                ap.error(f"unknown workload {k!r}")
    flush_buf = torch.empty(args.flush_mib * (1 << 20) // 4, dtype=torch.float32,
                            device="cuda:0")
    head = measure_solve(w, args.workload, args, flush_buf, headline=True)
    print(f"bench.py: {args.workload} {head['ms_per_step']:.4f} ms/step, kernel "
          f"{head['kernels'][0]['ms_avg']:.4f} ms", file=sys.stderr, flush=True)
    nested = {}
    for key in others:
        r = measure_solve(WORKLOADS[key], key, args, flush_buf, headline=False)
        nested[key] = r
        print(f"bench.py: {key} {r['ms_per_step']:.4f} ms/step", file=sys.stderr, flush=True)

    time_major = args.layout == "time"
    dom = max(head["kernels"], key=lambda k: k["ms_avg"])
    traffic = measured_traffic(args.workload + (f"_time_major_{args.route}" if time_major else ""))
    line = {
        "metric": METRIC,
        "value": head["elem_per_s"],
        "unit": "elem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"ms": args.settle_ms, "steps": head["settle"]["steps"],
                   "kind": "untimed back-to-back steps before the warm-up, so that the "
                           "GPU clocks reach their steady state"},
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16-in/f32" if w.u_dtype == "bf16" else "f32",
        "data": data_recipe(w),
        "config": {"workload": w.name, "B": w.B, "T": w.T, "D": w.D, "tol": w.tol,
                   "layout": ("time-major: u gate blocks of one [B][T][G*D] tensor, "
                              f"states [B][T][D]; {args.route} route") if time_major else
                             "channel-major [B][D][T] planes",
                   "max_iters": w.max_iters, "seed": w.seed, "tiling": head["tiling"],
                   "newton_updates": head["newton_updates"],
                   "newton_updates_mean": head["newton_updates_mean"],
                   "converged": head["converged"], "max_abs_res": head["max_abs_res"]},
        # HBM is the roof the metric is quoted against: algorithmic bytes per
        # launch over the kernel's HIP-event average with the MALL evicted
        # before every launch; the VALU issue fraction rides along
        "roofline": {"bound": "hbm", "achieved": dom["achieved"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": dom["hbm_frac"], "traffic": traffic,
                     "algorithmic_bytes": dom["bytes"], "kernel": dom["kernel"],
                     "kernel_ms_avg": dom["ms_avg"], "kernel_ms_min": dom["ms_min"],
                     "kernel_ms_avg_back_to_back": dom["ms_avg_back_to_back"],
                     "timing": f"HIP events on the launch stream, {args.steps} launches, "
                               f"a {args.flush_mib} MiB write before each (outside the "
                               "event pair)",
                     "valu": dom.get("valu")},
        "kernels": head["kernels"],
        "gpu_sequential": head["gpu_sequential"],
        "configs": {args.workload: {k: head[k] for k in ("workload", "ms_per_step", "elem_per_s",
                                                         "newton_updates_mean", "kernels")}},
    }
    for key, r in nested.items():
        line["configs"][key] = r
    if "copy_calibration_bytes" in head:
        line["copy_calibration_bytes"] = head["copy_calibration_bytes"]
    if "cpu_baseline" in head:
        line["cpu_baseline"] = head["cpu_baseline"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
