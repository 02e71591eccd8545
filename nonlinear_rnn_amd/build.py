"""Build libpararnn.so (HIP, gfx950) in-tree.

``python -m nonlinear_rnn_amd.build`` compiles the host ABI
(``csrc/pararnn.hip``) and the kernel instantiations (``csrc/inst_*.hip``,
one per cell and projection dtype, compiled in parallel) with hipcc and links
``nonlinear_rnn_amd/libpararnn.so``.  Packed FP32 instruction
selection is switched off for the device code; every kernel is written for
wave64 CDNA4 and needs no other target.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpararnn.so")
ARCH = os.environ.get("PARARNN_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libpararnn.so)")


def compile_flags():
    return ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


SOURCES = ["pararnn.hip", "inst_gru_f32.hip", "inst_gru_bf16.hip", "inst_gru_bf16_seq.hip",
           "inst_lstm_f32.hip", "inst_lstm_bf16.hip", "inst_scan.hip", "inst_seq.hip",
           "inst_project.hip"]

# Per-unit scheduler choice, by measurement: the block-sequential ParaGRU
# kernel on bf16 projections that the long, many-channel solves use runs 2%
# faster when the machine scheduler favours instruction-level parallelism
# over occupancy (B=4 T=16384 D=4096: 1.208 -> 1.182 ms per step); every
# other kernel keeps the default (with the ILP scheduler the float32 ParaGRU
# and the ParaLSTM kernels ran up to 17% slower, and other bf16 ParaGRU
# tilings spilled up to 24 registers).
EXTRA_FLAGS = {"inst_gru_bf16_seq.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "is not a recognized feature for this target" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every translation unit (in parallel) and link the library."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc] + compile_flags() + EXTRA_FLAGS.get(src, [])
                    + ["-c", os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or min(len(cmds), max(1, os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
