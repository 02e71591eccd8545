"""Build tests/c_abi_check (test infrastructure): a C++ consumer of
libpararnn.so through its C ABI alone, checked against liboracle.so.
Host code only; hipcc links the HIP runtime.  Run by
tests/test_gpu_c_abi.py."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_abi_check.cpp")
EXE = os.path.join(HERE, "c_abi_check")


def build(verbose: bool = False) -> str:
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    from nonlinear_rnn_amd import build as hip_build
    tmp = EXE + ".tmp"
    cmd = ["/opt/rocm/bin/hipcc", *hip_build.compile_flags(), SRC, "-o", tmp,
           "-L" + os.path.join(ROOT, "nonlinear_rnn_amd"), "-lpararnn",
           "-L" + os.path.join(ROOT, "oracle"), "-loracle",
           "-Wl,-rpath,$ORIGIN/../nonlinear_rnn_amd", "-Wl,-rpath,$ORIGIN/../oracle"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(ln for ln in res.stdout.splitlines()
                    if "is not a recognized feature for this target" not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
