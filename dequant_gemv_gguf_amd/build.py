"""Build the gfx950 shared library libkqgemv.so in-tree with hipcc.

All HIP code is compiled with packed fp32 instructions disabled: hipcc would
otherwise form v_pk_{add,mul,fma}_f32 from ordinary float code."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "kqgemv.hip")
INC = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libkqgemv.so")
ARCH = os.environ.get("KQ_OFFLOAD_ARCH", "gfx950")

FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def build(verbose=False, extra=()):
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc] + FLAGS + list(extra) + ["-I", INC, SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
