"""Build the gfx950 shared library libkqgemv.so in-tree with hipcc.

The library is several objects compiled in parallel: the C ABI
(csrc/kqgemv.hip), the GGUF reader and the host-streamed calls (csrc/kq_gguf.cpp,
csrc/kq_stream.cpp, host code), and csrc/kq_inst.hip once per block format and once per
pair of K-quant formats served by one mixed launch (each instantiates the
launchers and kernels of its format or pair).  They are linked with
--no-undefined, so an instantiation missing from the lists below fails the
build.

All HIP code is compiled with packed fp32 instructions disabled: hipcc would
otherwise form v_pk_{add,mul,fma}_f32 from ordinary float code.  The target
feature has to reach the device compile through -Xclang (the clang driver
forwards no -Xclang option through -Xarch_device), so the host pass sees it
too and prints that x86 does not know it; that line is harmless and is
dropped from the build log."""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INC = os.path.join(ROOT, "include")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkqgemv.so")
# the measurement kernels (include/kqprobe.h), a library of their own
PROBE_LIB = os.path.join(HERE, "libkqprobe.so")
ARCH = os.environ.get("KQ_OFFLOAD_ARCH", "gfx950")

FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # the first dwords of every kernel's arguments (the batch-1 kernels
         # put the activation pointer, K and the thread count there, the
         # routed-expert kernel the activation and expert-id pointers, K, k,
         # the activation mode and the token count) arrive in SGPRs at wave
         # launch, so the first loads need no scalar load before them; a
         # kernel keeps a prologue that loads them itself where the firmware
         # does not preload
         "-mllvm", "-amdgpu-kernarg-preload-count=8",
         "-Wall", "-Wno-unused-function"]

# what the host (x86) pass prints for the device-only target feature above
HOST_FEATURE_NOTE = "'-packed-fp32-ops' is not a recognized feature for this target"

# GGUF type ids of the formats, and the K-quant pairs (lower id first) that
# kq_impl.h declares mixed launchers for.
TYPES = (2, 8, 10, 11, 12, 13, 14)
PAIRS = ((10, 11), (10, 12), (10, 13), (10, 14), (11, 12), (11, 13), (11, 14),
         (12, 13), (12, 14), (13, 14))


def units():
    """(object name, source, defines) of every object of the library."""
    out = [("kqgemv", "kqgemv.hip", []), ("kq_gguf", "kq_gguf.cpp", []), ("kq_stream", "kq_stream.cpp", []),
           ("kq_mc", "kq_mc.hip", []),
           ("kq_probe", "kq_probe.hip", []), ("kq_stamps", "kq_stamps.hip", [])]
    out += [("kq_type%d" % t, "kq_inst.hip", ["-DKQ_INST_TYPE=%d" % t]) for t in TYPES]
    out += [("kq_mixed%d_%d" % p, "kq_inst.hip", ["-DKQ_INST_A=%d" % p[0], "-DKQ_INST_B=%d" % p[1]])
            for p in PAIRS]
    return out


def _jobs():
    for var in ("MAX_JOBS", "CMAKE_BUILD_PARALLEL_LEVEL"):
        v = os.environ.get(var, "")
        if v.isdigit() and int(v) > 0:
            return min(int(v), 16)
    return max(1, min(os.cpu_count() or 1, 16))


def build(verbose=False, extra=()):
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    os.makedirs(OBJ, exist_ok=True)
    cmds, objs = [], []
    for name, src, defs in units():
        o = os.path.join(OBJ, name + ".o")
        objs.append(o)
        # a fixed compilation-unit id (clang derives it from the source path
        # otherwise): the library's bytes do not depend on where it is built
        cuid = ["-cuid=kq_" + name]
        cmds.append([hipcc] + FLAGS + cuid + list(extra) + defs + ["-I", INC, "-c", os.path.join(CSRC, src), "-o", o])

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        out = "".join(line for line in r.stdout.splitlines(True) if HOST_FEATURE_NOTE not in line)
        return cmd, r.returncode, out

    failed = []
    with concurrent.futures.ThreadPoolExecutor(_jobs()) as pool:
        for cmd, rc, out in pool.map(run, cmds):
            if out.strip() and (verbose or rc):
                print(out, end="" if out.endswith("\n") else "\n", flush=True)
            if rc:
                failed.append(cmd)
    if failed:
        raise subprocess.CalledProcessError(1, failed[0])
    probe = [o for o in objs if o.endswith(("kq_probe.o", "kq_stamps.o"))]
    for lib, parts in ((LIB, [o for o in objs if o not in probe]), (PROBE_LIB, probe)):
        tmp = lib + ".tmp%d" % os.getpid()
        link = [hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-Wl,--no-undefined"] + parts + ["-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.check_call(link)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
