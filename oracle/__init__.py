"""CPU oracle for the fused K-quant dequant-GEMV -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import this package.  The GPU library never uses it and
shares no code with it.  The arithmetic lives in ``kq_oracle.c`` (plain C,
fp64 dots, exact integer weight numerators); this module only loads the shared
object and marshals numpy arrays.

Pinned against closed forms, exactly representable round trips, a library
(numpy fp64) cross-check and brute force in ``tests/test_oracle.py``.  What is
NOT pinned: agreement with real GGUF files (there are none to compare with);
the byte layouts follow the GGUF K-quant convention, a reading.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kq_oracle.c")
_LIB = os.path.join(_HERE, "libkq_oracle.so")
# The pin tests can be pointed at another build of the oracle (a copy with a
# planted mistake, which they must reject); it is loaded as given, not built.
_LIB_OVERRIDE = os.environ.get("KQ_ORACLE_LIB")

Q4_0, Q8_0, Q2_K, Q3_K, Q4_K, Q5_K, Q6_K = 2, 8, 10, 11, 12, 13, 14

_lib = None


def build(force=False):
    """Compile the oracle with gcc (plain -O2, OpenMP over output rows)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-shared", "-fPIC",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            build()
            lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.oracle_block_shape.argtypes = [ctypes.c_int, P, P]
        lib.oracle_dequant.argtypes = [ctypes.c_int, P, i64, P]
        lib.oracle_gemv.argtypes = [ctypes.c_int, P, i64, i64, P, ctypes.c_int, P, P]
        lib.oracle_moe.argtypes = [ctypes.c_int, P, i64, i64, i64, P, P, ctypes.c_int,
                                   ctypes.c_int, P, ctypes.c_int, P, P, P]
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def block_shape(qtype):
    qk, nb = ctypes.c_int(), ctypes.c_int()
    if _load().oracle_block_shape(qtype, ctypes.byref(qk), ctypes.byref(nb)):
        raise ValueError("unknown quant type %r" % (qtype,))
    return qk.value, nb.value


def set_threads(n=0):
    """Set (n > 0) and return the OpenMP thread count the oracle uses."""
    return _load().oracle_set_threads(int(n))


def dequant(qtype, blocks, n):
    """Expand ``n`` weights from the packed bytes ``blocks`` to fp32."""
    src = np.ascontiguousarray(np.frombuffer(memoryview(blocks).cast("B"), dtype=np.uint8)
                               if not isinstance(blocks, np.ndarray) else blocks.view(np.uint8).reshape(-1))
    out = np.empty(int(n), dtype=np.float32)
    r = _load().oracle_dequant(qtype, _ptr(src), int(n), _ptr(out))
    if r:
        raise ValueError("oracle_dequant failed (%d)" % r)
    return out


def gemv(qtype, W, N, K, x):
    """Return (y, S): y[M][N] = x . W^T in fp64 and S = sum |w*x| in fp64."""
    src = np.ascontiguousarray(W.view(np.uint8).reshape(-1))
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, int(K))
    M = x.shape[0]
    y = np.empty((M, int(N)), dtype=np.float64)
    S = np.empty((M, int(N)), dtype=np.float64)
    r = _load().oracle_gemv(qtype, _ptr(src), int(N), int(K), _ptr(x), M, _ptr(y), _ptr(S))
    if r:
        raise ValueError("oracle_gemv failed (%d)" % r)
    return y, S


def moe(qtype, W_exps, E, N, K, ids, route_w, x, x_mode):
    """Routed-expert GEMV.  Returns (y, S, err_flag); y is [T][k][N] when
    route_w is None, else the routing-weighted sum [T][N]."""
    src = np.ascontiguousarray(W_exps.view(np.uint8).reshape(-1))
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    x = np.ascontiguousarray(x, dtype=np.float32)
    rw = None if route_w is None else np.ascontiguousarray(route_w, dtype=np.float32).reshape(T, k)
    shape = (T, k, int(N)) if rw is None else (T, int(N))
    y = np.empty(shape, dtype=np.float64)
    S = np.empty(shape, dtype=np.float64)
    flag = np.zeros(1, dtype=np.int32)
    r = _load().oracle_moe(qtype, _ptr(src), int(E), int(N), int(K), _ptr(ids), _ptr(rw), T, k,
                           _ptr(x), int(x_mode), _ptr(y), _ptr(S), _ptr(flag))
    if r:
        raise ValueError("oracle_moe failed (%d)" % r)
    return y, S, int(flag[0])
