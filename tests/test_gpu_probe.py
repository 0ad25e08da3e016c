"""The measurement kernels of libkqprobe.so that run library code: the
stamped batch-1 passes (Q4_K's LDS ring, Q6_K's register ring) give the same
products as kq_qgemv_multi, bit for bit, and timestamps in phase order on real
XCDs."""
import ctypes
import os

import numpy as np
import pytest

import kqsynth

torch = pytest.importorskip("torch")
import dequant_gemv_gguf_amd as kq  # noqa: E402

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "dequant_gemv_gguf_amd", "libkqprobe.so")


@pytest.fixture(scope="module")
def probe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L = ctypes.CDLL(PROBE)
    P = ctypes.c_void_p
    L.kqp_stamped_qgemv1.argtypes = [ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int64, P, P, P, ctypes.c_int, P, P]
    return L


@pytest.mark.parametrize("qt,Ns,K", [(kqsynth.Q4_K, [8192], 8192), (kqsynth.Q4_K, [3000, 2001], 8192),
                                     (kqsynth.Q4_K, [1500], 4096), (kqsynth.Q6_K, [2000], 28672),
                                     (kqsynth.Q6_K, [700, 301], 20480)],
                         ids=["q4k-wo", "q4k-two-matrices", "q4k-one-stripe", "q6k-long-rows", "q6k-two-matrices"])
def test_stamped_pass_equals_the_library_and_orders_its_stamps(probe, qt, Ns, K):
    print("stamped", kqsynth.TYPE_NAMES[qt], Ns, K, flush=True)
    Ws = [kqsynth.device_matrix(qt, n, K, seed=60 + i, device="cuda") for i, n in enumerate(Ns)]
    x = torch.from_numpy(kqsynth.activations(1, K, kqsynth.rng_for(61, K))).cuda()
    ys = [torch.full((1, n), float("nan"), device="cuda") for n in Ns]
    ref = [torch.full((1, n), float("nan"), device="cuda") for n in Ns]
    stamps = torch.zeros((4096, 8), dtype=torch.int64, device="cuda")
    cnt = len(Ns)
    grid = ctypes.c_int(0)
    r = probe.kqp_stamped_qgemv1(qt, cnt, (ctypes.c_void_p * cnt)(*[W.data_ptr() for W in Ws]),
                              (ctypes.c_int64 * cnt)(*Ns), K, ctypes.c_void_p(x.data_ptr()),
                              (ctypes.c_void_p * cnt)(*[y.data_ptr() for y in ys]),
                              ctypes.c_void_p(stamps.data_ptr()), 4096, ctypes.byref(grid), None)
    assert r == 0
    kq.kq_qgemv_multi(qt, Ws, Ns, K, x, 1, ref)
    torch.cuda.synchronize()
    for y, yr in zip(ys, ref):
        assert np.array_equal(y.cpu().numpy().view(np.uint32), yr.cpu().numpy().view(np.uint32))
    g = grid.value
    assert 1 <= g <= 4096
    st = stamps.cpu().numpy()[:g]
    assert np.all(st[:, 0] > 0)
    assert np.all(np.diff(st[:, :4], axis=1) >= 0)
    assert np.all(st[:, 4] < 8)
    span_us = (st[:, 3].max() - st[:, 0].min()) * 0.01
    assert 0 < span_us < 10000
