"""The 16x16x32 and 16x16x16 f16 matrix instructions of gfx950, as the
matrix-core verify kernels use them.  These tests pin the lane layouts the
kernels rest on -- A row i = lane % 16 holding k = kw * (lane // 16) .. + kw - 1
(kw = 8 or 4), B column j = lane % 16 holding the same k, and D element r of
lane l = D[4 * (l // 16) + r][l % 16] -- that fp16 subnormal B inputs (the
kernels pass quants as the subnormals q * 2^-24) are used as they are, and how
close a sum of random products comes to the exact one."""
import ctypes
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "dequant_gemv_gguf_amd", "libkqprobe.so")


@pytest.fixture(scope="module")
def probe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L = ctypes.CDLL(PROBE)
    P = ctypes.c_void_p
    L.kqp_mfma16.argtypes = [P, P, P, P, ctypes.c_int, P]
    return L


def run(L, a, b, c, k32):
    """a, b: [64][8] lane operands (fp16 values or raw uint16 patterns); c: [64][4]."""
    def dev16(v):
        v = np.asarray(v)
        if v.dtype == np.uint16:
            return torch.from_numpy(v.view(np.int16).copy()).cuda()
        return torch.from_numpy(v.astype(np.float16).view(np.int16)).cuda()
    A, B = dev16(a), dev16(b)
    C = torch.from_numpy(np.asarray(c, dtype=np.float32)).cuda()
    D = torch.empty((64, 4), dtype=torch.float32, device="cuda")
    assert L.kqp_mfma16(A.data_ptr(), B.data_ptr(), C.data_ptr(), D.data_ptr(), int(k32), None) == 0
    torch.cuda.synchronize()
    return D.cpu().numpy()


def matrices(a, b, c, kw):
    """The A [16][16kw/4], B, C [16][16] that the lane operands stand for under
    the layout above, and D = A.B + C in exact integer (or fp64) arithmetic."""
    K = 4 * kw
    A = np.zeros((16, K))
    B = np.zeros((K, 16))
    for l in range(64):
        for s in range(kw):
            A[l % 16, kw * (l // 16) + s] = a[l][s]
            B[kw * (l // 16) + s, l % 16] = b[l][s]
    Cm = np.zeros((16, 16))
    for l in range(64):
        for r in range(4):
            Cm[4 * (l // 16) + r, l % 16] = c[l][r]
    return A, B, Cm


def lanes_of(Dm):
    out = np.zeros((64, 4))
    for l in range(64):
        for r in range(4):
            out[l, r] = Dm[4 * (l // 16) + r, l % 16]
    return out


@pytest.mark.parametrize("k32", [1, 0])
def test_layout_exact_integers(probe, k32):
    kw = 8 if k32 else 4
    rng = np.random.default_rng(7 + k32)
    a = np.zeros((64, 8))
    b = np.zeros((64, 8))
    a[:, :kw] = rng.integers(-16, 17, size=(64, kw))
    b[:, :kw] = rng.integers(-16, 17, size=(64, kw))
    c = rng.integers(-1000, 1001, size=(64, 4)).astype(np.float64)
    A, B, Cm = matrices(a, b, c, kw)
    want = lanes_of(A @ B + Cm)
    got = run(probe, a, b, c, k32)
    assert np.array_equal(got, want.astype(np.float32))


@pytest.mark.parametrize("k32", [1, 0])
def test_subnormal_b_is_used_as_is(probe, k32):
    # B = q * 2^-24 (q < 1024: fp16 subnormal patterns), A integers: every
    # product and sum is a multiple of 2^-24 below 2^-1, so exact in fp32
    kw = 8 if k32 else 4
    rng = np.random.default_rng(11 + k32)
    a = np.zeros((64, 8))
    a[:, :kw] = rng.integers(-2048, 2049, size=(64, kw))
    q = np.zeros((64, 8), dtype=np.uint16)
    q[:, :kw] = rng.integers(0, 1024, size=(64, kw))
    c = np.zeros((64, 4))
    A, B, Cm = matrices(a, q.astype(np.float64) * 2.0 ** -24, c, kw)
    want = lanes_of(A @ B)
    got = run(probe, a, q, c, k32)
    assert np.array_equal(got, want.astype(np.float32))
    assert np.count_nonzero(got) > 60


@pytest.mark.parametrize("k32", [1, 0])
def test_random_sum_close_to_exact(probe, k32):
    # a sum of kw * 4 products of random fp16 values plus C, against fp64:
    # within 2^-20 of sum |a*b| + |c| (recorded, not a rounding model)
    kw = 8 if k32 else 4
    rng = np.random.default_rng(13 + k32)
    a = np.zeros((64, 8))
    b = np.zeros((64, 8))
    a[:, :kw] = rng.standard_normal((64, kw)).astype(np.float16)
    b[:, :kw] = rng.standard_normal((64, kw)).astype(np.float16)
    c = rng.standard_normal((64, 4)).astype(np.float32).astype(np.float64)
    A, B, Cm = matrices(a, b, c, kw)
    want = lanes_of(A @ B + Cm)
    mag = lanes_of(np.abs(A) @ np.abs(B) + np.abs(Cm))
    got = run(probe, a, b, c, k32).astype(np.float64)
    err = np.abs(got - want) / mag
    print("16x16x%d: worst |D - exact| / (sum|a*b| + |c|) = 2^%.1f" % (4 * kw, np.log2(err.max() + 1e-300)))
    assert err.max() <= 2.0 ** -20
