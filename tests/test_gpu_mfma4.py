"""The 4x4x4 (16 blocks) f16 matrix instruction of gfx950, as the GEMV
kernels use it: lane l's own four weights as its row of A, its own four
activations as its column of B, so that element l % 4 of its result is its
own four-term dot product added to element l % 4 of its accumulator.  These
tests pin that property (on exact small integers and on random values), that
fp16 subnormal A inputs are used as they are (the kernels pass 4-bit quants as
the subnormals q * 2^-24), and record how the instruction rounds."""
import ctypes
import os
import sys

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
    L.kqp_mfma4.argtypes = [P, P, P, P, P]
    L.kqp_mfma4_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P]
    return L


def run(L, a, b, c):
    A = torch.from_numpy(a.astype(np.float16).reshape(64, 4)).cuda()
    B = torch.from_numpy(b.astype(np.float16).reshape(64, 4)).cuda()
    C = torch.from_numpy(c.astype(np.float32).reshape(64, 4)).cuda()
    D = torch.empty((64, 4), dtype=torch.float32, device="cuda")
    assert L.kqp_mfma4(A.data_ptr(), B.data_ptr(), C.data_ptr(), D.data_ptr(), None) == 0
    torch.cuda.synchronize()
    return D.cpu().numpy()


def diag(D):
    return D[np.arange(64), np.arange(64) % 4]


def test_diagonal_is_the_lanes_own_dot_exact_integers(probe):
    rng = np.random.default_rng(0)
    a = rng.integers(-8, 9, size=(64, 4))
    b = rng.integers(-8, 9, size=(64, 4))
    c = rng.integers(-100, 101, size=(64, 4))
    D = run(probe, a, b, c)
    want = (a * b).sum(axis=1) + c[np.arange(64), np.arange(64) % 4]
    assert np.array_equal(diag(D), want.astype(np.float32))
    # the whole result, for the record: lane 4q + j holds column j of block q
    blk = np.arange(64) // 4
    full = np.zeros((64, 4))
    for l in range(64):
        for i in range(4):
            r = 4 * blk[l] + i
            full[l, i] = (a[r] * b[l]).sum() + c[l, i]
    print("element i of lane 4q + j is row i, column j of block q:", np.array_equal(D, full), flush=True)


def test_subnormal_a_inputs_are_not_flushed(probe):
    rng = np.random.default_rng(1)
    q = rng.integers(0, 16, size=(64, 4))
    a = (q * 2.0 ** -24).astype(np.float16)           # exact fp16 subnormals
    assert np.all((a.astype(np.float64) == q * 2.0 ** -24))
    b = rng.standard_normal((64, 4)).astype(np.float16)
    c = np.zeros((64, 4))
    D = run(probe, a, b, c)
    exact = (q * 2.0 ** -24 * b.astype(np.float64)).sum(axis=1)
    # every product is exact in fp32 (4 + 11 significant bits); the sum of four
    # is within one rounding of the exact value
    got = diag(D).astype(np.float64)
    assert np.count_nonzero(got) == np.count_nonzero(exact)
    mag = (q * 2.0 ** -24 * np.abs(b.astype(np.float64))).sum(axis=1)
    rel = np.abs(got - exact) / np.where(mag > 0, mag, 1)
    print("mfma4 subnormal A: max |error| / sum|a*b| = 2^%.2f" % np.log2(max(rel.max(), 2.0 ** -60)), flush=True)
    assert np.all(rel <= 2.0 ** -16)


def test_rounding_of_the_sum(probe):
    # random halves and accumulators: compare with one rounding of the exact
    # sum, and with four fp32 fused multiply-adds in order k = 0..3
    rng = np.random.default_rng(2)
    hits_once, hits_seq, n, worst, worst_big = 0, 0, 0, 0.0, 0.0
    for t in range(20):
        a = rng.standard_normal((64, 4)).astype(np.float16)
        b = rng.standard_normal((64, 4)).astype(np.float16)
        c = (rng.standard_normal((64, 4)) * 4).astype(np.float32)
        D = diag(run(probe, a, b, c))
        cd = c[np.arange(64), np.arange(64) % 4].astype(np.float64)
        prod = a.astype(np.float64) * b.astype(np.float64)
        once = (cd + prod.sum(axis=1)).astype(np.float32)
        seq = cd.astype(np.float32)
        for k in range(4):
            seq = (seq.astype(np.float64) + prod[:, k]).astype(np.float32)
        hits_once += int(np.sum(D == once))
        hits_seq += int(np.sum(D == seq))
        n += 64
        err = np.abs(D.astype(np.float64) - (cd + prod.sum(axis=1)))
        mag = np.abs(cd) + np.abs(prod).sum(axis=1)
        worst = max(worst, float((err / mag).max())) if t else float((err / mag).max())
        # relative to the largest term instead
        big = np.maximum(np.abs(cd), np.abs(prod).max(axis=1))
        worst_big = max(worst_big, float((err / big).max())) if t else float((err / big).max())
        assert np.all(err <= mag * 2.0 ** -16)
    print("mfma4 rounding: equal to one rounding of the exact sum %d/%d, to sequential fp32 adds %d/%d; "
          "max |error| / (|c| + sum|a*b|) = 2^%.2f, / max term = 2^%.2f"
          % (hits_once, n, hits_seq, n, np.log2(worst), np.log2(worst_big)), flush=True)
    sys.stdout.flush()


def test_issue_rate(probe):
    sink = torch.empty(256 * 16 * 64, dtype=torch.int32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for chains in (1, 4, 8):
        for waves in (4, 16):
            iters = 4096
            assert probe.kqp_mfma4_rate(cus, waves, chains, iters, sink.data_ptr(), None) == 0
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            assert probe.kqp_mfma4_rate(cus, waves, chains, iters, sink.data_ptr(), None) == 0
            b.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b)
            n = cus * waves * chains * iters
            print("mfma4 rate: %d waves/CU, %d chains: %.1f G instr/s, %.2f instr/clk/CU at 2.4 GHz" % (
                waves, chains, n / ms / 1e6, n / (ms * 1e-3) / 2.4e9 / cus), flush=True)


def split_fp16(x):
    hi = x.astype(np.float16)
    lo = (x - hi.astype(np.float32)).astype(np.float16)
    return hi, lo


def test_a_rows_are_independent(probe):
    # the same activations in A rows 0 and 2 (and 1 and 3) give the same bits
    rng = np.random.default_rng(3)
    x = rng.standard_normal((16, 4)).astype(np.float32)
    hi, lo = split_fp16(x)
    a = np.zeros((64, 4), dtype=np.float16)
    for q in range(16):
        a[4 * q + 0], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3] = hi[q], lo[q], hi[q], lo[q]
    b = (rng.integers(0, 16, size=(64, 4)) + 1024).astype(np.float16)
    c = np.zeros((64, 4), dtype=np.float32)
    for it in range(8):
        c = run(probe, a, b, c)
    assert np.array_equal(c[:, 0].view(np.uint32), c[:, 2].view(np.uint32))
    assert np.array_equal(c[:, 1].view(np.uint32), c[:, 3].view(np.uint32))


@pytest.mark.parametrize("enc", ["subnormal", "offset1024"])
def test_chained_subblock_precision(probe, enc):
    # one 32-weight sub-block per lane row: 8 chained instructions of 4
    # weights, activations as fp16 hi/lo limbs in A rows 0 and 1; error of the
    # dot against the exact sum, relative to sum|q*x|
    rng = np.random.default_rng(4)
    worst, rms, n = 0.0, 0.0, 0
    for trial in range(8):
        q = rng.integers(0, 16, size=(8, 64, 4))        # [instr][lane][k]
        x = rng.standard_normal((8, 16, 4)).astype(np.float32)   # [instr][block][k]
        c = np.zeros((64, 4), dtype=np.float32)
        for it in range(8):
            hi, lo = split_fp16(x[it])
            a = np.zeros((64, 4), dtype=np.float16)
            for blk in range(16):
                a[4 * blk], a[4 * blk + 1] = hi[blk], lo[blk]
            if enc == "subnormal":
                b = (q[it] * 2.0 ** -24).astype(np.float16)
            else:
                b = (q[it] + 1024).astype(np.float16)
            c = run(probe, a, b, c)
        lane = np.arange(64)
        xs = x[:, lane // 4, :]                          # [instr][lane][k]
        xr = np.stack([split_fp16(x[i])[0].astype(np.float64)[lane // 4] +
                       split_fp16(x[i])[1].astype(np.float64)[lane // 4] for i in range(8)])
        got = c[:, 0].astype(np.float64) + c[:, 1].astype(np.float64)
        if enc == "subnormal":
            exact = (q * xr).sum(axis=(0, 2)) * 2.0 ** -24
            scale = (q * np.abs(xs)).sum(axis=(0, 2)) * 2.0 ** -24
        else:
            exact = (q * xr).sum(axis=(0, 2)) + 1024 * xr.sum(axis=(0, 2))
            got = got  # the offset is removed below in exact arithmetic
            scale = (q * np.abs(xs)).sum(axis=(0, 2))
            got = got - 1024 * xr.sum(axis=(0, 2))
            exact = exact - 1024 * xr.sum(axis=(0, 2))
        rel = np.abs(got - exact) / scale
        worst = max(worst, float(rel.max()))
        rms += float((rel ** 2).sum())
        n += rel.size
    print("chained sub-block, %s weights: max |err| / sum|q*x| = 2^%.2f, rms 2^%.2f" % (
        enc, np.log2(worst), np.log2(np.sqrt(rms / n))), flush=True)
