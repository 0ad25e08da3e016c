"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on the
same seeded inputs.  Dequantized values must be bit-exact; GEMV outputs must
satisfy |y_gpu - y_oracle| <= 1e-4 * sum|w*x| + 1e-6 element by element.
Shapes span several work-group tiles, ragged row and unit tails, several K
chunks, 2-byte-aligned rows (Q6_K with K = 768, Q8_0 with an odd block count)
and the degenerate cases (one block, one row, N = 0)."""
import sys

from fractions import Fraction

import numpy as np
import pytest

import kqsynth
import oracle

torch = pytest.importorskip("torch")
import dequant_gemv_gguf_amd as kq  # noqa: E402

pytestmark = pytest.mark.gpu

TYPES = [kqsynth.Q4_K, kqsynth.Q6_K, kqsynth.Q2_K, kqsynth.Q8_0, kqsynth.Q4_0, kqsynth.Q5_K, kqsynth.Q3_K]
TOL_REL, TOL_ABS = 1e-4, 1e-6


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def qmat(qtype, N, K, seed):
    return kqsynth.matrix(qtype, N, K, kqsynth.rng_for(seed, qtype, N, K))


def gpu_gemv(qtype, W, N, K, x):
    M = x.shape[0]
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    kq.kq_qgemv(qtype, dev(W) if isinstance(W, np.ndarray) else W, N, K, dev(x), M, y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def check_close(y, yo, S, what=""):
    err = np.abs(y.astype(np.float64) - yo)
    bound = TOL_REL * S + TOL_ABS
    worst = float((err / bound).max()) if err.size else 0.0
    assert np.all(err <= bound), "%s: worst |dy|/bound = %.3g" % (what, worst)
    return worst


# ---- dequant: bit-exact -------------------------------------------------------

@pytest.mark.parametrize("qtype", TYPES)
@pytest.mark.parametrize("nblocks", [1, 3, 257, 1000])
def test_dequant_bit_exact(qtype, nblocks):
    say("dequant", kqsynth.TYPE_NAMES[qtype], nblocks)
    rng = kqsynth.rng_for(11, qtype, nblocks)
    blk = kqsynth.blocks(qtype, nblocks, rng)
    # plant fp16 subnormal and negative scales in a third of the blocks
    qk, nb, d_off, dmin_off = kqsynth.BLOCK[qtype]
    sub = rng.integers(1, 1024, size=nblocks).astype(np.uint16)
    sub[::2] |= 0x8000
    pick = np.arange(nblocks) % 3 == 0
    blk[pick, d_off:d_off + 2] = sub[pick].view(np.uint8).reshape(-1, 2)
    n = nblocks * qk
    ref = oracle.dequant(qtype, blk, n)
    out = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    kq.kq_dequant(qtype, dev(blk), n, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


# ---- qgemv: tolerance, over shapes and M ----------------------------------------

SHAPES = {
    kqsynth.Q4_K: [(1, 256), (7, 1280), (37, 4096), (130, 12544), (300, 2048)],
    kqsynth.Q6_K: [(1, 256), (9, 768), (37, 4096), (130, 12544), (70, 1280)],
    kqsynth.Q2_K: [(1, 256), (7, 1280), (37, 4096), (130, 12544), (300, 2048)],
    kqsynth.Q8_0: [(1, 32), (9, 1184), (37, 4096), (130, 12544), (70, 96)],
    kqsynth.Q4_0: [(1, 32), (9, 1184), (37, 4096), (130, 12544), (70, 96)],
    kqsynth.Q5_K: [(1, 256), (7, 1280), (37, 4096), (130, 12544), (300, 2048)],
    kqsynth.Q3_K: [(1, 256), (9, 768), (37, 4096), (130, 12544), (70, 1280)],
}


@pytest.mark.parametrize("qtype", TYPES)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
def test_qgemv_matches_oracle(qtype, M):
    worst = 0.0
    for (N, K) in SHAPES[qtype]:
        say("qgemv", kqsynth.TYPE_NAMES[qtype], "M", M, "N", N, "K", K)
        W = qmat(qtype, N, K, 1)
        x = kqsynth.activations(M, K, kqsynth.rng_for(2, M, K))
        y = gpu_gemv(qtype, W, N, K, x)
        yo, S = oracle.gemv(qtype, W, N, K, x)
        worst = max(worst, check_close(y, yo, S, "%s N=%d K=%d M=%d" % (kqsynth.TYPE_NAMES[qtype], N, K, M)))
    say("  worst |dy|/bound", worst)


@pytest.mark.parametrize("qtype", TYPES)
def test_qgemv_one_hot_is_bit_exact(qtype):
    # one nonzero product per output: every partial is exact, so y is the
    # dequantized column itself
    N, K = 45, 4096 + 256
    W = qmat(qtype, N, K, 3)
    dense = oracle.dequant(qtype, W, N * K).reshape(N, K)
    cols = [0, 1, 17, 63, 64, 255, 4100, K - 1]
    x = np.zeros((8, K), dtype=np.float32)
    for r, c in enumerate(cols):
        x[r, c] = 1.0
    y = gpu_gemv(qtype, W, N, K, x)
    for r, c in enumerate(cols):
        assert np.array_equal(y[r], dense[:, c]), (r, c)


@pytest.mark.parametrize("qtype", TYPES)
def test_qgemv_rows_do_not_depend_on_M_and_reruns_are_identical(qtype):
    N, K = 96, 12544
    W = dev(qmat(qtype, N, K, 4))
    x = kqsynth.activations(8, K, kqsynth.rng_for(4, 8))
    y8 = gpu_gemv(qtype, W, N, K, x)
    for m in range(8):
        y1 = gpu_gemv(qtype, W, N, K, x[m:m + 1])
        assert np.array_equal(y1[0].view(np.uint32), y8[m].view(np.uint32)), m
    for M in (3, 5):
        yM = gpu_gemv(qtype, W, N, K, x[:M])
        assert np.array_equal(yM.view(np.uint32), y8[:M].view(np.uint32))
    again = gpu_gemv(qtype, W, N, K, x)
    assert np.array_equal(again.view(np.uint32), y8.view(np.uint32))


def test_qgemv_degenerate_sizes():
    K = 256
    W = qmat(kqsynth.Q4_K, 1, K, 5)
    x = kqsynth.activations(1, K, kqsynth.rng_for(5))
    y = gpu_gemv(kqsynth.Q4_K, W, 1, K, x)
    yo, S = oracle.gemv(kqsynth.Q4_K, W, 1, K, x)
    check_close(y, yo, S)
    # N = 0 launches nothing and leaves y untouched
    yt = torch.full((1, 4), 7.0, device="cuda")
    kq.kq_qgemv(kqsynth.Q4_K, dev(W), 0, K, dev(x), 1, yt)
    torch.cuda.synchronize()
    assert torch.all(yt == 7.0)


def test_qgemv_zero_weights_and_large_activations():
    # zero scales give exact zeros whatever x holds; huge x stays finite
    K, N = 2048, 20
    W = qmat(kqsynth.Q4_K, N, K, 6).reshape(N, -1, 144).copy()
    W[:, :, 0:4] = 0                       # d = dmin = 0
    W = W.reshape(N, -1)
    x = (kqsynth.activations(2, K, kqsynth.rng_for(6)) * 1e30).astype(np.float32)
    y = gpu_gemv(kqsynth.Q4_K, W, N, K, x)
    assert np.all(y == 0)


# ---- grouped launch: several matrices sharing x ------------------------------------

MULTI = [
    # (type, K, row counts): small K packs several rows per step (segment
    # starts padded), more than 8 matrices take several launches, N = 0 is
    # skipped, 2-byte-aligned Q6_K/Q8_0 rows
    (kqsynth.Q4_K, 256, [7, 1, 5, 0, 13]),
    (kqsynth.Q4_K, 1280, [3, 64, 9]),
    (kqsynth.Q4_K, 4096, [37, 1, 130, 2, 5, 8, 3, 11, 4, 19]),
    (kqsynth.Q6_K, 768, [9, 70, 1]),
    (kqsynth.Q6_K, 12544, [30, 7, 12]),
    (kqsynth.Q2_K, 2048, [33, 300, 1]),
    (kqsynth.Q8_0, 1184, [9, 17, 4]),
    (kqsynth.Q8_0, 4096, [37, 5]),
    (kqsynth.Q4_0, 1184, [9, 17, 4]),
    (kqsynth.Q5_K, 4096, [37, 1, 130, 2, 5, 8, 3, 11, 4, 19]),
    (kqsynth.Q3_K, 768, [9, 70, 1]),
    (kqsynth.Q3_K, 12544, [30, 7, 12]),
]


@pytest.mark.parametrize("case", MULTI, ids=lambda c: "%s-K%d-%d" % (kqsynth.TYPE_NAMES[c[0]], c[1], len(c[2])))
@pytest.mark.parametrize("M", [1, 3, 8])
def test_qgemv_multi_equals_separate_calls(case, M):
    qtype, K, Ns = case
    say("qgemv_multi", kqsynth.TYPE_NAMES[qtype], "K", K, "Ns", Ns, "M", M)
    Ws = [qmat(qtype, max(n, 1), K, 40 + i)[:n] for i, n in enumerate(Ns)]
    x = kqsynth.activations(M, K, kqsynth.rng_for(41, M, K))
    Wd = [dev(w) if n else None for w, n in zip(Ws, Ns)]
    ys = [torch.full((M, n), float("nan"), device="cuda") if n else None for n in Ns]
    kq.kq_qgemv_multi(qtype, Wd, Ns, K, dev(x), M, ys)
    torch.cuda.synchronize()
    for i, n in enumerate(Ns):
        if n == 0:
            continue
        got = ys[i].cpu().numpy()
        one = gpu_gemv(qtype, Wd[i], n, K, x)
        assert np.array_equal(got.view(np.uint32), one.view(np.uint32)), i
        yo, S = oracle.gemv(qtype, Ws[i], n, K, x)
        check_close(got, yo, S, "matrix %d" % i)


MIXED = [
    # (K, [(type, N), ...]): two K-quant formats share one launch at M = 1;
    # a third format, or Q8_0, goes through its own launches
    (4096, [(kqsynth.Q4_K, 37), (kqsynth.Q6_K, 9), (kqsynth.Q4_K, 130)]),
    (2048, [(kqsynth.Q6_K, 33), (kqsynth.Q2_K, 300), (kqsynth.Q4_K, 5), (kqsynth.Q6_K, 1)]),
    (1280, [(kqsynth.Q2_K, 7), (kqsynth.Q4_K, 64), (kqsynth.Q4_K, 3)]),
    (4096, [(kqsynth.Q8_0, 17), (kqsynth.Q4_K, 20), (kqsynth.Q6_K, 0)]),
    (768, [(kqsynth.Q6_K, 70), (kqsynth.Q2_K, 0), (kqsynth.Q4_K, 0)]),
    (4096, [(kqsynth.Q5_K, 37), (kqsynth.Q3_K, 9), (kqsynth.Q5_K, 130)]),
    (2048, [(kqsynth.Q3_K, 33), (kqsynth.Q6_K, 300), (kqsynth.Q5_K, 5), (kqsynth.Q2_K, 40),
            (kqsynth.Q4_K, 7)]),
    (1280, [(kqsynth.Q4_0, 7), (kqsynth.Q5_K, 64), (kqsynth.Q4_K, 3), (kqsynth.Q8_0, 5)]),
    (768, [(kqsynth.Q3_K, 70), (kqsynth.Q4_K, 9)]),
    # five stripes per row: each format would take the 16-wave configuration,
    # so the two go to launches of their own
    (20480, [(kqsynth.Q5_K, 40), (kqsynth.Q6_K, 21), (kqsynth.Q5_K, 7)]),
    # more matrices of one format than a launch takes: a mixed launch of 8 + 3,
    # then the remaining two in a grouped launch
    (2048, [(kqsynth.Q4_K, 3 + 5 * i) for i in range(10)] + [(kqsynth.Q6_K, 1 + 9 * i) for i in range(3)]),
]


@pytest.mark.parametrize("case", MIXED, ids=lambda c: "K%d-" % c[0] + "+".join(
    "%s%d" % (kqsynth.TYPE_NAMES[t], n) for t, n in c[1]))
@pytest.mark.parametrize("M", [1, 2])
def test_qgemv_multi_mixed_formats(case, M):
    K, mats = case
    say("qgemv_multi mixed K", K, mats, "M", M)
    if any(K % kqsynth.BLOCK[t][0] for t, _ in mats):
        pytest.skip("K does not suit every format")
    Ws = [qmat(t, max(n, 1), K, 50 + i)[:n] for i, (t, n) in enumerate(mats)]
    x = kqsynth.activations(M, K, kqsynth.rng_for(51, M, K))
    Wd = [dev(w) if n else None for w, (t, n) in zip(Ws, mats)]
    ys = [torch.full((M, n), float("nan"), device="cuda") if n else None for t, n in mats]
    kq.kq_qgemv_multi([t for t, _ in mats], Wd, [n for _, n in mats], K, dev(x), M, ys)
    torch.cuda.synchronize()
    for i, (t, n) in enumerate(mats):
        if n == 0:
            continue
        got = ys[i].cpu().numpy()
        one = gpu_gemv(t, Wd[i], n, K, x)
        assert np.array_equal(got.view(np.uint32), one.view(np.uint32)), i
        yo, S = oracle.gemv(t, Ws[i], n, K, x)
        check_close(got, yo, S, "matrix %d" % i)


@pytest.mark.parametrize("K,mats", [(8192, [(kqsynth.Q4_K, 1024), (kqsynth.Q6_K, 1024), (kqsynth.Q4_K, 8192)]),
                                    (8192, [(kqsynth.Q4_K, 20480), (kqsynth.Q6_K, 1024)]),
                                    (4096, [(kqsynth.Q4_K, 1024), (kqsynth.Q6_K, 1024), (kqsynth.Q4_K, 4096)]),
                                    (2048, [(kqsynth.Q4_K, 24000), (kqsynth.Q6_K, 3000)]),
                                    (1024, [(kqsynth.Q6_K, 6000), (kqsynth.Q4_K, 48000)]),
                                    (2048, [(kqsynth.Q5_K, 24000), (kqsynth.Q3_K, 3000)])],
                         ids=["70B-wk+wv+wq", "long-Q4_K", "8B-wk+wv+wq", "K2048-Q4_K+Q6_K", "K1024-Q6_K+Q4_K",
                              "K2048-Q5_K+Q3_K"])
def test_qgemv_multi_mixed_full_size(K, mats):
    # a 70B and an 8B layer's k, v and q projections in one launch (Q4_K,
    # Q6_K, Q4_K: the 8-wave configuration), and Q4_K rows too many for it
    # beside Q6_K rows (separate 16-wave launches); rows shorter than 64 units (two or
    # four rows per wave: the kernels with the lane count set at run time) in
    # launches too large for the small-launch kernel (over 20 MB), with and
    # without a Q4_K side
    say("qgemv_multi mixed full size", mats)
    Ws = [kqsynth.device_matrix(t, n, K, seed=70 + i, device="cuda") for i, (t, n) in enumerate(mats)]
    x = kqsynth.activations(1, K, kqsynth.rng_for(71))
    ys = [torch.empty((1, n), device="cuda") for _, n in mats]
    kq.kq_qgemv_multi([t for t, _ in mats], Ws, [n for _, n in mats], K, dev(x), 1, ys)
    torch.cuda.synchronize()
    for i, (t, n) in enumerate(mats):
        one = gpu_gemv(t, Ws[i], n, K, x)
        assert np.array_equal(ys[i].cpu().numpy().view(np.uint32), one.view(np.uint32)), i
        rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(n + i).integers(0, n, 30)]))
        Wr = Ws[i][torch.from_numpy(rows).cuda()].cpu().numpy()
        yo, S = oracle.gemv(t, Wr, len(rows), K, x)
        check_close(ys[i].cpu().numpy()[:, rows], yo, S, "matrix %d" % i)


@pytest.mark.parametrize("Ns,K,M", [([1024, 8192], 8192, 1), ([28672, 28672], 8192, 1), ([28672, 28672], 8192, 2),
                                    ([14336, 14336], 4096, 1)],
                         ids=["wk+wq", "w1+w3", "w1+w3-M2", "8B-w1+w3"])
def test_qgemv_multi_full_size_projections(Ns, K, M):
    # a 70B layer's k and q projections, or a 70B or 8B layer's gate and up
    # projections (Q4_K), in one launch as the bench issues them
    Ws = [kqsynth.device_matrix(kqsynth.Q4_K, n, K, seed=60 + i, device="cuda") for i, n in enumerate(Ns)]
    x = kqsynth.activations(M, K, kqsynth.rng_for(61, M))
    ys = [torch.empty((M, n), device="cuda") for n in Ns]
    kq.kq_qgemv_multi(kqsynth.Q4_K, Ws, Ns, K, dev(x), M, ys)
    torch.cuda.synchronize()
    for i, n in enumerate(Ns):
        one = gpu_gemv(kqsynth.Q4_K, Ws[i], n, K, x)
        assert np.array_equal(ys[i].cpu().numpy().view(np.uint32), one.view(np.uint32)), i
        rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(n).integers(0, n, 30)]))
        Wr = Ws[i][torch.from_numpy(rows).cuda()].cpu().numpy()
        yo, S = oracle.gemv(kqsynth.Q4_K, Wr, len(rows), K, x)
        check_close(ys[i].cpu().numpy()[:, rows], yo, S, "matrix %d" % i)


# ---- full-size shapes, sampled rows -----------------------------------------------

FULL = [
    ("70B w1", kqsynth.Q4_K, 28672, 8192),
    ("70B w2", kqsynth.Q6_K, 8192, 28672),
    ("70B wk", kqsynth.Q4_K, 1024, 8192),
    ("70B w1 Q2_K", kqsynth.Q2_K, 28672, 8192),
    ("70B w2 Q8_0", kqsynth.Q8_0, 8192, 28672),
    ("Q6_K K=40960", kqsynth.Q6_K, 3000, 40960),
    ("70B w1 Q5_K", kqsynth.Q5_K, 28672, 8192),
    ("70B w2 Q3_K", kqsynth.Q3_K, 8192, 28672),
    ("70B w1 Q4_0", kqsynth.Q4_0, 28672, 8192),
    ("70B wo", kqsynth.Q4_K, 8192, 8192),
    ("8B wo", kqsynth.Q4_K, 4096, 4096),
    ("8B w2", kqsynth.Q6_K, 4096, 14336),
]


@pytest.mark.parametrize("name,qtype,N,K", FULL)
@pytest.mark.parametrize("M", [1, 8])
def test_full_size_sampled_rows(name, qtype, N, K, M):
    say("full", name, "M", M)
    W = kqsynth.device_matrix(qtype, N, K, seed=1234 + qtype, device="cuda")
    x = kqsynth.activations(M, K, kqsynth.rng_for(7, M, K))
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    kq.kq_qgemv(qtype, W, N, K, dev(x), M, y)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, N - 1, N - 2], np.random.default_rng(N + K).integers(0, N, 60)]))
    Wr = W[torch.from_numpy(rows).cuda()].cpu().numpy()
    yo, S = oracle.gemv(qtype, Wr, len(rows), K, x)
    worst = check_close(y.cpu().numpy()[:, rows], yo, S, name)
    say("  worst |dy|/bound", worst)
    del W


# Q4_K batch-1 launches stream the weights through a ring in LDS when the ring
# fits beside the staged activations (K <= 13568); shapes at the edges of that
# path: two and four short rows per wave step, a ragged row count, three
# stripes of 15 waves, the longest rows that fit (a partial last stripe, 163456
# of 163840 LDS bytes) and the first that do not (register ring).  Each is
# checked on sampled rows against the oracle and bit for bit against the
# two-row kernel (a row's bits do not depend on M).
Q4K_RING = [(65536, 2048), (100003, 1024), (24000, 12288), (9000, 13568), (5000, 13824)]


@pytest.mark.parametrize("N,K", Q4K_RING)
def test_q4k_lds_ring_shapes(N, K):
    qtype = kqsynth.Q4_K
    say("q4k ring", N, K)
    W = kqsynth.device_matrix(qtype, N, K, seed=N + K, device="cuda")
    x = kqsynth.activations(2, K, kqsynth.rng_for(11, N, K))
    y1 = torch.empty((1, N), dtype=torch.float32, device="cuda")
    y2 = torch.empty((2, N), dtype=torch.float32, device="cuda")
    kq.kq_qgemv(qtype, W, N, K, dev(x[:1]), 1, y1)
    kq.kq_qgemv(qtype, W, N, K, dev(x), 2, y2)
    torch.cuda.synchronize()
    a, b = y1.cpu().numpy()[0], y2.cpu().numpy()[0]
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "M = 1 and M = 2 rows differ"
    rows = np.unique(np.concatenate([[0, 1, 2, 3, N - 1, N - 2], np.random.default_rng(N).integers(0, N, 40)]))
    Wr = W[torch.from_numpy(rows).cuda()].cpu().numpy()
    yo, S = oracle.gemv(qtype, Wr, len(rows), K, x[:1])
    worst = check_close(y1.cpu().numpy()[:, rows], yo, S, "Q4_K %dx%d" % (N, K))
    say("  worst |dy|/bound", worst)
    del W


# Q4_K at M = 2 with rows of 64 units or more in 1 or 2 stripes runs the
# LDS-ring kernel with both activation rows in registers: a 70B wk + wq group,
# wo, w1 + w3 with a ragged group, an 8B projection and a 3-row matrix; a
# 16384-column matrix (4 stripes: no LDS for the ring beside two staged rows),
# a short-row matrix and a 3-stripe one take the batch-M kernel.  Sampled rows against the oracle and every row bit for
# bit against M = 1.
Q4K_RING_M2 = [([1024, 8192], 8192), ([8192], 8192), ([28672, 28001], 8192), ([4096], 4096), ([2000], 16384),
               ([3], 8192), ([5001], 2048), ([3000], 12288)]


@pytest.mark.parametrize("Ns,K", Q4K_RING_M2)
def test_q4k_lds_ring_two_rows(Ns, K):
    qtype = kqsynth.Q4_K
    say("q4k ring M=2", Ns, K)
    Ws = [kqsynth.device_matrix(qtype, n, K, seed=77 + i, device="cuda") for i, n in enumerate(Ns)]
    x = kqsynth.activations(2, K, kqsynth.rng_for(12, K, len(Ns)))
    y1 = [torch.empty((1, n), dtype=torch.float32, device="cuda") for n in Ns]
    y2 = [torch.empty((2, n), dtype=torch.float32, device="cuda") for n in Ns]
    types = [qtype] * len(Ns)
    kq.kq_qgemv_multi(types, Ws, Ns, K, dev(x[:1]), 1, y1)
    kq.kq_qgemv_multi(types, Ws, Ns, K, dev(x), 2, y2)
    x1 = x[1:2].copy()
    y1b = [torch.empty((1, n), dtype=torch.float32, device="cuda") for n in Ns]
    kq.kq_qgemv_multi(types, Ws, Ns, K, dev(x1), 1, y1b)
    torch.cuda.synchronize()
    for i, n in enumerate(Ns):
        a = y2[i].cpu().numpy()
        assert np.array_equal(a[0].view(np.uint32), y1[i].cpu().numpy()[0].view(np.uint32)), "row 0 differs from M = 1"
        assert np.array_equal(a[1].view(np.uint32), y1b[i].cpu().numpy()[0].view(np.uint32)), "row 1 differs from M = 1"
        rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(n).integers(0, n, 30)]))
        Wr = Ws[i][torch.from_numpy(rows).cuda()].cpu().numpy()
        yo, S = oracle.gemv(qtype, Wr, len(rows), K, x)
        worst = check_close(a[:, rows], yo, S, "Q4_K M=2 %dx%d" % (n, K))
        say("  worst |dy|/bound", worst)


# ---- routed experts ---------------------------------------------------------------

def moe_inputs(qtype, E, N, K, T, k, seed, x_mode):
    rng = kqsynth.rng_for(seed, qtype, E, N, K)
    W = kqsynth.blocks(qtype, E * N * (K // kqsynth.BLOCK[qtype][0]), rng)
    ids, p = kqsynth.routing(T, k, E, kqsynth.rng_for(seed, 1))
    x = kqsynth.activations(T * (k if x_mode else 1), K, kqsynth.rng_for(seed, 2))
    return W, ids, p, x


def gpu_moe(qtype, W, E, N, K, ids, p, x, x_mode):
    T, k = ids.shape
    shape = (T, k, N) if p is None else (T, N)
    y = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    ws = None if p is None else torch.empty(kq.kq_qmoe_workspace_bytes(T, k, N) // 4, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    kq.kq_qmoe_gemv(qtype, W if not isinstance(W, np.ndarray) else dev(W), E, N, K, dev(ids),
                    None if p is None else dev(p), T, k, dev(x), x_mode, y, ws, flag)
    torch.cuda.synchronize()
    return y.cpu().numpy(), int(flag.item())


MOE_CASES = [
    # (qtype, E, N, K, T, k, x_mode): the MoE FFN shapes (gate/up Q4_K 768x2048,
    # down Q6_K 2048x768 with 630-byte rows) and smaller ragged ones
    (kqsynth.Q4_K, 128, 768, 2048, 1, 8, 0),
    (kqsynth.Q4_K, 128, 768, 2048, 8, 8, 0),
    (kqsynth.Q6_K, 128, 2048, 768, 1, 8, 1),
    (kqsynth.Q6_K, 128, 2048, 768, 8, 8, 1),
    (kqsynth.Q2_K, 16, 100, 512, 5, 4, 0),
    (kqsynth.Q8_0, 12, 70, 96, 3, 5, 1),
    # one token: the split-grid path, more slots than segments of a launch
    (kqsynth.Q2_K, 40, 300, 4096, 1, 16, 1),
    (kqsynth.Q8_0, 20, 33, 1184, 1, 3, 0),
    (kqsynth.Q6_K, 6, 5, 256, 1, 6, 0),
    (kqsynth.Q5_K, 24, 96, 2048, 4, 6, 0),
    (kqsynth.Q3_K, 24, 200, 768, 2, 8, 1),
    (kqsynth.Q4_0, 10, 40, 1184, 1, 4, 1),
    # 128 slots over 40 experts: the member scan across two waves, batches of 8
    (kqsynth.Q4_K, 40, 96, 512, 8, 16, 0),
    (kqsynth.Q6_K, 40, 64, 768, 8, 16, 1),
]


@pytest.mark.parametrize("case", MOE_CASES)
@pytest.mark.parametrize("combine", [False, True])
def test_qmoe_matches_oracle(case, combine):
    qtype, E, N, K, T, k, x_mode = case
    say("qmoe", kqsynth.TYPE_NAMES[qtype], E, N, K, T, k, x_mode, combine)
    W, ids, p, x = moe_inputs(qtype, E, N, K, T, k, 8, x_mode)
    pw = p if combine else None
    y, flag = gpu_moe(qtype, W, E, N, K, ids, pw, x, x_mode)
    yo, S, oflag = oracle.moe(qtype, W, E, N, K, ids, pw, x, x_mode)
    assert flag == 0 and oflag == 0
    check_close(y, yo, S, "qmoe")


def test_qmoe_single_slot_equals_qgemv_bits():
    qtype, E, N, K = kqsynth.Q4_K, 16, 768, 2048
    W, _, _, x = moe_inputs(qtype, E, N, K, 1, 1, 9, 0)
    Wd = dev(W.reshape(-1))
    per = N * kqsynth.row_bytes(qtype, K)
    for e in (0, 7, 15):
        y, _ = gpu_moe(qtype, Wd, E, N, K, np.array([[e]], np.int32), np.ones((1, 1), np.float32), x, 0)
        yg = gpu_gemv(qtype, Wd[e * per:(e + 1) * per], N, K, x)
        assert np.array_equal(y.view(np.uint32), yg.view(np.uint32))


def test_qmoe_shared_expert_groups_and_bad_ids():
    # every slot routes to one expert: a group of T*k = 40 slots served in
    # batches of up to 8 rows; then out-of-range ids give zeros and the flag
    qtype, E, N, K, T, k = kqsynth.Q6_K, 9, 64, 768, 5, 8
    W, _, p, x = moe_inputs(qtype, E, N, K, T, k, 10, 1)
    ids = np.full((T, k), 3, dtype=np.int32)
    y, flag = gpu_moe(qtype, W, E, N, K, ids, None, x, 1)
    yo, S, _ = oracle.moe(qtype, W, E, N, K, ids, None, x, 1)
    assert flag == 0
    check_close(y, yo, S, "shared expert")
    ids[1, 2] = E
    ids[4, 7] = -5
    y, flag = gpu_moe(qtype, W, E, N, K, ids, None, x, 1)
    yo, S, oflag = oracle.moe(qtype, W, E, N, K, ids, None, x, 1)
    assert flag == 1 and oflag == 1
    assert np.all(y[1, 2] == 0) and np.all(y[4, 7] == 0)
    check_close(y, yo, S, "bad ids")
    yc, flag = gpu_moe(qtype, W, E, N, K, ids, p, x, 1)
    yoc, Sc, _ = oracle.moe(qtype, W, E, N, K, ids, p, x, 1)
    check_close(yc, yoc, Sc, "bad ids combined")


@pytest.mark.parametrize("x_mode", [0, 1])
def test_qmoe_one_token_bad_ids_and_bits(x_mode):
    # one token: each slot equals a batch-1 product on its expert bit for bit;
    # out-of-range ids give zeros and the flag
    qtype, E, N, K, k = kqsynth.Q6_K, 10, 2048, 768, 8
    W, ids, p, x = moe_inputs(qtype, E, N, K, 1, k, 12, x_mode)
    Wd = dev(W.reshape(-1))
    ids[0, 2] = E + 3
    ids[0, 5] = -1
    y, flag = gpu_moe(qtype, Wd, E, N, K, ids, None, x, x_mode)
    assert flag == 1
    per = N * kqsynth.row_bytes(qtype, K)
    for j in range(k):
        e = ids[0, j]
        if e < 0 or e >= E:
            assert np.all(y[0, j] == 0)
            continue
        xr = x[j:j + 1] if x_mode else x[0:1]
        yg = gpu_gemv(qtype, Wd[e * per:(e + 1) * per], N, K, xr)
        assert np.array_equal(y[0, j].view(np.uint32), yg[0].view(np.uint32)), j
    yo, S, oflag = oracle.moe(qtype, W, E, N, K, ids, None, x, x_mode)
    assert oflag == 1
    check_close(y, yo, S, "one token")
    yc, _ = gpu_moe(qtype, Wd, E, N, K, ids, p, x, x_mode)
    yoc, Sc, _ = oracle.moe(qtype, W, E, N, K, ids, p, x, x_mode)
    check_close(yc, yoc, Sc, "one token combined")


def test_qmoe_slot_rows_do_not_depend_on_grouping():
    # a slot's output is bit-identical whether its expert is shared or not
    qtype, E, N, K, T, k = kqsynth.Q4_K, 32, 256, 2048, 8, 4
    W, ids, _, x = moe_inputs(qtype, E, N, K, T, k, 11, 0)
    Wd = dev(W.reshape(-1))
    ids[:, 0] = 5                        # expert 5 shared by all 8 tokens
    y, _ = gpu_moe(qtype, Wd, E, N, K, ids, None, x, 0)
    per = N * kqsynth.row_bytes(qtype, K)
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            yg = gpu_gemv(qtype, Wd[e * per:(e + 1) * per], N, K, x[t:t + 1])
            assert np.array_equal(y[t, j].view(np.uint32), yg[0].view(np.uint32)), (t, j)


@pytest.mark.parametrize("case", [(kqsynth.Q4_K, 128, 768, 2048, 8, 8, 0), (kqsynth.Q6_K, 128, 2048, 768, 8, 8, 1),
                                  (kqsynth.Q4_K, 20, 200, 1024, 8, 8, 0), (kqsynth.Q2_K, 9, 77, 512, 5, 6, 1)],
                         ids=["gate-up", "down", "few-experts", "ragged"])
def test_qmoe_tokens_together_equal_one_token_calls(case):
    # per-slot outputs of T tokens routed together (experts chosen by several
    # tokens are read once for all of them) equal, bit for bit, those of each
    # token routed alone, for one tensor and for two in one launch
    qtype, E, N, K, T, k, x_mode = case
    say("qmoe tokens together", kqsynth.TYPE_NAMES[qtype], E, N, K, T, k, x_mode)
    Ws = [moe_inputs(qtype, E, N, K, T, k, 40 + i, x_mode)[0] for i in range(2)]
    _, ids, _, x = moe_inputs(qtype, E, N, K, T, k, 40, x_mode)
    ids[T - 1, :] = ids[0, :]                          # two tokens with the same experts
    Wd = [dev(W.reshape(-1)) for W in Ws]
    ys = [torch.full((T, k, N), float("nan"), device="cuda") for _ in range(2)]
    kq.kq_qmoe_gemv_multi(qtype, Wd, E, N, K, dev(ids), T, k, dev(x), x_mode, ys, None)
    one, _ = gpu_moe(qtype, Wd[0], E, N, K, ids, None, x, x_mode)
    torch.cuda.synchronize()
    rows = x.shape[0] // T
    for t in range(T):
        xt = x[t * rows:(t + 1) * rows]
        for i in range(2):
            yt, _ = gpu_moe(qtype, Wd[i], E, N, K, ids[t:t + 1], None, xt, x_mode)
            assert np.array_equal(ys[i].cpu().numpy()[t].view(np.uint32), yt[0].view(np.uint32)), (t, i)
            if i == 0:
                assert np.array_equal(one[t].view(np.uint32), yt[0].view(np.uint32)), t
    yo, S, _ = oracle.moe(qtype, Ws[0], E, N, K, ids, None, x, x_mode)
    check_close(one, yo, S, "tokens together")


def fma_f32(a, b, c):
    """fp32 fused multiply-add, exact: a*b + c rounded once to nearest, ties
    to even (subnormals kept), from exact rational arithmetic."""
    q = Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c))
    if q == 0:
        neg = (np.signbit(a) != np.signbit(b)) and np.signbit(c)
        return np.float32(-0.0 if neg else 0.0)
    neg, q = q < 0, abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    ulp = max(e - 23, -149)
    scaled = q / Fraction(2) ** ulp
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = np.float32(float(n) * 2.0 ** ulp)
    return -v if neg else v


def test_fma_f32_helper():
    # the rounding helper itself: exact cases, ties, subnormals
    assert fma_f32(np.float32(3), np.float32(5), np.float32(1)) == 16
    one, eps = np.float32(1), np.float32(2.0 ** -24)
    assert fma_f32(one, eps, one) == 1                       # tie to even: stays 1
    assert fma_f32(one, np.float32(3 * 2.0 ** -24), one) == np.float32(1 + 2.0 ** -22)
    tiny = np.float32(2.0 ** -100)
    assert fma_f32(tiny, np.float32(2.0 ** -48), np.float32(0)) == np.float32(2.0 ** -148)    # subnormal, exact
    assert fma_f32(tiny, np.float32(2.0 ** -50), np.float32(0)) == 0                           # half the least: even
    assert fma_f32(tiny, np.float32(3 * 2.0 ** -51), np.float32(0)) == np.float32(2.0 ** -149)
    assert fma_f32(np.float32(-2), np.float32(0), np.float32(0)).tobytes() == np.float32(0).tobytes()
    rng = np.random.default_rng(3)
    for a, b, c in rng.standard_normal((200, 3)).astype(np.float32):
        ref = np.float32(np.float64(a) * np.float64(b) + np.float64(c))   # exact product, one f64 rounding
        got = fma_f32(a, b, c)
        assert abs(float(got) - float(ref)) <= abs(float(ref)) * 2.0 ** -23


@pytest.mark.parametrize("case", [(kqsynth.Q6_K, 20, 96, 768, 1, 8, 1), (kqsynth.Q6_K, 20, 200, 768, 3, 12, 1),
                                  (kqsynth.Q4_K, 12, 72, 512, 2, 6, 0), (kqsynth.Q2_K, 40, 40, 4096, 1, 16, 1)],
                         ids=["one-launch", "k12-two-slots-per-wave", "shared-x", "two-launch"])
def test_qmoe_combine_bits(case):
    # the routing-weighted sum equals the per-slot outputs summed in ascending
    # slot order, one fp32 fma per term from +0, bit for bit -- whether the
    # sum runs in the products' launch or in a second one (the last case's
    # activation rows do not fit the one-launch kernel); a bad id adds zero
    qtype, E, N, K, T, k, x_mode = case
    say("qmoe combine bits", kqsynth.TYPE_NAMES[qtype], E, N, K, T, k, x_mode)
    W, ids, p, x = moe_inputs(qtype, E, N, K, T, k, 14, x_mode)
    ids[T - 1, k - 1] = E
    Wd = dev(W.reshape(-1))
    ys, f1 = gpu_moe(qtype, Wd, E, N, K, ids, None, x, x_mode)
    y, f2 = gpu_moe(qtype, Wd, E, N, K, ids, p, x, x_mode)
    assert f1 == 1 and f2 == 1
    for t in range(T):
        for o in range(N):
            acc = np.float32(0)
            for j in range(k):
                acc = fma_f32(p[t, j], ys[t, j, o], acc)
            assert acc.tobytes() == y[t, o].tobytes(), (t, o)
    yo, S, _ = oracle.moe(qtype, W, E, N, K, ids, p, x, x_mode)
    check_close(y, yo, S, "combined")


@pytest.mark.parametrize("T,x_mode,count", [(1, 0, 2), (8, 0, 2), (3, 1, 3), (8, 0, 4)])
def test_qmoe_multi_equals_separate_calls(T, x_mode, count):
    # an MoE layer's gate and up projections (and more tensors of the same
    # shape) in one launch: each output equals its own call bit for bit
    qtype, E, N, K, k = kqsynth.Q4_K, 24, 160, 1024, 8
    Ws = [moe_inputs(qtype, E, N, K, T, k, 20 + i, x_mode)[0] for i in range(count)]
    _, ids, _, x = moe_inputs(qtype, E, N, K, T, k, 20, x_mode)
    ids[0, 1] = E + 1                                   # one bad id: zeros and the flag
    Wd = [dev(W.reshape(-1)) for W in Ws]
    ys = [torch.full((T, k, N), float("nan"), device="cuda") for _ in range(count)]
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    kq.kq_qmoe_gemv_multi(qtype, Wd, E, N, K, dev(ids), T, k, dev(x), x_mode, ys, flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 1
    for i in range(count):
        one, f1 = gpu_moe(qtype, Wd[i], E, N, K, ids, None, x, x_mode)
        assert f1 == 1
        assert np.array_equal(ys[i].cpu().numpy().view(np.uint32), one.view(np.uint32)), i
        assert np.all(ys[i].cpu().numpy()[0, 1] == 0)
        yo, S, _ = oracle.moe(qtype, Ws[i], E, N, K, ids, None, x, x_mode)
        check_close(ys[i].cpu().numpy(), yo, S, "tensor %d" % i)


def test_qmoe_slot_major_path_bits():
    # activation rows too large for the token-major kernel (k = 4 rows of
    # K = 8192 per token): the slot-major kernel serves the call, alone and
    # grouped, and every slot still equals a batch-1 product bit for bit
    qtype, E, N, K, T, k = kqsynth.Q4_K, 12, 96, 8192, 2, 4
    say("qmoe slot-major", E, N, K, T, k)
    Ws = [moe_inputs(qtype, E, N, K, T, k, 30 + i, 1)[0] for i in range(2)]
    _, ids, p, x = moe_inputs(qtype, E, N, K, T, k, 30, 1)
    ids[1, :] = ids[0, :]                               # both tokens share their experts
    Wd = [dev(W.reshape(-1)) for W in Ws]
    per = N * kqsynth.row_bytes(qtype, K)
    ys = [torch.full((T, k, N), float("nan"), device="cuda") for _ in range(2)]
    kq.kq_qmoe_gemv_multi(qtype, Wd, E, N, K, dev(ids), T, k, dev(x), 1, ys, None)
    torch.cuda.synchronize()
    for i in range(2):
        one, _ = gpu_moe(qtype, Wd[i], E, N, K, ids, None, x, 1)
        assert np.array_equal(ys[i].cpu().numpy().view(np.uint32), one.view(np.uint32)), i
        for t in range(T):
            for j in range(k):
                e = ids[t, j]
                yg = gpu_gemv(qtype, Wd[i][e * per:(e + 1) * per], N, K, x[t * k + j:t * k + j + 1])
                assert np.array_equal(one[t, j].view(np.uint32), yg[0].view(np.uint32)), (i, t, j)
    yc, _ = gpu_moe(qtype, Wd[0], E, N, K, ids, p, x, 1)
    yo, S, _ = oracle.moe(qtype, Ws[0], E, N, K, ids, p, x, 1)
    check_close(yc, yo, S, "slot-major combined")


def test_concurrent_host_threads_give_the_same_bits():
    # calls from several host threads on their own streams, with kernels that
    # raise their LDS limit (batch-M with long rows, routed experts at T = 8):
    # every result equals the single-threaded one bit for bit
    import threading
    cases = []
    for i, (qt, N, K, M) in enumerate([(kqsynth.Q4_K, 300, 28672, 8), (kqsynth.Q6_K, 200, 12544, 5),
                                       (kqsynth.Q4_K, 1000, 8192, 1), (kqsynth.Q2_K, 400, 16384, 3)]):
        W = dev(qmat(qt, N, K, 80 + i))
        x = dev(kqsynth.activations(M, K, kqsynth.rng_for(81, i)))
        cases.append((qt, N, K, M, W, x))
    ref = []
    for (qt, N, K, M, W, x) in cases:
        y = torch.empty((M, N), device="cuda")
        kq.kq_qgemv(qt, W, N, K, x, M, y)
        ref.append(y)
    torch.cuda.synchronize()
    errors = []

    def work(c):
        try:
            st = torch.cuda.Stream()
            qt, N, K, M, W, x = cases[c]
            outs = [torch.empty((M, N), device="cuda") for _ in range(6)]
            with torch.cuda.stream(st):
                for y in outs:
                    kq.kq_qgemv(qt, W, N, K, x, M, y, st)
            st.synchronize()
            for y in outs:
                if not torch.equal(y.view(torch.int32), ref[c].view(torch.int32)):
                    errors.append(c)
        except Exception as e:          # reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=work, args=(c,)) for c in range(len(cases)) for _ in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors


@pytest.mark.parametrize("qtype", [kqsynth.Q4_K, kqsynth.Q6_K, kqsynth.Q8_0, kqsynth.Q3_K])
@pytest.mark.parametrize("M", [1, 3])
def test_maximum_K(qtype, M):
    # K = 2^20, the largest K the calls accept: rows longer than any LDS
    # staging, served by the chunked kernel; K + one block is refused
    K, N = 1 << 20, 3
    say("max K", kqsynth.TYPE_NAMES[qtype], "M", M)
    W = qmat(qtype, N, K, 90)
    x = kqsynth.activations(M, K, kqsynth.rng_for(91, M))
    y = gpu_gemv(qtype, W, N, K, x)
    yo, S = oracle.gemv(qtype, W, N, K, x)
    check_close(y, yo, S, "K = 2^20")
    y1 = gpu_gemv(qtype, W, N, K, x[:1])
    assert np.array_equal(y1[0].view(np.uint32), y[0].view(np.uint32))
    with pytest.raises(kq.KQError) as e:
        kq.kq_qgemv(qtype, dev(W[:, :kq.kq_row_bytes(qtype, 256 if qtype != kqsynth.Q8_0 else 32)]), 1,
                    K + (256 if qtype != kqsynth.Q8_0 else 32), dev(x[:, :1024]), 1, torch.empty(1, 1, device="cuda"))
    assert e.value.status == -2


def test_qmoe_long_expert_rows():
    # Q4_K / Q6_K experts with rows of 4096 columns or more (the routed
    # kernels' longer K chunks), against the oracle slot by slot
    for qtype, E, N, K, T, k, x_mode in [(kqsynth.Q4_K, 12, 96, 8192, 2, 4, 1), (kqsynth.Q6_K, 6, 40, 4096, 3, 2, 0)]:
        W, ids, p, x = moe_inputs(qtype, E, N, K, T, k, 31, x_mode)
        y, flag = gpu_moe(qtype, W, E, N, K, ids, None, x, x_mode)
        yo, S, _ = oracle.moe(qtype, W, E, N, K, ids, None, x, x_mode)
        assert flag == 0
        check_close(y, yo, S, "qmoe %s K=%d" % (kqsynth.TYPE_NAMES[qtype], K))
