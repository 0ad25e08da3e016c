"""GPU parity of the matrix-core verify GEMV (kq_qgemv_mc / kq_qgemv_mc_multi,
Q4_K and Q6_K) against the CPU oracle: every output within
1e-4 * sum|w*x| + 1e-6.  Shapes span ragged row tiles, K with fewer 256-column
blocks than the kernel's 8 waves and with a ragged last round of blocks,
2-byte-aligned Q6_K rows (an odd number of blocks), grids of more than 16 row
tiles per compute unit, grouped and two-format calls; the 70B verify shapes
are checked on sampled rows at M = 1, 2, 4 and 8.  A position's result must
not depend on M or on the other positions (bit for bit), a grouped call must
give each matrix's separate-call bits, and reruns must be identical."""
import sys

import numpy as np
import pytest

import kqsynth
import oracle

torch = pytest.importorskip("torch")
import dequant_gemv_gguf_amd as kq  # noqa: E402

pytestmark = pytest.mark.gpu

TOL_REL, TOL_ABS = 1e-4, 1e-6
MC_TYPES = [kqsynth.Q4_K, kqsynth.Q6_K]


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


def mc_gemv(qtype, W, N, K, x):
    M = x.shape[0]
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    kq.kq_qgemv_mc(qtype, W if isinstance(W, torch.Tensor) else dev(W), N, K,
                   x if isinstance(x, torch.Tensor) else dev(x), M, y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def check_close(y, yo, S, what=""):
    err = np.abs(y.astype(np.float64) - yo)
    bound = TOL_REL * S + TOL_ABS
    worst = float((err / bound).max()) if err.size else 0.0
    assert np.all(err <= bound), "%s: worst |dy|/bound = %.3g" % (what, worst)
    return worst


CASES = [(37, 256), (16, 512), (300, 768), (33, 1280), (129, 2048), (64, 2304), (250, 4096), (17, 4352),
         (1, 256), (40, 8192)]


@pytest.mark.parametrize("qtype", MC_TYPES)
@pytest.mark.parametrize("N,K", CASES)
@pytest.mark.parametrize("M", [1, 2, 3, 8])
def test_mc_matches_oracle(qtype, N, K, M):
    say("mc", kqsynth.TYPE_NAMES[qtype], N, K, M)
    W = kqsynth.matrix(qtype, N, K, kqsynth.rng_for(3, qtype, N, K))
    x = kqsynth.activations(M, K, kqsynth.rng_for(4, M, K))
    y = mc_gemv(qtype, W, N, K, x)
    yo, S = oracle.gemv(qtype, W, N, K, x)
    check_close(y, yo, S, "mc %s N=%d K=%d M=%d" % (kqsynth.TYPE_NAMES[qtype], N, K, M))


@pytest.mark.parametrize("qtype", MC_TYPES)
def test_mc_positions_do_not_depend_on_M_and_reruns_are_identical(qtype):
    N, K = 200, 3072
    W = dev(kqsynth.matrix(qtype, N, K, kqsynth.rng_for(5, qtype)))
    x = kqsynth.activations(8, K, kqsynth.rng_for(6, K))
    y8 = mc_gemv(qtype, W, N, K, x)
    assert np.array_equal(mc_gemv(qtype, W, N, K, x).view(np.uint32), y8.view(np.uint32))
    for M in (1, 2, 5):
        for p0 in (0, 8 - M):
            yM = mc_gemv(qtype, W, N, K, x[p0:p0 + M])
            assert np.array_equal(yM.view(np.uint32), y8[p0:p0 + M].view(np.uint32)), (M, p0)


def test_mc_extreme_activations():
    # one position zero, one with a huge dynamic range inside a block, one tiny
    qtype, N, K = kqsynth.Q4_K, 48, 1024
    W = kqsynth.matrix(qtype, N, K, kqsynth.rng_for(8, qtype))
    x = kqsynth.activations(4, K, kqsynth.rng_for(9, K))
    x[0] = 0.0
    x[1, ::97] *= 3.0e4
    x[2] *= 1.0e-30
    x[3, :256] = 0.0
    y = mc_gemv(qtype, W, N, K, x)
    yo, S = oracle.gemv(qtype, W, N, K, x)
    check_close(y, yo, S, "extreme")
    assert np.all(y[0] == 0.0)


def test_mc_many_tiles_per_compute_unit():
    # more than 16 row tiles per compute unit: extra work-groups beyond one per CU
    qtype, N, K = kqsynth.Q4_K, 70000, 256
    W = kqsynth.matrix(qtype, N, K, kqsynth.rng_for(10, qtype))
    x = kqsynth.activations(3, K, kqsynth.rng_for(11, K))
    y = mc_gemv(qtype, W, N, K, x)
    yo, S = oracle.gemv(qtype, W, N, K, x)
    check_close(y, yo, S, "many tiles")


@pytest.mark.parametrize("mats", [
    [(kqsynth.Q4_K, 1024), (kqsynth.Q4_K, 8192 // 8), (kqsynth.Q6_K, 1000)],
    [(kqsynth.Q6_K, 33), (kqsynth.Q4_K, 0), (kqsynth.Q4_K, 77)] + [(kqsynth.Q4_K, 16 * i + 3) for i in range(9)],
])
@pytest.mark.parametrize("M", [1, 4, 8])
def test_mc_multi_equals_separate_calls(mats, M):
    K = 2048
    x = kqsynth.activations(M, K, kqsynth.rng_for(12, M, K))
    xd = dev(x)
    Ws, ys, host = [], [], []
    for i, (qt, N) in enumerate(mats):
        Wh = kqsynth.matrix(qt, N, K, kqsynth.rng_for(13, i, qt, N)) if N else np.zeros(0, np.uint8)
        host.append(Wh)
        Ws.append(dev(Wh) if N else None)
        ys.append(torch.empty((M, N), dtype=torch.float32, device="cuda") if N else None)
    kq.kq_qgemv_mc_multi([qt for qt, _ in mats], Ws, [N for _, N in mats], K, xd, M, ys)
    torch.cuda.synchronize()
    for (qt, N), Wh, Wd, y in zip(mats, host, Ws, ys):
        if not N:
            continue
        alone = mc_gemv(qt, Wd, N, K, xd)
        assert np.array_equal(y.cpu().numpy().view(np.uint32), alone.view(np.uint32))
        yo, S = oracle.gemv(qt, Wh, N, K, x)
        check_close(y.cpu().numpy(), yo, S, "multi %s N=%d" % (kqsynth.TYPE_NAMES[qt], N))


FULL = [
    ("70B w1+w3", kqsynth.Q4_K, [28672, 28672], 8192),
    ("70B wk+wq", kqsynth.Q4_K, [1024, 8192], 8192),
    ("70B wv", kqsynth.Q6_K, [1024], 8192),
    ("70B wo", kqsynth.Q4_K, [8192], 8192),
    ("70B w2", kqsynth.Q6_K, [8192], 28672),
    ("8B w2", kqsynth.Q6_K, [4096], 14336),
]


@pytest.mark.parametrize("name,qtype,Ns,K", FULL)
@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_mc_full_size_sampled_rows(name, qtype, Ns, K, M):
    say("mc full", name, "M", M)
    Ws = [kqsynth.device_matrix(qtype, N, K, seed=4321 + i + qtype, device="cuda") for i, N in enumerate(Ns)]
    x = kqsynth.activations(M, K, kqsynth.rng_for(17, M, K))
    ys = [torch.empty((M, N), dtype=torch.float32, device="cuda") for N in Ns]
    kq.kq_qgemv_mc_multi(qtype, Ws, Ns, K, dev(x), M, ys)
    torch.cuda.synchronize()
    for N, W, y in zip(Ns, Ws, ys):
        rows = np.unique(np.concatenate([[0, 1, 15, 16, N - 1, N - 2],
                                         np.random.default_rng(N + K + M).integers(0, N, 40)]))
        Wr = W[torch.from_numpy(rows).cuda()].cpu().numpy()
        yo, S = oracle.gemv(qtype, Wr, len(rows), K, x)
        worst = check_close(y.cpu().numpy()[:, rows], yo, S, name)
        say("  worst |dy|/bound", worst)
    del Ws


def test_mc_argument_errors_launch_nothing():
    # kq_status: -1 type, -2 shape, -3 M, -4 NULL, -5 alignment
    K = 512
    W = dev(kqsynth.matrix(kqsynth.Q4_K, 8, K, kqsynth.rng_for(1)))
    x = dev(kqsynth.activations(2, K, kqsynth.rng_for(2)))
    y = torch.full((2, 8), 7.0, device="cuda")
    L = kq.lib()
    P = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    assert L.kq_qgemv_mc(kqsynth.Q2_K, P(W), 8, K, P(x), 2, P(y), None) == -1
    assert L.kq_qgemv_mc(kqsynth.Q4_K, P(W), 8, K, None, 2, P(y), None) == -4
    assert L.kq_qgemv_mc(kqsynth.Q4_K, P(W), 8, K, P(x), 9, P(y), None) == -3
    assert L.kq_qgemv_mc(kqsynth.Q4_K, P(W), 8, K + 32, P(x), 2, P(y), None) == -2
    assert L.kq_qgemv_mc(kqsynth.Q4_K, P(W), 8, K, P(x), 2, P(y) + 4, None) == -5
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


@pytest.mark.parametrize("M", [1, 4, 8])
def test_mc_two_formats_in_one_launch(M):
    # a layer's k, q (Q4_K) and v (Q6_K) at 70B shapes: one launch serves both
    # formats; each matrix keeps its separate-call bits
    K = 8192
    mats = [(kqsynth.Q4_K, 1024), (kqsynth.Q6_K, 1024), (kqsynth.Q4_K, 8192)]
    x = kqsynth.activations(M, K, kqsynth.rng_for(21, M, K))
    xd = dev(x)
    Ws = [kqsynth.device_matrix(qt, N, K, seed=77 + i, device="cuda") for i, (qt, N) in enumerate(mats)]
    ys = [torch.empty((M, N), dtype=torch.float32, device="cuda") for _, N in mats]
    kq.kq_qgemv_mc_multi([qt for qt, _ in mats], Ws, [N for _, N in mats], K, xd, M, ys)
    torch.cuda.synchronize()
    for (qt, N), W, y in zip(mats, Ws, ys):
        alone = mc_gemv(qt, W, N, K, xd)
        assert np.array_equal(y.cpu().numpy().view(np.uint32), alone.view(np.uint32)), kqsynth.TYPE_NAMES[qt]
        rows = np.unique(np.concatenate([[0, 15, 16, N - 1], np.random.default_rng(N + M).integers(0, N, 30)]))
        Wr = W[torch.from_numpy(rows).cuda()].cpu().numpy()
        yo, S = oracle.gemv(qt, Wr, len(rows), K, x)
        check_close(y.cpu().numpy()[:, rows], yo, S, "two formats %s N=%d" % (kqsynth.TYPE_NAMES[qt], N))


def test_mc_concurrent_host_threads_give_the_same_bits():
    # calls from several host threads on their own streams (every launch needs
    # more than 64 KB of LDS, a limit raised per kernel and device): each
    # result equals the single-threaded one bit for bit
    import threading
    cases = []
    for i, (qt, N, K, M) in enumerate([(kqsynth.Q4_K, 3000, 8192, 8), (kqsynth.Q6_K, 700, 28672, 4),
                                       (kqsynth.Q4_K, 64, 4096, 2), (kqsynth.Q6_K, 5000, 2048, 8)]):
        W = dev(kqsynth.matrix(qt, N, K, kqsynth.rng_for(30, i, qt)))
        x = dev(kqsynth.activations(M, K, kqsynth.rng_for(31, i)))
        cases.append((qt, N, K, M, W, x))
    ref = [mc_gemv(qt, W, N, K, x) for (qt, N, K, M, W, x) in cases]
    errors = []

    def work(c):
        try:
            st = torch.cuda.Stream()
            qt, N, K, M, W, x = cases[c]
            outs = [torch.empty((M, N), device="cuda") for _ in range(5)]
            with torch.cuda.stream(st):
                for y in outs:
                    kq.kq_qgemv_mc(qt, W, N, K, x, M, y, st)
            st.synchronize()
            for y in outs:
                if not np.array_equal(y.cpu().numpy().view(np.uint32), ref[c].view(np.uint32)):
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
