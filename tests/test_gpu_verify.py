"""GPU parity of the speculative-verify pass at its own shapes: one layer of
the Llama-3-70B-shaped model (wq/wo 8192x8192, wk/wv 1024x8192, w1/w3
28672x8192, w2 8192x28672) with M in {1, 2, 4, 8} activation rows, in the
Q4_K_M mix and re-encoded all-Q2_K and all-Q8_0, issued as the benchmark
issues it (k+q+v in one grouped call, wo, w1+w3 in one grouped call, w2).

Several positions verified in one pass of the weights is the speculative
step of the Kortex summary ("Out-of-core LLM inference engine written from
scratch in Rust", section Approach); Q2_K and Q8_0 are on the RunNburn post's
list of formats.  Each output is checked on sampled rows against the oracle
(|dy| <= 1e-4 * sum|w*x| + 1e-6) and every row bit for bit against M = 1
calls on the same activation row: a verify pass must give each position the
bits the plain pass gives it.

Also here: batch-M launches in which every wave makes more than one row step
(rows beyond 8 waves x compute units x 2) for the formats whose register
ring the 70B verify shapes do not reach at M = 3, and a two-format launch of
short rows (fewer than 64 units) large enough for the persistent kernel."""
import sys

import numpy as np
import pytest

import kqsynth
import oracle

torch = pytest.importorskip("torch")
import dequant_gemv_gguf_amd as kq  # noqa: E402

pytestmark = pytest.mark.gpu

TOL_REL, TOL_ABS = 1e-4, 1e-6


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_close(y, yo, S, what=""):
    err = np.abs(y.astype(np.float64) - yo)
    bound = TOL_REL * S + TOL_ABS
    worst = float((err / bound).max()) if err.size else 0.0
    assert np.all(err <= bound), "%s: worst |dy|/bound = %.3g" % (what, worst)
    return worst


def sample_rows(N, seed, extra=40):
    fixed = [0, 1, N // 2, N - 2, N - 1]
    return np.unique(np.concatenate([fixed, np.random.default_rng(seed).integers(0, N, extra)]))


def layer_groups(quant):
    """The 70B layer in the benchmark's call order, grouped by shared input."""
    spec = kqsynth.LLAMA3_70B
    layer = kqsynth.dense_layer(spec["hidden"], spec["ffn"], spec["kv"])
    if quant is not None:
        layer = kqsynth.reencode(layer, quant)
    by = {name: t for t in layer for name in [t[0]]}
    return [[by["wv"], by["wk"], by["wq"]], [by["wo"]], [by["w1"], by["w3"]], [by["w2"]]]


def run_group(grp, Ws, x, M):
    ys = [torch.full((M, N), float("nan"), device="cuda") for (_, _, N, _) in grp]
    K = grp[0][3]
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    if len(grp) == 1:
        kq.kq_qgemv(grp[0][1], Ws[0], grp[0][2], K, xd, M, ys[0])
    else:
        kq.kq_qgemv_multi([t for (_, t, _, _) in grp], Ws, [N for (_, _, N, _) in grp], K, xd, M, ys)
    return ys


@pytest.mark.parametrize("quant", [None, kqsynth.Q2_K, kqsynth.Q8_0], ids=["q4_k_m", "q2_k", "q8_0"])
@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_verify_layer_as_the_benchmark_issues_it(quant, M):
    worst = 0.0
    for gi, grp in enumerate(layer_groups(quant)):
        K = grp[0][3]
        say("verify", "q4_k_m" if quant is None else kqsynth.TYPE_NAMES[quant], "M", M, "group",
            "+".join(n for (n, _, _, _) in grp), "K", K)
        Ws = [kqsynth.device_matrix(t, N, K, seed=9000 + 10 * gi + i, device="cuda")
              for i, (_, t, N, _) in enumerate(grp)]
        x = kqsynth.activations(M, K, kqsynth.rng_for(90, gi, M))
        ys = run_group(grp, Ws, x, M)
        # the same matrices one activation row at a time
        ones = [run_group(grp, Ws, x[m:m + 1], 1) for m in range(M)] if M > 1 else None
        torch.cuda.synchronize()
        for i, (name, t, N, _) in enumerate(grp):
            got = ys[i].cpu().numpy()
            if ones is not None:
                for m in range(M):
                    one = ones[m][i].cpu().numpy()[0]
                    assert np.array_equal(got[m].view(np.uint32), one.view(np.uint32)), \
                        "%s row %d differs from its M = 1 call" % (name, m)
            rows = sample_rows(N, N + K + gi + i)
            Wr = Ws[i][torch.from_numpy(rows).cuda()].cpu().numpy()
            yo, S = oracle.gemv(t, Wr, len(rows), K, x)
            worst = max(worst, check_close(got[:, rows], yo, S, "%s %s M=%d" % (
                name, kqsynth.TYPE_NAMES[t], M)))
        del Ws, ys, ones
    say("  worst |dy|/bound", worst)


# Batch-M launches with several row steps per wave: Q5_K and Q3_K at M = 3
# (two-deep register ring across row steps), Q6_K at M = 4 with two K chunks
# (running row sums in LDS across chunks and steps), each with a ragged row
# count.
MULTISTEP = [(kqsynth.Q5_K, 28672 - 3, 8192, 3), (kqsynth.Q3_K, 8192 + 5, 28672, 3),
             (kqsynth.Q3_K, 20001, 8192, 3), (kqsynth.Q5_K, 9001, 28672, 3),
             (kqsynth.Q6_K, 12289, 28672, 4)]


@pytest.mark.parametrize("qtype,N,K,M", MULTISTEP,
                         ids=["%s-%dx%d-M%d" % (kqsynth.TYPE_NAMES[t], n, k, m) for (t, n, k, m) in MULTISTEP])
def test_batch_m_several_steps_per_wave(qtype, N, K, M):
    say("batch-M multistep", kqsynth.TYPE_NAMES[qtype], N, K, "M", M)
    W = kqsynth.device_matrix(qtype, N, K, seed=N + K + M, device="cuda")
    x = kqsynth.activations(M, K, kqsynth.rng_for(91, N, K, M))
    y = torch.empty((M, N), device="cuda")
    kq.kq_qgemv(qtype, W, N, K, torch.from_numpy(x).cuda(), M, y)
    ones = []
    for m in range(M):
        o = torch.empty((1, N), device="cuda")
        kq.kq_qgemv(qtype, W, N, K, torch.from_numpy(np.ascontiguousarray(x[m:m + 1])).cuda(), 1, o)
        ones.append(o)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    for m in range(M):
        assert np.array_equal(got[m].view(np.uint32), ones[m].cpu().numpy()[0].view(np.uint32)), m
    rows = sample_rows(N, N * 7 + K)
    Wr = W[torch.from_numpy(rows).cuda()].cpu().numpy()
    yo, S = oracle.gemv(qtype, Wr, len(rows), K, x)
    say("  worst |dy|/bound", check_close(got[:, rows], yo, S, "%s %dx%d M=%d" % (
        kqsynth.TYPE_NAMES[qtype], N, K, M)))


# Two formats side by side in one persistent launch with rows of fewer than 64
# units (K = 2048: 32 units, two rows per wave step), above the size the
# non-persistent grouped kernel takes.
@pytest.mark.parametrize("mats", [[(kqsynth.Q4_K, 24000), (kqsynth.Q6_K, 3000)],
                                  [(kqsynth.Q2_K, 30001), (kqsynth.Q5_K, 4000), (kqsynth.Q2_K, 77)]],
                         ids=["q4k+q6k", "q2k+q5k"])
def test_mixed_short_rows_persistent(mats):
    K = 2048
    assert sum(n * kqsynth.row_bytes(t, K) for t, n in mats) > 20 << 20
    say("mixed short rows", mats)
    Ws = [kqsynth.device_matrix(t, n, K, seed=95 + i, device="cuda") for i, (t, n) in enumerate(mats)]
    x = kqsynth.activations(1, K, kqsynth.rng_for(95))
    xd = torch.from_numpy(x).cuda()
    ys = [torch.full((1, n), float("nan"), device="cuda") for _, n in mats]
    kq.kq_qgemv_multi([t for t, _ in mats], Ws, [n for _, n in mats], K, xd, 1, ys)
    sep = []
    for i, (t, n) in enumerate(mats):
        o = torch.empty((1, n), device="cuda")
        kq.kq_qgemv(t, Ws[i], n, K, xd, 1, o)
        sep.append(o)
    torch.cuda.synchronize()
    for i, (t, n) in enumerate(mats):
        got = ys[i].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), sep[i].cpu().numpy().view(np.uint32)), i
        rows = sample_rows(n, n + i)
        Wr = Ws[i][torch.from_numpy(rows).cuda()].cpu().numpy()
        yo, S = oracle.gemv(t, Wr, len(rows), K, x)
        check_close(got[:, rows], yo, S, "matrix %d" % i)


# Batch-1 Q6_K launches of long rows (K >= 20480, the 16-wave configuration
# with one row step in flight per wave): a wave making more than 64 row steps
# (parked sums flushed mid-run), one step, a ragged row count, and two
# matrices in one launch; every row bit for bit against row 0 of an M = 2 call
# (the batch-M kernel) and sampled rows against the oracle.
Q6K_LONG = [(33000, 20480), (100, 20480), (1025, 28672)]


@pytest.mark.parametrize("N,K", Q6K_LONG, ids=["%dx%d" % c for c in Q6K_LONG])
def test_q6k_long_rows(N, K):
    qtype = kqsynth.Q6_K
    say("q6_k long rows", N, K)
    W = kqsynth.device_matrix(qtype, N, K, seed=N + 3 * K, device="cuda")
    x = kqsynth.activations(2, K, kqsynth.rng_for(96, N, K))
    y1 = torch.full((1, N), float("nan"), device="cuda")
    y2 = torch.full((2, N), float("nan"), device="cuda")
    kq.kq_qgemv(qtype, W, N, K, torch.from_numpy(np.ascontiguousarray(x[:1])).cuda(), 1, y1)
    kq.kq_qgemv(qtype, W, N, K, torch.from_numpy(x).cuda(), 2, y2)
    torch.cuda.synchronize()
    got = y1.cpu().numpy()
    assert np.array_equal(got[0].view(np.uint32), y2.cpu().numpy()[0].view(np.uint32))
    rows = sample_rows(N, N + K)
    Wr = W[torch.from_numpy(rows).cuda()].cpu().numpy()
    yo, S = oracle.gemv(qtype, Wr, len(rows), K, x[:1])
    say("  worst |dy|/bound", check_close(got[:, rows], yo, S, "Q6_K %dx%d" % (N, K)))


def test_q6k_long_rows_grouped():
    qtype, K, ns = kqsynth.Q6_K, 28672, [300, 700]
    say("q6_k long rows, two matrices", ns, K)
    Ws = [kqsynth.device_matrix(qtype, n, K, seed=97 + i, device="cuda") for i, n in enumerate(ns)]
    x = kqsynth.activations(1, K, kqsynth.rng_for(97))
    xd = torch.from_numpy(x).cuda()
    ys = [torch.full((1, n), float("nan"), device="cuda") for n in ns]
    kq.kq_qgemv_multi([qtype] * len(ns), Ws, ns, K, xd, 1, ys)
    sep = []
    for i, n in enumerate(ns):
        o = torch.empty((1, n), device="cuda")
        kq.kq_qgemv(qtype, Ws[i], n, K, xd, 1, o)
        sep.append(o)
    torch.cuda.synchronize()
    for i, n in enumerate(ns):
        got = ys[i].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), sep[i].cpu().numpy().view(np.uint32)), i
        rows = sample_rows(n, n + i)
        Wr = Ws[i][torch.from_numpy(rows).cuda()].cpu().numpy()
        yo, S = oracle.gemv(qtype, Wr, len(rows), K, x)
        check_close(got[:, rows], yo, S, "matrix %d" % i)


# Batch-1 Q4_K launches on the LDS ring with many row steps per wave: more
# than 64 (parked sums flushed mid-run), ragged row counts, the w1+w3 row
# count as one matrix, rows of one stripe, and two matrices in one launch;
# every row bit for bit against row 0 of an M = 2 call (another kernel) and
# sampled rows against the oracle, twice in a row.
Q4K_LONG = [(140001, 8192), (29000, 8192), (57344, 8192), (20001, 4096)]


@pytest.mark.parametrize("N,K", Q4K_LONG, ids=["%dx%d" % c for c in Q4K_LONG])
def test_q4k_long_launches(N, K):
    qtype = kqsynth.Q4_K
    say("q4_k long launch", N, K)
    W = kqsynth.device_matrix(qtype, N, K, seed=N + 5 * K, device="cuda")
    x = kqsynth.activations(2, K, kqsynth.rng_for(98, N, K))
    y2 = torch.full((2, N), float("nan"), device="cuda")
    kq.kq_qgemv(qtype, W, N, K, torch.from_numpy(x).cuda(), 2, y2)
    for rep in range(2):
        y1 = torch.full((1, N), float("nan"), device="cuda")
        kq.kq_qgemv(qtype, W, N, K, torch.from_numpy(np.ascontiguousarray(x[:1])).cuda(), 1, y1)
        torch.cuda.synchronize()
        got = y1.cpu().numpy()
        assert np.array_equal(got[0].view(np.uint32), y2.cpu().numpy()[0].view(np.uint32)), rep
    rows = sample_rows(N, N + K)
    Wr = W[torch.from_numpy(rows).cuda()].cpu().numpy()
    yo, S = oracle.gemv(qtype, Wr, len(rows), K, x[:1])
    say("  worst |dy|/bound", check_close(got[:, rows], yo, S, "Q4_K %dx%d" % (N, K)))


def test_q4k_long_launch_grouped():
    qtype, K, ns = kqsynth.Q4_K, 8192, [28672, 28672 - 77]
    say("q4_k long launch, two matrices", ns, K)
    Ws = [kqsynth.device_matrix(qtype, n, K, seed=99 + i, device="cuda") for i, n in enumerate(ns)]
    x = kqsynth.activations(1, K, kqsynth.rng_for(99))
    xd = torch.from_numpy(x).cuda()
    for rep in range(2):
        ys = [torch.full((1, n), float("nan"), device="cuda") for n in ns]
        kq.kq_qgemv_multi([qtype] * len(ns), Ws, ns, K, xd, 1, ys)
        torch.cuda.synchronize()
        if rep == 0:
            first = [y.cpu().numpy() for y in ys]
        else:
            for a, y in zip(first, ys):
                assert np.array_equal(a.view(np.uint32), y.cpu().numpy().view(np.uint32))
    for i, n in enumerate(ns):
        rows = sample_rows(n, n + i)
        Wr = Ws[i][torch.from_numpy(rows).cuda()].cpu().numpy()
        yo, S = oracle.gemv(qtype, Wr, len(rows), K, x)
        check_close(first[i][:, rows], yo, S, "matrix %d" % i)
