"""GPU parity over a seeded sweep of shapes.  The launcher chooses among its
kernels by format, row length, row count, M and grouping; the cases here are
drawn at random (fixed seed) across those choices: every format, K from one
block to 32768 columns, N from 1 to ~40000 rows, M from 1 to 8, single and
grouped launches (one format, or several K-quant formats sharing K).  Each
output is checked on sampled rows against the CPU oracle
(|dy| <= 1e-4 * sum|w*x| + 1e-6), each row of an M > 1 call bit for bit
against the M = 1 call on its activation row, and each matrix of a grouped
launch bit for bit against its own call.  Routed-expert calls (every format,
E up to 64, T up to 8, k up to 16, shared or per-slot activations, per-slot
outputs or their routing-weighted sum) are checked in full against the
oracle, and per-slot outputs bit for bit against the plain GEMV of the
slot's expert.  Standalone dequantization of 1 to 300000 blocks of every
format is checked bit for bit on every block or on sampled ones."""
import math
import sys

import numpy as np
import pytest

import kqsynth
import oracle

torch = pytest.importorskip("torch")
import dequant_gemv_gguf_amd as kq  # noqa: E402

pytestmark = pytest.mark.gpu

TYPES = [kqsynth.Q4_K, kqsynth.Q6_K, kqsynth.Q2_K, kqsynth.Q8_0, kqsynth.Q4_0, kqsynth.Q5_K, kqsynth.Q3_K]
KQUANTS = [kqsynth.Q2_K, kqsynth.Q3_K, kqsynth.Q4_K, kqsynth.Q5_K, kqsynth.Q6_K]
TOL_REL, TOL_ABS = 1e-4, 1e-6
MAX_WEIGHTS = 1 << 28


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def log_uniform(rng, lo, hi):
    return int(round(math.exp(rng.uniform(math.log(lo), math.log(hi)))))


def draw_k(rng, qtype):
    qk = kqsynth.BLOCK[qtype][0]
    return qk * log_uniform(rng, 1, 32768 // qk)


def draw_n(rng, K, hi=40000):
    return max(1, min(log_uniform(rng, 1, hi), MAX_WEIGHTS // K))


def single_cases(seed=2026, count=96):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        qtype = TYPES[i % len(TYPES)]
        K = draw_k(rng, qtype)
        out.append((qtype, draw_n(rng, K), K, int(rng.integers(1, 9)), 1000 + i))
    return out


def grouped_cases(seed=2027, count=32):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        mixed = i % 2 == 1
        K = draw_k(rng, kqsynth.Q4_K)
        n = int(rng.integers(2, 6))
        types = [int(rng.choice(KQUANTS)) for _ in range(n)] if mixed else [TYPES[i % len(TYPES)]] * n
        if not mixed:
            K = draw_k(rng, types[0])
        Ns = [0 if rng.random() < 0.1 else draw_n(rng, K, 30000 // n) for _ in range(n)]
        M = 1 if mixed and i % 4 == 1 else int(rng.integers(1, 9))
        out.append((types, Ns, K, M, 2000 + i))
    return out


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def sampled_rows(N, seed, n=24):
    r = np.random.default_rng(seed).integers(0, N, n)
    return np.unique(np.concatenate([[0, N - 1], r]))


def check_rows(qtype, W, N, K, x, y, seed, what):
    rows = sampled_rows(N, seed)
    Wr = W[torch.from_numpy(rows).cuda()].cpu().numpy()
    yo, S = oracle.gemv(qtype, Wr, len(rows), K, x)
    err = np.abs(y[:, rows].astype(np.float64) - yo)
    bound = TOL_REL * S + TOL_ABS
    assert np.all(err <= bound), "%s: worst |dy|/bound = %.3g" % (what, float((err / bound).max()))


def gemv(qtype, W, N, K, x):
    y = torch.full((x.shape[0], N), float("nan"), device="cuda")
    kq.kq_qgemv(qtype, W, N, K, dev(x), x.shape[0], y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("case", single_cases(),
                         ids=lambda c: "%s-N%d-K%d-M%d" % (kqsynth.TYPE_NAMES[c[0]], c[1], c[2], c[3]))
def test_sweep_single(case):
    qtype, N, K, M, seed = case
    say("sweep", kqsynth.TYPE_NAMES[qtype], "N", N, "K", K, "M", M)
    W = kqsynth.device_matrix(qtype, N, K, seed=seed, device="cuda")
    x = kqsynth.activations(M, K, kqsynth.rng_for(seed, M, K))
    y = gemv(qtype, W, N, K, x)
    check_rows(qtype, W, N, K, x, y, seed, "N=%d K=%d M=%d" % (N, K, M))
    if M > 1:
        for m in sorted({0, M // 2, M - 1}):
            one = gemv(qtype, W, N, K, x[m:m + 1])
            assert np.array_equal(one[0].view(np.uint32), y[m].view(np.uint32)), "row %d of M=%d" % (m, M)
    del W


@pytest.mark.parametrize("case", grouped_cases(),
                         ids=lambda c: "K%d-M%d-" % (c[2], c[3]) + "+".join(
                             "%s%d" % (kqsynth.TYPE_NAMES[t], n) for t, n in zip(c[0], c[1])))
def test_sweep_grouped(case):
    types, Ns, K, M, seed = case
    say("sweep grouped", [kqsynth.TYPE_NAMES[t] for t in types], Ns, "K", K, "M", M)
    Ws = [kqsynth.device_matrix(t, max(n, 1), K, seed=seed + i, device="cuda") for i, (t, n) in enumerate(zip(types, Ns))]
    x = kqsynth.activations(M, K, kqsynth.rng_for(seed, M, K))
    ys = [torch.full((M, n), float("nan"), device="cuda") if n else None for n in Ns]
    kq.kq_qgemv_multi(types, [W if n else None for W, n in zip(Ws, Ns)], Ns, K, dev(x), M, ys)
    torch.cuda.synchronize()
    for i, (t, n) in enumerate(zip(types, Ns)):
        if n == 0:
            continue
        got = ys[i].cpu().numpy()
        one = gemv(t, Ws[i], n, K, x)
        assert np.array_equal(got.view(np.uint32), one.view(np.uint32)), "matrix %d" % i
        check_rows(t, Ws[i], n, K, x, got, seed + i, "matrix %d" % i)
    del Ws


# ---- routed experts ------------------------------------------------------------

def moe_cases(seed=2028, count=32):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        qtype = TYPES[i % len(TYPES)]
        qk = kqsynth.BLOCK[qtype][0]
        K = qk * log_uniform(rng, 1, 8192 // qk)
        E = log_uniform(rng, 1, 64)
        k = int(rng.integers(1, min(E, 16) + 1))
        T = int(rng.integers(1, 9))
        # the oracle computes every output: at most ~5e7 multiply-adds a case
        N = max(1, min(log_uniform(rng, 1, 3000), int(5e7) // (T * k * K)))
        out.append((qtype, E, N, K, T, k, i % 2, (i // 2) % 2 == 1, 3000 + i))
    return out


@pytest.mark.parametrize("case", moe_cases(),
                         ids=lambda c: "%s-E%d-N%d-K%d-T%d-k%d-x%d-%s" % (
                             kqsynth.TYPE_NAMES[c[0]], c[1], c[2], c[3], c[4], c[5], c[6], "sum" if c[7] else "slots"))
def test_sweep_moe(case):
    qtype, E, N, K, T, k, x_mode, combine, seed = case
    say("sweep moe", kqsynth.TYPE_NAMES[qtype], "E", E, "N", N, "K", K, "T", T, "k", k, "x_mode", x_mode, combine)
    W = kqsynth.blocks(qtype, E * N * (K // kqsynth.BLOCK[qtype][0]), kqsynth.rng_for(seed, 1))
    ids, p = kqsynth.routing(T, k, E, kqsynth.rng_for(seed, 2))
    x = kqsynth.activations(T * (k if x_mode else 1), K, kqsynth.rng_for(seed, 3))
    pw = p if combine else None
    Wd = dev(W.reshape(-1))
    y = torch.full((T, N) if combine else (T, k, N), float("nan"), device="cuda")
    ws = torch.empty(kq.kq_qmoe_workspace_bytes(T, k, N) // 4 + 1, device="cuda") if combine else None
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    kq.kq_qmoe_gemv(qtype, Wd, E, N, K, dev(ids), None if pw is None else dev(pw), T, k, dev(x), x_mode, y, ws, flag)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    yo, S, oflag = oracle.moe(qtype, W, E, N, K, ids, pw, x, x_mode)
    assert int(flag.item()) == 0 and oflag == 0
    err = np.abs(got.astype(np.float64) - yo)
    bound = TOL_REL * S + TOL_ABS
    assert np.all(err <= bound), "worst |dy|/bound = %.3g" % float((err / bound).max())
    if not combine:
        # a slot's outputs are the bits of the plain GEMV of its expert on its activation row
        per = N * kqsynth.row_bytes(qtype, K)
        for t, j in sorted({(0, 0), (T - 1, k - 1), (T // 2, k // 2)}):
            e = int(ids[t, j])
            xr = x[t * k + j if x_mode else t][None, :]
            one = gemv(qtype, Wd[e * per:(e + 1) * per].clone(), N, K, xr)   # a 16-byte aligned copy
            assert np.array_equal(one[0].view(np.uint32), got[t, j].view(np.uint32)), (t, j)


# ---- standalone dequantization --------------------------------------------------

def dequant_cases(seed=2029, count=21):
    rng = np.random.default_rng(seed)
    return [(TYPES[i % len(TYPES)], log_uniform(rng, 1, 300000), 4000 + i) for i in range(count)]


@pytest.mark.parametrize("case", dequant_cases(), ids=lambda c: "%s-%d" % (kqsynth.TYPE_NAMES[c[0]], c[1]))
def test_sweep_dequant(case):
    qtype, nblocks, seed = case
    say("sweep dequant", kqsynth.TYPE_NAMES[qtype], nblocks)
    qk = kqsynth.BLOCK[qtype][0]
    W = kqsynth.device_matrix(qtype, nblocks, qk, seed=seed, device="cuda")   # nblocks rows of one block
    n = nblocks * qk
    out = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    kq.kq_dequant(qtype, W, n, out)
    torch.cuda.synchronize()
    # every block of a short run, sampled blocks (first and last included) of a long one
    picks = np.arange(nblocks) if nblocks <= 4096 else sampled_rows(nblocks, seed, 2000)
    blk = W[torch.from_numpy(picks).cuda()].cpu().numpy()
    ref = oracle.dequant(qtype, blk, len(picks) * qk).reshape(len(picks), qk)
    got = out.view(nblocks, qk)[torch.from_numpy(picks).cuda()].cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
