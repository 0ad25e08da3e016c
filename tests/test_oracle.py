"""Pins for the CPU oracle, against things other than the oracle itself:
numpy's fp16 decoder (every bit pattern), exact rational closed forms of the
block formulas from independently encoded fields, exactly representable
round trips, special cases, one-hot and all-ones activations, a numpy fp64
matmul cross-check and exact rational brute force on tiny GEMVs."""
from fractions import Fraction

import numpy as np
import pytest

import kq_fields as F
import kqsynth
import oracle

TYPES = [F.Q4_K, F.Q6_K, F.Q2_K, F.Q8_0, F.Q4_0, F.Q5_K, F.Q3_K]


def deq(qtype, raw, n):
    return oracle.dequant(qtype, np.frombuffer(raw, dtype=np.uint8), n)


# ---- the encoder itself -------------------------------------------------------

@pytest.mark.parametrize("qtype", TYPES)
def test_encoder_places_every_bit_once(qtype):
    # Bits.put asserts no bit is written twice and encode asserts every bit of
    # the block is covered: the field packing is a bijection of bit positions.
    rng = np.random.default_rng(1)
    for _ in range(5):
        F.encode(qtype, F.random_fields(qtype, rng))


@pytest.mark.parametrize("qtype", TYPES)
def test_encoder_max_fields_fill_block(qtype):
    full = {
        F.Q4_K: dict(d=0xFFFF, dmin=0xFFFF, sc=[63] * 8, m=[63] * 8, q=[15] * 256),
        F.Q6_K: dict(d=0xFFFF, sc=[-1] * 16, q=[63] * 256),
        F.Q2_K: dict(d=0xFFFF, dmin=0xFFFF, sc=[15] * 16, m=[15] * 16, q=[3] * 256),
        F.Q8_0: dict(d=0xFFFF, q=[-1] * 32),
        F.Q4_0: dict(d=0xFFFF, q=[15] * 32),
        F.Q5_K: dict(d=0xFFFF, dmin=0xFFFF, sc=[63] * 8, m=[63] * 8, q=[31] * 256),
        F.Q3_K: dict(d=0xFFFF, sc=[63] * 16, q=[3] * 256),
    }[qtype]
    assert F.encode(qtype, full) == b"\xff" * F.NBYTES[qtype]


# ---- fp16 decoding against numpy ---------------------------------------------

def test_fp16_decode_every_pattern_matches_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = np.isfinite(bits.view(np.float16))
    bits = bits[finite]
    nb = bits.size
    blk = np.zeros((nb, 34), dtype=np.uint8)
    blk[:, 0:2] = bits.view(np.uint8).reshape(nb, 2)
    blk[:, 2] = 1                      # q0 = +1  -> w = d
    blk[:, 3] = 0xFF                   # q1 = -1  -> w = -d
    w = oracle.dequant(F.Q8_0, blk, nb * 32).reshape(nb, 32)
    ref = bits.view(np.float16).astype(np.float32)
    assert np.array_equal(w[:, 0].view(np.uint32), (ref + np.float32(0)).view(np.uint32))
    assert np.array_equal(w[:, 1], -ref)
    assert np.all(w[:, 2:] == 0)


# ---- closed forms from independently encoded fields ---------------------------

@pytest.mark.parametrize("qtype", TYPES)
@pytest.mark.parametrize("subnormal", [False, True])
def test_dequant_matches_exact_closed_form(qtype, subnormal):
    rng = np.random.default_rng(100 + qtype + subnormal)
    for _ in range(20):
        f = F.random_fields(qtype, rng, subnormal_d=subnormal)
        got = deq(qtype, F.encode(qtype, f), F.QK[qtype])
        want = np.array([F.round_f32(v) for v in F.exact(qtype, f)], dtype=np.float32)
        assert np.array_equal(got.view(np.uint32), (want + np.float32(0)).view(np.uint32)), f


@pytest.mark.parametrize("qtype", TYPES)
def test_full_fp16_range_scales(qtype):
    # d and dmin anywhere in the finite fp16 range, including the largest.
    rng = np.random.default_rng(7 + qtype)
    for _ in range(20):
        f = F.random_fields(qtype, rng)
        for key in ("d", "dmin"):
            if key in f:
                while True:
                    b = int(rng.integers(0, 0x7C00))
                    if rng.random() < 0.5:
                        b |= 0x8000
                    f[key] = b
                    break
        got = deq(qtype, F.encode(qtype, f), F.QK[qtype])
        want = np.array([F.round_f32(v) for v in F.exact(qtype, f)], dtype=np.float32)
        assert np.array_equal(got.view(np.uint32), (want + np.float32(0)).view(np.uint32))


def test_rounding_is_to_nearest_even_not_truncation():
    # d*sc*q needs 21 bits and dmin*m 17: choose fields whose exact weight
    # lies between two fp32 values, so that RNE and truncation differ.
    f = dict(d=F.f16_bits(1.0009765625), dmin=0x0001, sc=[63] * 8, m=[1] * 8, q=[15] * 256)
    vals = F.exact_q4k(**f)
    got = deq(F.Q4_K, F.encode_q4k(**f), 256)
    for e in (0, 100, 255):
        exact = vals[e]
        assert Fraction(float(got[e])) != exact           # rounding happened
        lo = np.float32(float(exact))                      # reference RNE
        assert got[e] == lo
        assert abs(Fraction(float(got[e])) - exact) <= abs(Fraction(float(np.nextafter(got[e], np.float32(0)))) - exact)


# ---- special cases --------------------------------------------------------------

def test_q4k_special_cases():
    one, half = F.f16_bits(1.0), F.f16_bits(0.5)
    sc = [1, 2, 3, 4, 5, 6, 7, 63]
    m = [0, 1, 2, 3, 62, 63, 5, 9]
    q = [e % 16 for e in range(256)]
    w = deq(F.Q4_K, F.encode_q4k(one, half, sc, m, q), 256)
    for e in range(256):
        j = e // 32
        assert w[e] == sc[j] * q[e] - 0.5 * m[j]       # exactly representable
    # q = 0 -> -dmin*m ; sc = m = 0 -> +0
    w = deq(F.Q4_K, F.encode_q4k(one, half, [0] * 8, [0] * 8, [7] * 256), 256)
    assert np.all(w.view(np.uint32) == 0)
    w = deq(F.Q4_K, F.encode_q4k(one, half, sc, m, [0] * 256), 256)
    assert np.all(w == np.repeat(-0.5 * np.array(m, dtype=np.float32), 32))


def test_q6k_special_cases():
    d = F.f16_bits(0.25)
    sc = [-128, 127, -1, 1] * 4
    # q = 32 -> +0 for either sign of d*sc ; sc = -128, q = 0 -> d*4096
    w = deq(F.Q6_K, F.encode_q6k(d, sc, [32] * 256), 256)
    assert np.all(w.view(np.uint32) == 0)
    w = deq(F.Q6_K, F.encode_q6k(d, sc, [0] * 256), 256)
    assert w[0] == 0.25 * 4096 and w[16] == 0.25 * 127 * -32
    w = deq(F.Q6_K, F.encode_q6k(F.f16_bits(-0.25), sc, [63] * 256), 256)
    assert w[0] == -0.25 * -128 * 31


def test_q2k_special_cases():
    one, two = F.f16_bits(1.0), F.f16_bits(2.0)
    sc = list(range(16))
    m = list(range(15, -1, -1))
    q = [(e // 7) % 4 for e in range(256)]
    w = deq(F.Q2_K, F.encode_q2k(one, two, sc, m, q), 256)
    for e in range(256):
        assert w[e] == sc[e // 16] * q[e] - 2 * m[e // 16]


def test_q80_special_cases():
    d = F.f16_bits(0.001)
    q = [-127, 127, 0, 1] * 8
    w = deq(F.Q8_0, F.encode_q80(d, q), 32)
    dv = float(np.float16(0.001))
    assert w[0] == np.float32(-127 * dv) and w[1] == np.float32(127 * dv) and w[2] == 0


def test_q40_special_cases():
    one = F.f16_bits(1.0)
    q = [e % 16 for e in range(32)]
    w = deq(F.Q4_0, F.encode_q40(one, q), 32)
    assert list(w) == [float(v - 8) for v in q]
    w = deq(F.Q4_0, F.encode_q40(F.f16_bits(-0.5), [8] * 32), 32)
    assert np.all(w.view(np.uint32) == 0)                # q = 8 -> +0 for either sign of d


def test_q5k_special_cases():
    one, half = F.f16_bits(1.0), F.f16_bits(0.5)
    sc = [1, 2, 3, 4, 5, 6, 7, 63]
    m = [0, 1, 2, 3, 62, 63, 5, 9]
    q = [(e * 7) % 32 for e in range(256)]
    w = deq(F.Q5_K, F.encode_q5k(one, half, sc, m, q), 256)
    for e in range(256):
        assert w[e] == sc[e // 32] * q[e] - 0.5 * m[e // 32]
    w = deq(F.Q5_K, F.encode_q5k(one, half, [1] * 8, [0] * 8, [16] * 256), 256)
    assert np.all(w == 16)                               # the high bit alone


def test_q3k_special_cases():
    one = F.f16_bits(1.0)
    sc = list(range(0, 64, 4))
    q = [(e % 8) - 4 for e in range(256)]
    w = deq(F.Q3_K, F.encode_q3k(one, sc, q), 256)
    for e in range(256):
        assert w[e] == (sc[e // 16] - 32) * q[e]
    w = deq(F.Q3_K, F.encode_q3k(F.f16_bits(-2.0), [32] * 16, q), 256)
    assert np.all(w.view(np.uint32) == 0)                # sc = 32 -> +0
    w = deq(F.Q3_K, F.encode_q3k(one, [0] * 16, [-4] * 256), 256)
    assert np.all(w == 128)                              # (0 - 32) * (-4)


@pytest.mark.parametrize("qtype", TYPES)
def test_subnormal_scales_are_not_flushed(qtype):
    for p in range(0, 10):                       # d = 2^-24 .. 2^-15
        f = F.random_fields(qtype, np.random.default_rng(p))
        f["d"] = 1 << p
        if "dmin" in f:
            f["dmin"] = 1 << (9 - p)
        w = deq(qtype, F.encode(qtype, f), F.QK[qtype])
        want = np.array([F.round_f32(v) for v in F.exact(qtype, f)], dtype=np.float32)
        assert np.array_equal(w, want)
        assert np.any(w != 0)


# ---- GEMV pins ------------------------------------------------------------------

def _random_matrix(qtype, N, K, seed):
    return kqsynth.matrix(qtype, N, K, kqsynth.rng_for(seed, qtype, N, K))


@pytest.mark.parametrize("qtype", TYPES)
def test_gemv_one_hot_gives_columns_exactly(qtype):
    N, K = 6, 512
    W = _random_matrix(qtype, N, K, 3)
    dense = oracle.dequant(qtype, W, N * K).reshape(N, K)
    cols = [0, 1, 31, 32, 255, 256, 300, 511]
    x = np.zeros((len(cols), K), dtype=np.float32)
    for r, c in enumerate(cols):
        x[r, c] = 1.0
    y, S = oracle.gemv(qtype, W, N, K, x)
    for r, c in enumerate(cols):
        assert np.array_equal(y[r], dense[:, c].astype(np.float64))
        assert np.array_equal(S[r], np.abs(dense[:, c]).astype(np.float64))


def test_gemv_all_ones_closed_form_q4k():
    # x = 1: y = sum over sub-blocks j of (d*sc_j*sum_e q_e - 32*dmin*m_j),
    # with fields chosen so that every weight is exactly representable.
    rng = np.random.default_rng(11)
    rows, want = [], []
    for _ in range(3):
        blocks, total = [], Fraction(0)
        for _ in range(2):
            d, dmin = F.f16_bits(0.125), F.f16_bits(0.0625)
            sc = [int(v) for v in rng.integers(0, 64, 8)]
            m = [int(v) for v in rng.integers(0, 64, 8)]
            q = [int(v) for v in rng.integers(0, 16, 256)]
            blocks.append(F.encode_q4k(d, dmin, sc, m, q))
            for j in range(8):
                total += Fraction(1, 8) * sc[j] * sum(q[32 * j:32 * j + 32]) - 32 * Fraction(1, 16) * m[j]
        rows.append(b"".join(blocks))
        want.append(total)
    W = np.frombuffer(b"".join(rows), dtype=np.uint8)
    y, _ = oracle.gemv(F.Q4_K, W, 3, 512, np.ones((1, 512), dtype=np.float32))
    assert [Fraction(v) for v in y[0]] == want


@pytest.mark.parametrize("qtype", TYPES)
def test_gemv_matches_numpy_fp64_matmul(qtype):
    N, K, M = 37, 1024, 3
    W = _random_matrix(qtype, N, K, 5)
    x = kqsynth.activations(M, K, kqsynth.rng_for(5, 99))
    y, S = oracle.gemv(qtype, W, N, K, x)
    dense = oracle.dequant(qtype, W, N * K).reshape(N, K).astype(np.float64)
    ref = x.astype(np.float64) @ dense.T
    mag = np.abs(x.astype(np.float64)) @ np.abs(dense).T
    assert np.all(np.abs(y - ref) <= 1e-12 * mag)
    assert np.allclose(S, mag, rtol=1e-12, atol=0)


@pytest.mark.parametrize("qtype", TYPES)
def test_gemv_brute_force_exact_rational(qtype):
    rng = np.random.default_rng(21 + qtype)
    for (N, K, M) in [(2, 256, 1), (4, 512, 3), (3, 256, 8)]:
        qk = F.QK[qtype]
        fields = [[F.random_fields(qtype, rng) for _ in range(K // qk)] for _ in range(N)]
        W = np.frombuffer(b"".join(F.encode(qtype, f) for row in fields for f in row), dtype=np.uint8)
        x = rng.standard_normal((M, K)).astype(np.float32)
        y, S = oracle.gemv(qtype, W, N, K, x)
        for o in range(N):
            w = [F.round_f32(v) for f in fields[o] for v in F.exact(qtype, f)]
            for m in range(M):
                exact = sum(Fraction(float(w[i])) * Fraction(float(x[m, i])) for i in range(K))
                mag = sum(abs(Fraction(float(w[i])) * Fraction(float(x[m, i]))) for i in range(K))
                assert abs(Fraction(y[m, o]) - exact) <= K * Fraction(2) ** -52 * mag
                assert abs(Fraction(S[m, o]) - mag) <= K * Fraction(2) ** -52 * mag


def test_gemv_rejects_bad_shapes():
    W = np.zeros(144, dtype=np.uint8)
    with pytest.raises(ValueError):
        oracle.gemv(F.Q4_K, W, 1, 100, np.zeros((1, 100), np.float32))
    with pytest.raises(ValueError):
        oracle.dequant(99, W, 256)


# ---- MoE pins ---------------------------------------------------------------------

def _moe_inputs(qtype, E, N, K, T, k, seed):
    W = np.concatenate([_random_matrix(qtype, N, K, seed * 1000 + e).reshape(-1) for e in range(E)])
    ids, p = kqsynth.routing(T, k, E, kqsynth.rng_for(seed, 1))
    return W, ids, p


def test_moe_single_slot_equals_gemv_on_that_expert():
    E, N, K = 5, 16, 512
    W, _, _ = _moe_inputs(F.Q4_K, E, N, K, 1, 1, 1)
    per_expert = W.size // E
    x = kqsynth.activations(1, K, kqsynth.rng_for(1, 2))
    for e in range(E):
        y, S, flag = oracle.moe(F.Q4_K, W, E, N, K, np.array([[e]]), np.ones((1, 1), np.float32), x, 0)
        yg, Sg = oracle.gemv(F.Q4_K, W[e * per_expert:(e + 1) * per_expert], N, K, x)
        assert flag == 0 and np.array_equal(y, yg) and np.array_equal(S, Sg)


@pytest.mark.parametrize("x_mode", [0, 1])
def test_moe_per_slot_and_combined(x_mode):
    E, N, K, T, k = 8, 12, 256, 3, 4
    W, ids, p = _moe_inputs(F.Q6_K, E, N, K, T, k, 2)
    per_expert = W.size // E
    x = kqsynth.activations(T * (k if x_mode else 1), K, kqsynth.rng_for(2, 3))
    y, S, flag = oracle.moe(F.Q6_K, W, E, N, K, ids, None, x, x_mode)
    assert flag == 0 and y.shape == (T, k, N)
    for t in range(T):
        for j in range(k):
            xs = x[t * k + j] if x_mode else x[t]
            yg, Sg = oracle.gemv(F.Q6_K, W[ids[t, j] * per_expert:(ids[t, j] + 1) * per_expert], N, K, xs)
            assert np.array_equal(y[t, j], yg[0]) and np.array_equal(S[t, j], Sg[0])
    yc, Sc, _ = oracle.moe(F.Q6_K, W, E, N, K, ids, p, x, x_mode)
    ref = np.zeros((T, N))
    for j in range(k):                       # ascending slot order, fp64
        ref += p[:, j:j + 1].astype(np.float64) * y[:, j, :]
    assert np.array_equal(yc, ref)
    assert np.allclose(Sc, np.einsum("tj,tjn->tn", np.abs(p.astype(np.float64)), S), rtol=1e-15)


def test_moe_slot_permutation_changes_combine_only_by_rounding():
    E, N, K, T, k = 16, 8, 512, 2, 8
    W, ids, p = _moe_inputs(F.Q2_K, E, N, K, T, k, 4)
    x = kqsynth.activations(T, K, kqsynth.rng_for(4, 5))
    y1, S1, _ = oracle.moe(F.Q2_K, W, E, N, K, ids, p, x, 0)
    perm = np.random.default_rng(0).permutation(k)
    y2, S2, _ = oracle.moe(F.Q2_K, W, E, N, K, ids[:, perm], p[:, perm], x, 0)
    assert np.allclose(y1, y2, rtol=0, atol=1e-13 * S1.max())


def test_moe_all_ids_equal_is_dense_gemv_and_bad_ids_flag():
    E, N, K, T, k = 4, 8, 256, 2, 3
    W, _, _ = _moe_inputs(F.Q8_0, E, N, K, T, k, 6)
    per_expert = W.size // E
    x = kqsynth.activations(T, K, kqsynth.rng_for(6, 7))
    ids = np.full((T, k), 2, dtype=np.int32)
    y, _, flag = oracle.moe(F.Q8_0, W, E, N, K, ids, None, x, 0)
    yg, _ = oracle.gemv(F.Q8_0, W[2 * per_expert:3 * per_expert], N, K, x)
    assert flag == 0
    for j in range(k):
        assert np.array_equal(y[:, j, :], yg)
    ids[1, 1] = E            # out of range -> zero contribution and flag
    ids[0, 2] = -1
    y, _, flag = oracle.moe(F.Q8_0, W, E, N, K, ids, None, x, 0)
    assert flag == 1 and np.all(y[1, 1] == 0) and np.all(y[0, 2] == 0)
    assert np.array_equal(y[1, 0], yg[1])


# ---- the synthetic generator's recipe -------------------------------------------

def test_synth_recipe_properties():
    rng = kqsynth.rng_for(0, 1)
    b = kqsynth.blocks(kqsynth.Q8_0, 4000, rng)
    q = b[:, 2:].view(np.int8)
    assert q.min() == -127 and q.max() == 127
    d = b[:, 0:2].copy().view(np.float16).astype(np.float64)
    assert np.all(d >= 0) and 0.7e-3 < d.mean() < 0.9e-3
    a = kqsynth.blocks(kqsynth.Q4_K, 8, kqsynth.rng_for(0, 1, 2))
    c = kqsynth.blocks(kqsynth.Q4_K, 8, kqsynth.rng_for(0, 1, 2))
    assert np.array_equal(a, c)
    ids, p = kqsynth.routing(8, 8, 128, kqsynth.rng_for(0, 3))
    assert all(len(set(r)) == 8 for r in ids.tolist())
    assert np.allclose(p.sum(axis=1), 1, atol=1e-6)
