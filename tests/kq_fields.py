"""Test-side field encoder and exact closed forms for the block formats.

Written independently of the oracle's decoder, from the GGUF K-quant layout
(a reading; the pages name Q2_K..Q6_K and Q8_0 but print no layout): every
field is placed bit by bit, and the expected weights are computed with exact
rational arithmetic from the fields.  Agreement between this encoder and the
oracle's decoder pins the oracle's element index maps; the bit-placement
bijection tests pin the encoder itself.
"""
from fractions import Fraction

import numpy as np

Q4_0, Q8_0, Q2_K, Q3_K, Q4_K, Q5_K, Q6_K = 2, 8, 10, 11, 12, 13, 14
QK = {Q4_0: 32, Q8_0: 32, Q2_K: 256, Q3_K: 256, Q4_K: 256, Q5_K: 256, Q6_K: 256}
NBYTES = {Q4_0: 18, Q8_0: 34, Q2_K: 84, Q3_K: 110, Q4_K: 144, Q5_K: 176, Q6_K: 210}


class Bits:
    """A little-endian bit buffer with write-once checking."""

    def __init__(self, nbytes):
        self.buf = bytearray(nbytes)
        self.used = [False] * (nbytes * 8)

    def put(self, bitpos, width, value):
        assert 0 <= value < (1 << width), (value, width)
        for i in range(width):
            p = bitpos + i
            assert not self.used[p], "bit %d written twice" % p
            self.used[p] = True
            if (value >> i) & 1:
                self.buf[p // 8] |= 1 << (p % 8)

    def put_u16(self, byte, v):
        self.put(8 * byte, 16, int(v))

    def full(self):
        return all(self.used)


def f16_bits(x):
    return int(np.array([x], dtype=np.float16).view(np.uint16)[0])


def f16_exact(bits):
    """Exact rational value of a finite fp16 bit pattern."""
    sign = -1 if bits >> 15 else 1
    e = (bits >> 10) & 31
    m = bits & 1023
    assert e != 31
    if e == 0:
        return sign * Fraction(m, 1 << 24)
    return sign * Fraction(1024 + m, 1 << 10) * (Fraction(2) ** (e - 15))


def encode_q4k(d, dmin, sc, m, q):
    """d, dmin: fp16 bit patterns; sc, m: 8 values 0..63; q: 256 values 0..15."""
    b = Bits(144)
    b.put_u16(0, d)
    b.put_u16(2, dmin)
    for j in range(4):
        b.put(8 * (4 + j), 6, sc[j])            # scale j, low 6 bits of byte j
        b.put(8 * (4 + j) + 6, 2, sc[j + 4] >> 4)  # top 2 bits of scale j+4
        b.put(8 * (8 + j), 6, m[j])             # min j, low 6 bits of byte 4+j
        b.put(8 * (8 + j) + 6, 2, m[j + 4] >> 4)   # top 2 bits of min j+4
        b.put(8 * (12 + j), 4, sc[j + 4] & 15)  # low 4 bits of scale j+4
        b.put(8 * (12 + j) + 4, 4, m[j + 4] & 15)  # low 4 bits of min j+4
    for e in range(256):
        chunk, sub, within = e // 64, (e // 32) % 2, e % 32
        byte = 16 + 32 * chunk + within
        b.put(8 * byte + 4 * sub, 4, q[e])
    assert b.full()
    return bytes(b.buf)


def encode_q6k(d, sc, q):
    """d: fp16 bits; sc: 16 int8 values; q: 256 values 0..63."""
    b = Bits(210)
    for e in range(256):
        half, grp, lane = e // 128, (e % 128) // 32, e % 32
        lo_byte = 64 * half + 32 * (grp % 2) + lane
        b.put(8 * lo_byte + (0 if grp < 2 else 4), 4, q[e] & 15)
        b.put(8 * (128 + 32 * half + lane) + 2 * grp, 2, q[e] >> 4)
    for i in range(16):
        b.put(8 * (192 + i), 8, sc[i] & 0xFF)
    b.put_u16(208, d)
    assert b.full()
    return bytes(b.buf)


def encode_q2k(d, dmin, sc, m, q):
    """d, dmin: fp16 bits; sc, m: 16 values 0..15; q: 256 values 0..3."""
    b = Bits(84)
    for i in range(16):
        b.put(8 * i, 4, sc[i])
        b.put(8 * i + 4, 4, m[i])
    for e in range(256):
        half, shift, t = e // 128, (e % 128) // 32, e % 32
        b.put(8 * (16 + 32 * half + t) + 2 * shift, 2, q[e])
    b.put_u16(80, d)
    b.put_u16(82, dmin)
    assert b.full()
    return bytes(b.buf)


def encode_q80(d, q):
    """d: fp16 bits; q: 32 int8 values."""
    b = Bits(34)
    b.put_u16(0, d)
    for e in range(32):
        b.put(8 * (2 + e), 8, q[e] & 0xFF)
    assert b.full()
    return bytes(b.buf)


def encode_q40(d, q):
    """d: fp16 bits; q: 32 values 0..15 (weight e = d*(q_e - 8)); weights 0..15
    in the low nibbles of the 16 quant bytes, 16..31 in the high nibbles."""
    b = Bits(18)
    b.put_u16(0, d)
    for e in range(32):
        b.put(8 * (2 + e % 16) + (4 if e >= 16 else 0), 4, q[e])
    assert b.full()
    return bytes(b.buf)


def _put_k4_scales(b, at, sc, m):
    """The 6-bit scale / min packing shared by Q4_K and Q5_K, at byte `at`."""
    for j in range(4):
        b.put(8 * (at + j), 6, sc[j])
        b.put(8 * (at + j) + 6, 2, sc[j + 4] >> 4)
        b.put(8 * (at + 4 + j), 6, m[j])
        b.put(8 * (at + 4 + j) + 6, 2, m[j + 4] >> 4)
        b.put(8 * (at + 8 + j), 4, sc[j + 4] & 15)
        b.put(8 * (at + 8 + j) + 4, 4, m[j + 4] & 15)


def encode_q5k(d, dmin, sc, m, q):
    """d, dmin: fp16 bits; sc, m: 8 values 0..63; q: 256 values 0..31.  Low
    4 bits of q as in Q4_K (bytes 48..175), bit 4 of q_e is bit e//32 of
    byte 16 + e%32."""
    b = Bits(176)
    b.put_u16(0, d)
    b.put_u16(2, dmin)
    _put_k4_scales(b, 4, sc, m)
    for e in range(256):
        chunk, sub, within = e // 64, (e // 32) % 2, e % 32
        b.put(8 * (48 + 32 * chunk + within) + 4 * sub, 4, q[e] & 15)
        b.put(8 * (16 + within) + e // 32, 1, q[e] >> 4)
    assert b.full()
    return bytes(b.buf)


def encode_q3k(d, sc, q):
    """d: fp16 bits; sc: 16 stored 6-bit scales 0..63 (used as sc - 32);
    q: 256 values -4..3.  q + 4 = q2 + 4*hbit: q2 in bits 2j..2j+1 of byte
    32 + 32h + l, hbit in bit e//32 of byte l (h = e//128, j = (e%128)//32,
    l = e%32).  Scale i: low 4 bits in byte 96 + i%8 (low nibble for i < 8,
    high nibble otherwise), top 2 bits in bits 2*(i//4)..+1 of byte 104 + i%4."""
    b = Bits(110)
    for e in range(256):
        h, j, l = e // 128, (e % 128) // 32, e % 32
        u = q[e] + 4
        b.put(8 * (32 + 32 * h + l) + 2 * j, 2, u & 3)
        b.put(8 * l + e // 32, 1, u >> 2)
    for i in range(16):
        b.put(8 * (96 + i % 8) + (4 if i >= 8 else 0), 4, sc[i] & 15)
        b.put(8 * (104 + i % 4) + 2 * (i // 4), 2, sc[i] >> 4)
    b.put_u16(108, d)
    assert b.full()
    return bytes(b.buf)


# ---- exact weights from fields ---------------------------------------------

def exact_q4k(d, dmin, sc, m, q):
    D, Dm = f16_exact(d), f16_exact(dmin)
    return [D * sc[e // 32] * q[e] - Dm * m[e // 32] for e in range(256)]


def exact_q6k(d, sc, q):
    D = f16_exact(d)
    return [D * sc[e // 16] * (q[e] - 32) for e in range(256)]


def exact_q2k(d, dmin, sc, m, q):
    D, Dm = f16_exact(d), f16_exact(dmin)
    return [D * sc[e // 16] * q[e] - Dm * m[e // 16] for e in range(256)]


def exact_q80(d, q):
    D = f16_exact(d)
    return [D * q[e] for e in range(32)]


def exact_q40(d, q):
    D = f16_exact(d)
    return [D * (q[e] - 8) for e in range(32)]


def exact_q5k(d, dmin, sc, m, q):
    D, Dm = f16_exact(d), f16_exact(dmin)
    return [D * sc[e // 32] * q[e] - Dm * m[e // 32] for e in range(256)]


def exact_q3k(d, sc, q):
    D = f16_exact(d)
    return [D * (sc[e // 16] - 32) * q[e] for e in range(256)]


def round_f32(fr):
    """Correctly rounded fp32 of an exact rational whose numerator over 2^-24
    fits in 53 bits (true for every block weight): float() is then exact and
    the float64 -> float32 cast is the single rounding."""
    f = float(fr)
    assert Fraction(f) == fr
    return np.float32(f)


# ---- random fields -----------------------------------------------------------

def random_fields(qtype, rng, subnormal_d=False):
    def scale():
        if subnormal_d:
            return int(rng.integers(1, 1024))  # fp16 subnormal bit patterns
        return f16_bits(abs(rng.standard_normal()) * 1e-3)

    if qtype == Q4_K:
        return dict(d=scale(), dmin=scale(), sc=[int(v) for v in rng.integers(0, 64, 8)],
                    m=[int(v) for v in rng.integers(0, 64, 8)], q=[int(v) for v in rng.integers(0, 16, 256)])
    if qtype == Q6_K:
        return dict(d=scale(), sc=[int(v) for v in rng.integers(-128, 128, 16)],
                    q=[int(v) for v in rng.integers(0, 64, 256)])
    if qtype == Q2_K:
        return dict(d=scale(), dmin=scale(), sc=[int(v) for v in rng.integers(0, 16, 16)],
                    m=[int(v) for v in rng.integers(0, 16, 16)], q=[int(v) for v in rng.integers(0, 4, 256)])
    if qtype == Q4_0:
        return dict(d=scale(), q=[int(v) for v in rng.integers(0, 16, 32)])
    if qtype == Q5_K:
        return dict(d=scale(), dmin=scale(), sc=[int(v) for v in rng.integers(0, 64, 8)],
                    m=[int(v) for v in rng.integers(0, 64, 8)], q=[int(v) for v in rng.integers(0, 32, 256)])
    if qtype == Q3_K:
        return dict(d=scale(), sc=[int(v) for v in rng.integers(0, 64, 16)],
                    q=[int(v) for v in rng.integers(-4, 4, 256)])
    return dict(d=scale(), q=[int(v) for v in rng.integers(-127, 128, 32)])


ENCODE = {Q4_K: encode_q4k, Q6_K: encode_q6k, Q2_K: encode_q2k, Q8_0: encode_q80,
          Q4_0: encode_q40, Q5_K: encode_q5k, Q3_K: encode_q3k}
EXACT = {Q4_K: exact_q4k, Q6_K: exact_q6k, Q2_K: exact_q2k, Q8_0: exact_q80,
         Q4_0: exact_q40, Q5_K: exact_q5k, Q3_K: exact_q3k}


def encode(qtype, f):
    return ENCODE[qtype](**f)


def exact(qtype, f):
    return EXACT[qtype](**f)
