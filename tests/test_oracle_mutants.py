"""The oracle's pins reject a wrong oracle.

Each case below plants one plausible mistake in a copy of oracle/kq_oracle.c
(a dropped term, a wrong sign, index, shift or operand order, a truncating
rounding), builds it, and runs the pin tests of tests/test_oracle.py against
it: they must fail.  Nothing here touches the GPU library."""
import concurrent.futures
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kq_oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle.py")

# (name, text in the oracle, replacement, which occurrence)
MUTANTS = [
    ("f16 subnormal scale", "if (expo == 0) v = mant;", "if (expo == 0) v = mant << 1;", 0),
    ("f16 exponent bias", "else v = (1024 + mant) << (expo - 1);", "else v = (1024 + mant) << expo;", 0),
    ("f16 sign dropped", "*out = sign ? -v : v;", "*out = v;", 0),
    ("rounding drops the last bit", "float f = (float)num;", "float f = (float)(num - num % 2);", 0),
    ("Q4_K min dropped", "return weight_from_numerator(D * sc * q - Dmin * m);",
     "return weight_from_numerator(D * sc * q);", 0),
    ("Q4_K min sign", "return weight_from_numerator(D * sc * q - Dmin * m);",
     "return weight_from_numerator(D * sc * q + Dmin * m);", 0),
    ("Q4_K high scale bits from the wrong byte", "*sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);",
     "*sc = (s[j + 4] & 15) | ((s[j] >> 6) << 4);", 0),
    ("Q4_K nibbles swapped", "q = (j % 2 == 0) ? (byte & 15) : (byte >> 4);",
     "q = (j % 2 == 0) ? (byte >> 4) : (byte & 15);", 0),
    ("Q4_K element order", "byte = b[16 + 32 * (e / 64) + e % 32];\n    q = (j",
     "byte = b[16 + e / 2];\n    q = (j", 0),
    ("Q6_K offset dropped", "return weight_from_numerator(D * sc * (q - 32));",
     "return weight_from_numerator(D * sc * q);", 0),
    ("Q6_K high-bit shift", "int high = (b[128 + 32 * h + l] >> (2 * g)) & 3;",
     "int high = (b[128 + 32 * h + l] >> g) & 3;", 0),
    ("Q6_K unsigned scales", "int sc = (int8_t)b[192 + e / 16];", "int sc = b[192 + e / 16];", 0),
    ("Q6_K low nibble choice", "int low = (g < 2) ? (lowbyte & 15) : (lowbyte >> 4);",
     "int low = (g % 2 == 0) ? (lowbyte & 15) : (lowbyte >> 4);", 0),
    ("Q2_K scale and min swapped", "int sc = b[e / 16] & 15, m = b[e / 16] >> 4;",
     "int sc = b[e / 16] >> 4, m = b[e / 16] & 15;", 0),
    ("Q2_K quant shift", "int q = (b[16 + 32 * h + t] >> (2 * s)) & 3;", "int q = (b[16 + 32 * h + t] >> s) & 3;", 0),
    ("Q2_K min dropped", "return weight_from_numerator(D * sc * q - Dmin * m);",
     "return weight_from_numerator(D * sc * q);", 1),
    ("Q8_0 unsigned quants", "int q = (int8_t)b[2 + e];", "int q = b[2 + e];", 0),
    ("Q4_0 offset dropped", "return weight_from_numerator(D * (q - 8));", "return weight_from_numerator(D * q);", 0),
    ("Q4_0 nibbles interleaved", "int q = (e < 16) ? (b[2 + e] & 15) : (b[2 + e - 16] >> 4);",
     "int q = (e % 2 == 0) ? (b[2 + e / 2] & 15) : (b[2 + e / 2] >> 4);", 0),
    ("Q5_K high bit from the wrong position", "q = low | (((b[16 + e % 32] >> j) & 1) << 4);",
     "q = low | (((b[16 + e % 32] >> (j / 2)) & 1) << 4);", 0),
    ("Q5_K high bit dropped", "q = low | (((b[16 + e % 32] >> j) & 1) << 4);", "q = low;", 0),
    ("Q3_K mask sense inverted", "int q = ((b[l] >> (e / 32)) & 1) ? low : low - 4;",
     "int q = ((b[l] >> (e / 32)) & 1) ? low - 4 : low;", 0),
    ("Q3_K scale offset dropped", "int sc = q3k_scale(b + 96, e / 16) - 32;", "int sc = q3k_scale(b + 96, e / 16);", 0),
    ("Q3_K scale top bits transposed", "int top = (s[8 + i % 4] >> (2 * (i / 4))) & 3;",
     "int top = (s[8 + i / 4] >> (2 * (i % 4))) & 3;", 0),
    ("GEMV drops the last column", "for (i = 0; i < K; ++i) {", "for (i = 0; i < K - 1; ++i) {", 0),
    ("GEMV activation row stride", "const float *xm = x + (int64_t)m * K;", "const float *xm = x + (int64_t)m;", 0),
    ("GEMV output transposed", "y[(int64_t)m * N + o] = acc;", "y[(int64_t)o * M + m] = acc;", 0),
    ("MoE routing weight ignored", "y[(int64_t)t * N + o] += p * ys[o];", "y[(int64_t)t * N + o] += ys[o];", 0),
    ("MoE per-slot activations ignored", "(x_mode ? ((int64_t)t * k + j) * K : (int64_t)t * K)",
     "((int64_t)t * K)", 0),
    ("MoE bad id not flagged", "if (err_flag) *err_flag = 1;", "if (err_flag) *err_flag = 0;", 0),
    ("MoE ids transposed", "int32_t e = ids[t * k + j];", "int32_t e = ids[j * T + t];", 0),
]


def plant(text, old, new, nth):
    at = -1
    for _ in range(nth + 1):
        at = text.index(old, at + 1)
    return text[:at] + new + text[at + len(old):]


def run_pins_against(name, old, new, nth, workdir):
    text = open(SRC).read()
    assert text.count(old) > nth, "mutation site not found: %s" % name
    mutant = plant(text, old, new, nth)
    tag = "".join(c if c.isalnum() else "_" for c in name)
    csrc = os.path.join(workdir, tag + ".c")
    so = os.path.join(workdir, "lib" + tag + ".so")
    with open(csrc, "w") as f:
        f.write(mutant)
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-shared", "-fPIC", csrc, "-o", so, "-lm"])
    env = dict(os.environ, KQ_ORACLE_LIB=so, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    first_fail = next((ln for ln in r.stdout.splitlines() if ln.startswith("FAILED")), "")
    return name, r.returncode, first_fail


def test_every_planted_mistake_fails_a_pin(tmp_path):
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as pool:
        results = list(pool.map(lambda m: run_pins_against(*m, str(tmp_path)), MUTANTS))
    survivors = [name for (name, rc, _) in results if rc == 0]
    for (name, rc, first) in results:
        print("%-45s %s %s" % (name, "caught" if rc else "SURVIVED", first))
    assert not survivors, "pins did not catch: %s" % survivors
