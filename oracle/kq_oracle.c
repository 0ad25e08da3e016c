/*
 * kq_oracle.c -- plain, slow, obviously correct CPU oracle for the fused
 * K-quant dequant-GEMV.  TEST INFRASTRUCTURE ONLY: it exists so that the
 * tests, the smoke check and the CPU-baseline leg of the benchmark have an
 * independent answer to compare the GPU library against.  It shares no code,
 * header, table or helper with the GPU library and must never be linked into
 * it.
 *
 * What is computed, and where it comes from:
 *  - The pages describe engines whose quantized weights are expanded to real
 *    values only inside the matmul (Kortex, "Out-of-core LLM inference engine
 *    written from scratch in Rust", section Approach; "Kortex: Streaming 70B
 *    Models on Consumer GPUs", section Key components, item 3) and list native
 *    kernels for the GGUF K-quants Q2_K..Q6_K, Q4_0 and Q8_0 ("RunNburn - Run
 *    a 295B Moe from a 98GB GGUF on a 64GB RAM Desktop", the post).  Because the
 *    expansion happens only in registers, the fused result equals the plain
 *    definition written out here: expand every weight, then take the dot.
 *  - The pages give no byte layout.  The block layouts below follow the GGUF
 *    K-quant convention (outside the pages; a reading):
 *      Q4_K: 256 weights in 144 B, w = d*sc*q - dmin*m, 6-bit sc/m per 32.
 *      Q6_K: 256 weights in 210 B, w = d*sc*(q - 32), int8 sc per 16.
 *      Q2_K: 256 weights in  84 B, w = d*sc*q - dmin*m, 4-bit sc/m per 16.
 *      Q8_0:  32 weights in  34 B, w = d*q.
 *      Q4_0:  32 weights in  18 B, w = d*(q - 8), 4-bit q.
 *      Q5_K: 256 weights in 176 B, w = d*sc*q - dmin*m, 5-bit q, Q4_K scales.
 *      Q3_K: 256 weights in 110 B, w = d*(sc - 32)*q, q in -4..3, 6-bit sc
 *            per 16.
 *  - Several positions per pass (the speculative-verify pass of the Kortex
 *    page, section Approach) are M independent activation rows.
 *  - The MoE variant gathers the experts each token selected (the RunNburn
 *    post) and combines them with the routing weights.
 *
 * Arithmetic: every finite fp16 value is an integer multiple of 2^-24, so the
 * weight numerator n = w * 2^24 is an exact int64; the fp32 weight is the
 * single round-to-nearest-even conversion of n, scaled by 2^-24 (exact).  This
 * is the correctly rounded fp32 value of the exact real weight.  Dots are
 * taken in fp64 in ascending index order; every fp32*fp32 product is exact in
 * fp64.  No blocking, fusion or reordering.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC kq_oracle.c -o libkq_oracle.so -lm
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OT_Q4_0 = 2, OT_Q8_0 = 8, OT_Q2_K = 10, OT_Q3_K = 11, OT_Q4_K = 12, OT_Q5_K = 13, OT_Q6_K = 14 };

/* ---- fp16 ------------------------------------------------------------ */

/* IEEE binary16, little-endian in memory.  Returns 1 and the value times
 * 2^24 as an exact integer when the value is finite, 0 otherwise. */
static int f16_times_2p24(const uint8_t *p, int64_t *out)
{
    uint16_t h = (uint16_t)(p[0] | (p[1] << 8));
    int sign = h >> 15;
    int expo = (h >> 10) & 31;
    int64_t mant = h & 1023;
    int64_t v;
    if (expo == 31) return 0;
    if (expo == 0) v = mant;                      /* subnormal: mant * 2^-24 */
    else v = (1024 + mant) << (expo - 1);         /* (1024+mant) * 2^(expo-25) */
    *out = sign ? -v : v;
    return 1;
}

static double f16_double(const uint8_t *p)
{
    uint16_t h = (uint16_t)(p[0] | (p[1] << 8));
    int sign = h >> 15, expo = (h >> 10) & 31, mant = h & 1023;
    double v;
    if (expo == 31) v = mant ? NAN : INFINITY;
    else if (expo == 0) v = ldexp((double)mant, -24);
    else v = ldexp((double)(1024 + mant), expo - 25);
    return sign ? -v : v;
}

/* The fp32 weight of exact value num * 2^-24 (num an exact integer). */
static float weight_from_numerator(int64_t num)
{
    float f = (float)num;               /* one round-to-nearest-even */
    return f * 0x1p-24f;                /* exact: power-of-two scale, no subnormal */
}

/* ---- per-type block decode, one element at a time --------------------- */

/* Q4_K, 144 B: [0,2) d, [2,4) dmin, [4,16) eight 6-bit scales and eight 6-bit
 * mins, [16,144) 128 B of 4-bit quants.  Sub-block j = e/32 uses scale sc_j
 * and min m_j; scales 0..3 sit in the low 6 bits of bytes 0..3 (mins in bytes
 * 4..7); scales 4..7 take their low 4 bits from the low nibble of bytes 8..11
 * and their top 2 bits from the top of bytes 0..3 (mins: high nibble of bytes
 * 8..11 and top of bytes 4..7).  Element e lives in quant byte
 * 32*(e/64) + e%32, low nibble for even j, high nibble for odd j. */
static void q4k_scale_min(const uint8_t *s, int j, int *sc, int *m)
{
    if (j < 4) {
        *sc = s[j] & 63;
        *m = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
        *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

static float q4k_element(const uint8_t *b, int e)
{
    int64_t D, Dmin;
    int j = e / 32, sc, m, q;
    uint8_t byte;
    if (!f16_times_2p24(b, &D) || !f16_times_2p24(b + 2, &Dmin)) {
        int sc2, m2, q2;
        q4k_scale_min(b + 4, j, &sc2, &m2);
        byte = b[16 + 32 * (e / 64) + e % 32];
        q2 = (j % 2 == 0) ? (byte & 15) : (byte >> 4);
        return (float)(f16_double(b) * sc2 * q2 - f16_double(b + 2) * m2);
    }
    q4k_scale_min(b + 4, j, &sc, &m);
    byte = b[16 + 32 * (e / 64) + e % 32];
    q = (j % 2 == 0) ? (byte & 15) : (byte >> 4);
    return weight_from_numerator(D * sc * q - Dmin * m);
}

/* Q6_K, 210 B: [0,128) low 4 bits, [128,192) high 2 bits, [192,208) sixteen
 * int8 scales (one per 16 weights), [208,210) d.  For element e: h = e/128,
 * g = (e%128)/32, l = e%32; low bits from byte 64h + 32*(g%2) + l (low nibble
 * for g < 2, high nibble otherwise), high bits are bits 2g..2g+1 of byte
 * 128 + 32h + l; q = low | high<<4 in 0..63, weight d*sc*(q-32). */
static float q6k_element(const uint8_t *b, int e)
{
    int h = e / 128, g = (e % 128) / 32, l = e % 32;
    uint8_t lowbyte = b[64 * h + 32 * (g % 2) + l];
    int low = (g < 2) ? (lowbyte & 15) : (lowbyte >> 4);
    int high = (b[128 + 32 * h + l] >> (2 * g)) & 3;
    int q = low | (high << 4);
    int sc = (int8_t)b[192 + e / 16];
    int64_t D;
    if (!f16_times_2p24(b + 208, &D)) return (float)(f16_double(b + 208) * sc * (q - 32));
    return weight_from_numerator(D * sc * (q - 32));
}

/* Q2_K, 84 B: [0,16) one byte per 16 weights (low nibble scale, high nibble
 * min), [16,80) 2-bit quants, [80,82) d, [82,84) dmin.  For element e:
 * h = e/128, s = (e%128)/32, t = e%32; q = bits 2s..2s+1 of byte 16 + 32h + t. */
static float q2k_element(const uint8_t *b, int e)
{
    int h = e / 128, s = (e % 128) / 32, t = e % 32;
    int q = (b[16 + 32 * h + t] >> (2 * s)) & 3;
    int sc = b[e / 16] & 15, m = b[e / 16] >> 4;
    int64_t D, Dmin;
    if (!f16_times_2p24(b + 80, &D) || !f16_times_2p24(b + 82, &Dmin))
        return (float)(f16_double(b + 80) * sc * q - f16_double(b + 82) * m);
    return weight_from_numerator(D * sc * q - Dmin * m);
}

/* Q8_0, 34 B: [0,2) d, [2,34) 32 int8 quants; weight d*q. */
static float q80_element(const uint8_t *b, int e)
{
    int q = (int8_t)b[2 + e];
    int64_t D;
    if (!f16_times_2p24(b, &D)) return (float)(f16_double(b) * q);
    return weight_from_numerator(D * q);
}

/* Q4_0, 18 B: [0,2) d, [2,18) 4-bit quants; weight e < 16 is the low nibble
 * of quant byte e, weight e >= 16 the high nibble of byte e - 16; d*(q-8). */
static float q40_element(const uint8_t *b, int e)
{
    int q = (e < 16) ? (b[2 + e] & 15) : (b[2 + e - 16] >> 4);
    int64_t D;
    if (!f16_times_2p24(b, &D)) return (float)(f16_double(b) * (q - 8));
    return weight_from_numerator(D * (q - 8));
}

/* Q5_K, 176 B: [0,2) d, [2,4) dmin, [4,16) scales and mins packed as in
 * Q4_K, [16,48) high bits, [48,176) low 4 bits laid out as Q4_K's quants.
 * Element e: sub-block j = e/32; low 4 bits as Q4_K's element e; bit 4 is
 * bit j of byte 16 + e%32. */
static float q5k_element(const uint8_t *b, int e)
{
    int j = e / 32, sc, m, low, q;
    int64_t D, Dmin;
    uint8_t byte = b[48 + 32 * (e / 64) + e % 32];
    q4k_scale_min(b + 4, j, &sc, &m);
    low = (j % 2 == 0) ? (byte & 15) : (byte >> 4);
    q = low | (((b[16 + e % 32] >> j) & 1) << 4);
    if (!f16_times_2p24(b, &D) || !f16_times_2p24(b + 2, &Dmin))
        return (float)(f16_double(b) * sc * q - f16_double(b + 2) * m);
    return weight_from_numerator(D * sc * q - Dmin * m);
}

/* Q3_K, 110 B: [0,32) high-bit mask, [32,96) 2-bit quants, [96,108) sixteen
 * 6-bit scales, [108,110) d.  Element e: h = e/128, j = (e%128)/32, l = e%32;
 * two low bits are bits 2j..2j+1 of byte 32 + 32h + l; the mask bit is bit
 * e/32 of byte l; q = low - 4 when the mask bit is clear, low when set.
 * Scale i (one per 16 weights): its low 4 bits are the low nibble of byte
 * 96 + i (i < 8) or the high nibble of byte 96 + i - 8 (i >= 8); its top 2
 * bits are bits 2*(i/4)..2*(i/4)+1 of byte 104 + i%4; weight d*(sc-32)*q. */
static int q3k_scale(const uint8_t *s, int i)
{
    int low = (i < 8) ? (s[i] & 15) : (s[i - 8] >> 4);
    int top = (s[8 + i % 4] >> (2 * (i / 4))) & 3;
    return low | (top << 4);
}

static float q3k_element(const uint8_t *b, int e)
{
    int h = e / 128, j = (e % 128) / 32, l = e % 32;
    int low = (b[32 + 32 * h + l] >> (2 * j)) & 3;
    int q = ((b[l] >> (e / 32)) & 1) ? low : low - 4;
    int sc = q3k_scale(b + 96, e / 16) - 32;
    int64_t D;
    if (!f16_times_2p24(b + 108, &D)) return (float)(f16_double(b + 108) * sc * q);
    return weight_from_numerator(D * sc * q);
}

static int block_shape(int type, int *qk, int *bytes)
{
    switch (type) {
    case OT_Q4_0: *qk = 32; *bytes = 18; return 0;
    case OT_Q5_K: *qk = 256; *bytes = 176; return 0;
    case OT_Q3_K: *qk = 256; *bytes = 110; return 0;
    case OT_Q4_K: *qk = 256; *bytes = 144; return 0;
    case OT_Q6_K: *qk = 256; *bytes = 210; return 0;
    case OT_Q2_K: *qk = 256; *bytes = 84; return 0;
    case OT_Q8_0: *qk = 32; *bytes = 34; return 0;
    default: return -1;
    }
}

static float element(int type, const uint8_t *block, int e)
{
    switch (type) {
    case OT_Q4_K: return q4k_element(block, e);
    case OT_Q6_K: return q6k_element(block, e);
    case OT_Q2_K: return q2k_element(block, e);
    case OT_Q4_0: return q40_element(block, e);
    case OT_Q5_K: return q5k_element(block, e);
    case OT_Q3_K: return q3k_element(block, e);
    default: return q80_element(block, e);
    }
}

/* ---- exported entry points ------------------------------------------- */

int oracle_block_shape(int type, int *qk, int *bytes) { return block_shape(type, qk, bytes); }

/* Expand n weights (n a multiple of the block size) to fp32. */
int oracle_dequant(int type, const uint8_t *src, int64_t n, float *dst)
{
    int qk, bytes;
    int64_t i;
    if (block_shape(type, &qk, &bytes)) return -1;
    if (n < 0 || n % qk) return -2;
    for (i = 0; i < n; ++i)
        dst[i] = element(type, src + (i / qk) * bytes, (int)(i % qk));
    return 0;
}

/* y[m][o] = sum_i w[o][i] * x[m][i], S[m][o] = sum_i |w[o][i] * x[m][i]|,
 * both in fp64, ascending i.  W is N rows of K/qk blocks each; x is M rows of
 * K fp32.  Rows are independent, so they are spread over OpenMP threads; the
 * arithmetic of each output does not depend on the thread count. */
int oracle_gemv(int type, const uint8_t *W, int64_t N, int64_t K,
                const float *x, int M, double *y, double *S)
{
    int qk, bytes;
    int64_t row_bytes, o;
    int bad = 0;
    if (block_shape(type, &qk, &bytes)) return -1;
    if (K <= 0 || K % qk || N < 0 || M < 1) return -2;
    row_bytes = (K / qk) * bytes;
#pragma omp parallel
    {
        float *w = (float *)malloc((size_t)K * sizeof(float));
        if (!w) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(static)
        for (o = 0; o < N; ++o) {
            int m;
            int64_t i;
            if (!w) continue;
            oracle_dequant(type, W + o * row_bytes, K, w);
            for (m = 0; m < M; ++m) {
                double acc = 0.0, mag = 0.0;
                const float *xm = x + (int64_t)m * K;
                for (i = 0; i < K; ++i) {
                    double p = (double)w[i] * (double)xm[i];
                    acc += p;
                    mag += fabs(p);
                }
                y[(int64_t)m * N + o] = acc;
                if (S) S[(int64_t)m * N + o] = mag;
            }
        }
        free(w);
    }
    return bad ? -3 : 0;
}

/* Routed-expert GEMV.  W_exps holds E experts of N x K blocks, expert-major.
 * ids[T][k] selects experts (out-of-range ids contribute zero and set
 * *err_flag to 1); x is x[T][K] (x_mode 0, shared by the k slots of a token)
 * or x[T][k][K] (x_mode 1).  With route_w == NULL the per-slot products are
 * written to y[T][k][N]; otherwise y[T][N] = sum_j route_w[t][j] * slot_j in
 * ascending j, fp64, and S the matching sum of |route_w| * S_slot. */
int oracle_moe(int type, const uint8_t *W_exps, int64_t E, int64_t N, int64_t K,
               const int32_t *ids, const float *route_w, int T, int k,
               const float *x, int x_mode, double *y, double *S, int32_t *err_flag)
{
    int qk, bytes, t, j;
    int64_t row_bytes, o;
    double *ys, *ss;
    if (block_shape(type, &qk, &bytes)) return -1;
    if (K <= 0 || K % qk || N < 0 || E < 1 || T < 1 || k < 1) return -2;
    row_bytes = (K / qk) * bytes;
    ys = (double *)malloc((size_t)N * sizeof(double));
    ss = (double *)malloc((size_t)N * sizeof(double));
    if (!ys || !ss) { free(ys); free(ss); return -3; }
    if (route_w) {
        for (o = 0; o < (int64_t)T * N; ++o) { y[o] = 0.0; if (S) S[o] = 0.0; }
    }
    for (t = 0; t < T; ++t) {
        for (j = 0; j < k; ++j) {
            int32_t e = ids[t * k + j];
            const float *xs = x + (x_mode ? ((int64_t)t * k + j) * K : (int64_t)t * K);
            if (e < 0 || e >= E) {
                if (err_flag) *err_flag = 1;
                for (o = 0; o < N; ++o) { ys[o] = 0.0; ss[o] = 0.0; }
            } else {
                int r = oracle_gemv(type, W_exps + (int64_t)e * N * row_bytes, N, K, xs, 1, ys, ss);
                if (r) { free(ys); free(ss); return r; }
            }
            for (o = 0; o < N; ++o) {
                if (route_w) {
                    double p = (double)route_w[t * k + j];
                    y[(int64_t)t * N + o] += p * ys[o];
                    if (S) S[(int64_t)t * N + o] += fabs(p) * ss[o];
                } else {
                    y[((int64_t)t * k + j) * N + o] = ys[o];
                    if (S) S[((int64_t)t * k + j) * N + o] = ss[o];
                }
            }
        }
    }
    free(ys);
    free(ss);
    return 0;
}

int oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}
