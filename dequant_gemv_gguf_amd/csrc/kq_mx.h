// kq_mx.h -- the matrix-core form of the dequant-GEMV for Q4_K and Q6_K rows
// of at least 4096 columns, at M = 1..8 activation rows (included by
// kq_impl.h; uses its format helpers, segment cursor and buffer loads).
//
// The multiply-accumulate of the fused GEMV (weights expanded only in
// registers, several positions per pass: Kortex summary, section Approach;
// Kortex article, section Key components, item 3) is moved from the vector
// ALU to the matrix cores with the 4x4x4 f16 instruction of 16 blocks:
//
//  * a block of four lanes holds four ROWS at the same unit of 64 weights
//    (lane 4u + r: row r of the wave step, unit u of the stripe).  Its B
//    operand is the lane's own four weights of one 4-weight group -- the
//    quants as fp16 subnormal patterns, exactly as the vector path unpacks
//    them (a 4-bit q in the low bits of a half is q * 2^-24);
//  * the four A rows are the activations of that group as fp16 limbs:
//    row 2j + l is limb l (high, low) of position 2j of an A set, so one
//    instruction serves two positions and M = 8 needs four;
//  * element t of lane 4u + r's result is then row r's dot with A row t:
//    each lane accumulates its own row's sums for every position.  An output
//    element depends only on its own A row, B column and accumulator, so a
//    position's bits do not depend on M or on which A row carries it.
//
// Activations are scaled per (unit, position) by a power of two so that the
// largest of the unit's 64 values lies in [2^14, 2^15) before the split into
// two fp16 limbs (x = hi + lo to 22 bits); the scale is undone exactly on the
// unit's sum.  Per unit and position:
//   aq = sum over sub-blocks of scale * (sum of q * x over the sub-block)
//   am = sum over sub-blocks of min * (sum of x over the sub-block)
//   v  = aq * 2^(24 - shift) - KM * am
// with the sub-block dots accumulated by the matrix instruction in group
// order.  Row sums are ((0 + S_0) + S_1) + ... over stripes of 16 units, S_i
// the xor-butterfly sum of the stripe's unit values (lanes paired by unit
// bits 0, 1, 2, 3) -- the same for every M, launch shape and grouping.
// (included inside namespace kq)
#pragma once

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef u32 u2 __attribute__((ext_vector_type(2)));

constexpr int MX_US = 16;       // units per stripe (lane 4u + r: unit u)
constexpr int MX_G = 4;         // rows per wave step (lane 4u + r: row r)
constexpr int MX_KMIN = 4096;   // shortest rows served by this path

__device__ __forceinline__ f4 mfma4(u2 a, u2 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(h4, a), __builtin_bit_cast(h4, b), c, 0, 0, 0);
}

template <int PAT> __device__ __forceinline__ float swz(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), PAT));
}
// Sum over the 16 lanes that hold the same row (lane bits 2..5), in a fixed
// xor-butterfly: every lane ends with the same bits.
__device__ __forceinline__ float mx_stripe_sum(float v) {
    v = v + swz<0x101F>(v);   // lane ^ 4
    v = v + swz<0x201F>(v);   // lane ^ 8
    {
        const u32 b = __builtin_bit_cast(u32, v);
        const auto p = __builtin_amdgcn_permlane16_swap(b, b, false, false);   // lane ^ 16
        v = __builtin_bit_cast(float, (u32)p[0]) + __builtin_bit_cast(float, (u32)p[1]);
    }
    {
        const u32 b = __builtin_bit_cast(u32, v);
        const auto p = __builtin_amdgcn_permlane32_swap(b, b, false, false);   // lane ^ 32
        v = __builtin_bit_cast(float, (u32)p[0]) + __builtin_bit_cast(float, (u32)p[1]);
    }
    return v;
}

// ---- per-format pieces: a unit's 4-weight groups as B operands (halves in
// the group order k = 0, 2, 1, 3 -- the A operands follow the same order),
// its sub-block scales and mins, and its sub-block activation sums.
template <int T> struct MxFmt;

template <> struct MxFmt<T_Q4_K> {
    // unit = 64 weights: sub-block 0 (low nibbles, groups i = 0..7) and
    // sub-block 1 (high nibbles, 16 q); activations of group (sb, i) at
    // 32 sb + 4 i .. +3 of the unit
    static constexpr int NSB = 2, GPS = 8, SPAN = 4 * 144;
    static constexpr float KM = 1.f;
    typedef RawQ4K Raw;
    typedef RawQ4K Fields;
    static __device__ __forceinline__ Fields fields(const Raw &r) { return r; }
    static __device__ __forceinline__ u2 bop(const Fields &f, int sb, int i) {
        const u32 D = i < 4 ? f.qa[i & 3] : f.qb[i & 3];
        const u32 m = sb ? 0x00F000F0u : 0x000F000Fu;
        return (u2){D & m, (D >> 8) & m};
    }
    // aq scale per sub-block (1/16 folded into the high nibbles') and min
    static __device__ __forceinline__ void scales(const Fields &f, int g, float (&dsc)[NSB], float (&dmn)[NSB]) {
        const u32 h0 = f.h.x, h1 = f.h.y, h2 = f.h.z, h3 = f.h.w;
        const float d = half_lo(h0), dmin = half_lo(h0 >> 16);
        const u32 sel = (u32)(2 * g) | ((u32)(2 * g + 1) << 8) | 0x0C0C0000u;
        const u32 sc_lo = h1 & 0x3F3F3F3Fu, m_lo = h2 & 0x3F3F3F3Fu;
        const u32 sc_hi = (h3 & 0x0F0F0F0Fu) | ((h1 >> 2) & 0x30303030u);
        const u32 m_hi = ((h3 >> 4) & 0x0F0F0F0Fu) | ((h2 >> 2) & 0x30303030u);
        const u32 sc = __builtin_amdgcn_perm(sc_hi, sc_lo, sel);
        const u32 mm = __builtin_amdgcn_perm(m_hi, m_lo, sel);
        dsc[0] = d * (float)(sc & 0xFFu);
        dsc[1] = (d * 0.0625f) * (float)((sc >> 8) & 0xFFu);
        dmn[0] = dmin * (float)(mm & 0xFFu);
        dmn[1] = dmin * (float)((mm >> 8) & 0xFFu);
    }
    // sub-block sums from the unit's four 16-sums (runs at 0, 16, 32, 48)
    static __device__ __forceinline__ float sbsum(const float (&s)[4], int sb) { return sb ? s[2] + s[3] : s[0] + s[1]; }
};

template <> struct MxFmt<T_Q6_K> {
    // unit = 64 weights in four runs g of 16 (activations at 32 g .. +15 of
    // the unit's first), one scale each; runs 2 and 3 carry 16 q; groups
    // i = 0..3 of a run at 32 g + 4 i
    static constexpr int NSB = 4, GPS = 4, SPAN = 4 * 210;
    static constexpr float KM = 32.f;
    typedef RawQ6K Raw;
    typedef Q6KFields Fields;
    static __device__ __forceinline__ Fields fields(const Raw &r) { return ::kq::fields(r); }
    static __device__ __forceinline__ u2 bop(const Fields &f, int g, int k) {
        const u32 A = f.a[k], B = f.b[k], H = f.hq[k];
        switch (g) {
        case 0: return (u2){(A & 0x000F000Fu) | ((H << 4) & 0x00300030u), ((A >> 8) & 0x000F000Fu) | ((H >> 4) & 0x00300030u)};
        case 1: return (u2){(B & 0x000F000Fu) | ((H << 2) & 0x00300030u), ((B >> 8) & 0x000F000Fu) | ((H >> 6) & 0x00300030u)};
        case 2: return (u2){(A & 0x00F000F0u) | ((H << 4) & 0x03000300u), ((A >> 8) & 0x00F000F0u) | ((H >> 4) & 0x03000300u)};
        default: return (u2){(B & 0x00F000F0u) | ((H << 2) & 0x03000300u), ((B >> 8) & 0x00F000F0u) | ((H >> 6) & 0x03000300u)};
        }
    }
    static __device__ __forceinline__ void scales(const Fields &f, int sub, float (&dsc)[NSB], float (&dmn)[NSB]) {
        const int q2 = sub & 1;
        const u32 sel = (u32)q2 | ((u32)(q2 + 2) << 8) | ((u32)(q2 + 4) << 16) | ((u32)(q2 + 6) << 24);
        const u32 p = __builtin_amdgcn_perm(f.s1, f.s0, sel);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            dmn[g] = f.d * (float)(int)(signed char)(p >> (8 * g));
            dsc[g] = g < 2 ? dmn[g] : dmn[g] * 0.0625f;
        }
    }
    static __device__ __forceinline__ float sbsum(const float (&s)[4], int g) { return s[g]; }
};

template <int T> constexpr bool MX_FMT() { return T == T_Q4_K || T == T_Q6_K; }

// Weight ring geometry: a wave step is 4 rows x one stripe (16 units = 4
// blocks) of each, copied into LDS by buffer-to-LDS loads of 16 bytes a lane
// (one load covers 1 KB): piece p of a step is row p / PPR, bytes 16 (p % PPR)
// of its stripe, and lands at 16 p of the slot, so row r's stripe starts at
// 16 PPR r.  Q4_K stripes are 576 bytes (36 pieces, 16-byte aligned); Q6_K
// stripes are 840 bytes, 8-byte aligned for rows of K a multiple of 1024 (53
// pieces, the last 8 bytes past the stripe unused; past the matrix they read
// as zeros).  The last load of a step is switched off on the lanes past the
// step's pieces (a switched-off lane writes no LDS).
template <int T> struct MxRing;
template <> struct MxRing<T_Q4_K> {
    static constexpr int PPR = 36, NLD = 3, ROWB = 16 * PPR, SLOT = 4 * ROWB;
};
template <> struct MxRing<T_Q6_K> {
    static constexpr int PPR = 53, NLD = 4, ROWB = 16 * PPR, SLOT = 4 * ROWB;
};

// Q6_K unit from a ring slot: the same dword-aligned fields as load_unit reads
// from memory (blk: the block's first byte in LDS, 2-byte aligned)
__device__ __forceinline__ void read_unit(RawQ6K &r, const char *blk, int sub) {
    const int h = sub >> 1, q2 = sub & 1;
    const u32 sh = (u32)(uintptr_t)blk & 3u;
    const u32 *b = reinterpret_cast<const u32 *>(blk - sh);
    const int oa = (64 * h + 16 * q2) >> 2, oh = (128 + 32 * h + 16 * q2) >> 2, os = (192 + 8 * h) >> 2;
    r.a = (u4){b[oa], b[oa + 1], b[oa + 2], b[oa + 3]};
    r.a4 = b[oa + 4];
    r.b = (u4){b[oa + 8], b[oa + 9], b[oa + 10], b[oa + 11]};
    r.b4 = b[oa + 12];
    r.hq = (u4){b[oh], b[oh + 1], b[oh + 2], b[oh + 3]};
    r.h4 = b[oh + 4];
    r.s0 = b[os];
    r.s1 = b[os + 1];
    r.s2 = b[os + 2];
    r.dw = b[52];
    r.sh = sh;
}

// Staged activations of one position and one K chunk, as the A operands need
// them: for every 4 activations x0..x3 (elements 4j .. 4j+3 of the chunk) 16
// bytes -- the high limbs (x0, x2 | x1, x3) then the low limbs in the same
// order -- with 8 bytes of padding every 64 activations; the 16-sums of the
// fp32 activations; and per 128 activations the factor 2^(24 - shift) that
// undoes their scaling.  Offsets in bytes from the staging base.
__host__ __device__ constexpr int mx_limb_off(int j4) { return 16 * j4 + 8 * (j4 >> 4); }
__host__ __device__ constexpr size_t mx_stage_bytes(int cs) {
    // limbs (cs * 1024 activations), 16-sums (cs * 64), factors (cs * 8)
    return (size_t)mx_limb_off(cs * 256) + (size_t)cs * 64 * 4 + (size_t)cs * 8 * 4;
}

// One side of a launch (one format): this work-group's row slots.  Row
// steps are 4 rows (numbered rows of the segments, starts padded to 4); row
// slot rs of work-group b takes steps b * RS + rs + n * (nwg * RS).  A row
// is cut into stripes of 16 units; a work-group's waves cover `cs` stripes of
// one K chunk; chunk after chunk the same row steps are walked and the
// stripe sums added to the outputs in stripe order.
template <int T, int M, int D> struct MxSide {
    typedef MxFmt<T> X;
    typedef MxRing<T> RG;
    typedef typename X::Raw Raw;
    typedef typename X::Fields Fields;
    static constexpr int NA = (M + 1) / 2;                // A sets (two positions each)
    static constexpr int NG = X::NSB * X::GPS;            // 4-weight groups per unit (16)
    static constexpr int SLOT = RG::SLOT;
    // the sub-block activation sums: registers, or for Q6_K at M >= 5 (four
    // sub-blocks a unit) a per-wave LDS table [M][16 units][4]
    static constexpr bool SXL = (T == T_Q6_K && M >= 5);
    static constexpr int SXN = SXL ? 1 : M;
    static constexpr size_t SXL_BYTES = SXL ? (size_t)M * MX_US * X::NSB * 4 : 0;
    const Segs &sg;
    int64_t rb;
    int N, U, ns, cs, RS, rsl, st, wave, lane, r, u, W;
    int first_t, tstride, wsteps, nch, sub;
    SegCursor<true> cur;
    int ic, in_;                // issue position (chunk, step)
    char *ring;                 // this wave's D slots
    u32 voff[RG::NLD];          // the lane's piece offsets within a step
    // per-lane activations of the current chunk
    u2 A[NA][NG];
    float sx[SXN][X::NSB];
    float *sxl;                 // this wave's sum table (SXL)
    float sig[M];
    float keep[M];

    __device__ __forceinline__ MxSide(const Segs &s, int64_t rb_, int K, int cs_, int wave_, int lane_, int wg, int nwg,
                                      char *ring_, float *sxl_)
        : sg(s), rb(rb_), cs(cs_), wave(wave_), lane(lane_), ring(ring_), sxl(sxl_) {
        N = sg.start[sg.n];
        W = blockDim.x >> 6;
        RS = W / cs;
        rsl = wave / cs;
        st = wave - rsl * cs;
        r = lane & 3;
        u = lane >> 2;
        U = (K / Fmt<T>::QK) * Fmt<T>::UPB;
        ns = (U + MX_US - 1) / MX_US;
        nch = (ns + cs - 1) / cs;
        sub = u & 3;                                       // unit within its block (stripes hold whole blocks)
        const int nsteps = N / MX_G;
        first_t = wg * RS + rsl;
        tstride = nwg * RS;
        const int f0 = wg * RS;
        wsteps = f0 < nsteps ? (nsteps - f0 + tstride - 1) / tstride : 0;
        cur.set(sg, 0);
        ic = 0;
        in_ = 0;
#pragma unroll
        for (int k = 0; k < RG::NLD; ++k) {
            const int p = 64 * k + lane;                   // piece of the step
            const int pr = p / RG::PPR;
            voff[k] = p < 4 * RG::PPR ? (u32)((int64_t)pr * rb) + (u32)(16 * (p - RG::PPR * pr)) : OOB;
        }
#pragma unroll
        for (int m = 0; m < M; ++m) keep[m] = 0.f;
    }

    // the loads of the next step in issue order (chunk by chunk, each chunk's
    // steps in order); never conditional on the step: past the end an empty
    // buffer
    __device__ __forceinline__ void issue(int d) {
        const int c = ic, n = in_;
        if (++in_ >= wsteps) {
            in_ = 0;
            ++ic;
        }
        const int s = c * cs + st;                         // stripe
        const int t = first_t + n * tstride;
        const int row0 = MX_G * t;
        const bool live = c < nch && s < ns && wsteps > 0;
        cur.seek(sg, row0);
        const int local = row0 - cur.start;
        const int left = cur.rows - local;
        const int nr = (!live || row0 >= N || left <= 0) ? 0 : (left < MX_G ? left : MX_G);
        const int64_t soff = (int64_t)s * X::SPAN;
        const int64_t sb = rb - soff < X::SPAN ? rb - soff : X::SPAN;
        const uint8_t *base = cur.W + (nr ? (int64_t)local * rb + soff : 0);
        const rsrc_t rs = make_rsrc(base, nr ? (u32)((int64_t)(nr - 1) * rb + sb) : 0u);
        char *dst = ring + d * SLOT;
#pragma unroll
        for (int k = 0; k < RG::NLD; ++k) {
            if (k + 1 < RG::NLD || lane < 4 * RG::PPR - 64 * (RG::NLD - 1))
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (KQ_LDS void *)(dst + 1024 * k), 16, voff[k], 0, 0,
                                                         2 /* nt */);
        }
    }
    __device__ __forceinline__ void issue_first() {
#pragma unroll
        for (int d = 0; d < D; ++d) issue(d);
    }

    // Activations of one position for chunk c into the staging area, one
    // group of 16 per thread (threads past the chunk's groups -- whole waves
    // -- stage nothing): the group's loads (load_pos), then (store_pos) its
    // 16-sum, the largest magnitude of its 128-activation block (8
    // consecutive lanes) and its scaled limbs.
    __device__ __forceinline__ void load_pos(const float *__restrict__ xrow, int K, int c, f4 (&v)[4]) const {
        const int e = c * cs * MX_US * 64 + 16 * (int)threadIdx.x;
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = (f4){0.f, 0.f, 0.f, 0.f};
        if ((int)threadIdx.x < cs * MX_US * 4 && e < K) {
            const f4 *src = reinterpret_cast<const f4 *>(xrow + e);
#pragma unroll
            for (int k = 0; k < 4; ++k) v[k] = src[k];
        }
    }
    __device__ __forceinline__ void store_pos(const f4 (&v)[4], char *stg) const {
        const int idx = threadIdx.x;
        if (idx >= cs * MX_US * 4) return;
        float *ss = reinterpret_cast<float *>(stg + mx_limb_off(cs * 256));
        float *sg = ss + cs * 64;
        ss[idx] = sum16(v[0], v[1], v[2], v[3]);
        float mx = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            mx = __builtin_fmaxf(mx, __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(v[k].x), __builtin_fabsf(v[k].y)),
                                                     __builtin_fmaxf(__builtin_fabsf(v[k].z), __builtin_fabsf(v[k].w))));
        // the 128-activation block's largest (lanes 8j .. 8j+7)
        mx = __builtin_fmaxf(mx, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, mx), 0xB1,
                                                                                          0xF, 0xF, false)));
        mx = __builtin_fmaxf(mx, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, mx), 0x4E,
                                                                                          0xF, 0xF, false)));
        mx = __builtin_fmaxf(mx, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, mx), 0x141,
                                                                                          0xF, 0xF, false)));
        // scale so that the largest lies in [2^14, 2^15) (at most by 2^127)
        int sh = 0;
        if (mx > 0.f && mx <= 3.0e38f) {
            sh = 15 - __builtin_amdgcn_frexp_expf(mx);
            sh = sh < -103 ? -103 : (sh > 127 ? 127 : sh);
        }
        if ((idx & 7) == 0) sg[idx >> 3] = __builtin_ldexpf(1.0f, 24 - sh);
        const float sc = __builtin_ldexpf(1.0f, sh);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float a0 = v[k].x * sc, a1 = v[k].y * sc, a2 = v[k].z * sc, a3 = v[k].w * sc;
            const auto h02 = __builtin_amdgcn_cvt_pkrtz(a0, a2), h13 = __builtin_amdgcn_cvt_pkrtz(a1, a3);
            const auto l02 = __builtin_amdgcn_cvt_pkrtz(a0 - (float)h02[0], a2 - (float)h02[1]);
            const auto l13 = __builtin_amdgcn_cvt_pkrtz(a1 - (float)h13[0], a3 - (float)h13[1]);
            *reinterpret_cast<u4 *>(stg + mx_limb_off(4 * idx + k)) =
                (u4){__builtin_bit_cast(u32, h02), __builtin_bit_cast(u32, h13), __builtin_bit_cast(u32, l02),
                     __builtin_bit_cast(u32, l13)};
        }
    }
    // the lane's unit: its sub-block sums and factor for position P and, in
    // its A role (A set P / 2, rows 2 (P % 2) + limb), its limbs
    template <int P> __device__ __forceinline__ void take_pos(const char *stg) {
        const float *ss = reinterpret_cast<const float *>(stg + mx_limb_off(cs * 256));
        const float *sg = ss + cs * 64;
        const int e0 = unit_e0<T>(st * MX_US + u);          // within the chunk
        float s4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) s4[j] = ss[(e0 >> 4) + sum_run_stride<T>() * j];
        if constexpr (SXL) {
            if (r == 0) *reinterpret_cast<f4 *>(sxl + (P * MX_US + u) * 4) = (f4){s4[0], s4[1], s4[2], s4[3]};
        } else {
#pragma unroll
            for (int sb = 0; sb < X::NSB; ++sb) sx[P][sb] = X::sbsum(s4, sb);
        }
        sig[P] = sg[e0 >> 7];
        if ((r >> 1) == (P & 1)) {
            const int limb = r & 1;
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const int sb = g / X::GPS, i = g - sb * X::GPS;
                A[P / 2][g] = *reinterpret_cast<const u2 *>(stg + mx_limb_off((e0 + 32 * sb + 4 * i) >> 2) + 8 * limb);
            }
        }
    }
    // position by position: the next position's loads are issued before this
    // one's limbs are taken, so their latency hides behind it
    template <int P = 0> __device__ __forceinline__ void setup_rest(const float *__restrict__ x, int K, int c,
                                                                     char *stg, f4 (&v)[4]) {
        if constexpr (P < M) {
            store_pos(v, stg);
            wg_sync<true>();
            if constexpr (P + 1 < M) load_pos(x + (int64_t)(P + 1) * K, K, c, v);
            take_pos<P>(stg);
            wg_sync<true>();
            setup_rest<P + 1>(x, K, c, stg, v);
        }
    }
    __device__ __forceinline__ void setup_chunk(const float *__restrict__ x, int K, int c, char *stg) {
#pragma unroll
        for (int s = 0; s < NA; ++s)
#pragma unroll
            for (int g = 0; g < NG; ++g) A[s][g] = (u2){0u, 0u};
        f4 v[4];
        load_pos(x, K, c, v);
        setup_rest<0>(x, K, c, stg, v);
    }

    // the step's row sums of every position, parked in lane 4 (n mod 16) + r
    __device__ __forceinline__ void value(const Raw &raw, bool act, int n) {
        const Fields f = X::fields(raw);
        float dsc[X::NSB], dmn[X::NSB];
        X::scales(f, sub, dsc, dmn);
        float aq[2 * NA];
        // each sub-block's dot is folded into aq as its chain ends, in
        // ascending sub-block order
        auto fold = [&](int sb, int s, const f4 &acc) {
            const float p0 = acc.x + acc.y, p1 = acc.z + acc.w;
            aq[2 * s] = sb ? __builtin_fmaf(dsc[sb], p0, aq[2 * s]) : dsc[0] * p0;
            aq[2 * s + 1] = sb ? __builtin_fmaf(dsc[sb], p1, aq[2 * s + 1]) : dsc[0] * p1;
        };
        if constexpr (NA == 1) {
            // one A set: the sub-blocks' chains side by side
            f4 acc[X::NSB];
#pragma unroll
            for (int sb = 0; sb < X::NSB; ++sb) acc[sb] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < X::GPS; ++i)
#pragma unroll
                for (int sb = 0; sb < X::NSB; ++sb) acc[sb] = mfma4(A[0][sb * X::GPS + i], X::bop(f, sb, i), acc[sb]);
#pragma unroll
            for (int sb = 0; sb < X::NSB; ++sb) fold(sb, 0, acc[sb]);
        } else {
#pragma unroll
            for (int sb = 0; sb < X::NSB; ++sb) {
                f4 acc[NA];
#pragma unroll
                for (int s = 0; s < NA; ++s) acc[s] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < X::GPS; ++i) {
                    const u2 b = X::bop(f, sb, i);
#pragma unroll
                    for (int s = 0; s < NA; ++s) acc[s] = mfma4(A[s][sb * X::GPS + i], b, acc[s]);
                }
#pragma unroll
                for (int s = 0; s < NA; ++s) fold(sb, s, acc[s]);
            }
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float xm[X::NSB];
            if constexpr (SXL) {
                const f4 t = *reinterpret_cast<const f4 *>(sxl + (m * MX_US + u) * 4);
                xm[0] = t.x;
                xm[1] = t.y;
                xm[2] = t.z;
                xm[3] = t.w;
            } else {
#pragma unroll
                for (int sb = 0; sb < X::NSB; ++sb) xm[sb] = sx[m][sb];
            }
            float am = dmn[0] * xm[0];
#pragma unroll
            for (int sb = 1; sb < X::NSB; ++sb) am = __builtin_fmaf(dmn[sb], xm[sb], am);
            const float v = __builtin_fmaf(aq[m], sig[m], -X::KM * am);
            const float Sm = mx_stripe_sum(act ? v : 0.f);
            keep[m] = (u == (n & (MX_US - 1))) ? Sm : keep[m];
        }
    }

    // Stripe sums of steps [n0, n0 + 16) of chunk c: through LDS (the staging
    // area, idle between chunk set-ups), added to the outputs in stripe order
    // by the row slot's first stripe wave (every wave calls this at the same
    // steps).
    __device__ __forceinline__ void flush(int n0, int c, float *part) {
        const int nst = ns - c * cs < cs ? ns - c * cs : cs;  // stripes of this chunk
#pragma unroll
        for (int m = 0; m < M; ++m) part[(m * W + wave) * 64 + lane] = keep[m];
        wg_sync<true>();
        const int n = n0 + (lane >> 2);
        if (st == 0 && n < wsteps) {
            const int row = MX_G * (first_t + n * tstride) + r;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                float *o = out_of<true>(sg, N, row, m);
                if (o) {
                    float s = c == 0 ? 0.f : *o;
                    for (int w = 0; w < nst; ++w) s += part[(m * W + rsl * cs + w) * 64 + lane];
                    *o = s;
                }
            }
        }
        wg_sync<true>();
    }

    // walk every chunk's steps (chunk by chunk, the ring running across
    // chunks); the first D steps were issued (issue_first).  Every branch
    // below depends only on values uniform over the work-group, so the
    // barriers inside the chunk set-up and the flushes are reached by all
    // waves together.
    __device__ __forceinline__ void run(const float *__restrict__ x, int K, char *stg) {
        float *part = reinterpret_cast<float *>(stg);
        const int total = nch * wsteps;
        int c = 0, n = 0;
        bool act = st < ns && st * MX_US + u < U;
        for (int q0 = 0; q0 < total; q0 += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                if (q0 + d < total) {
                    if (n == 0 && c > 0) {
                        setup_chunk(x, K, c, stg);
                        const int s = c * cs + st;
                        act = s < ns && s * MX_US + u < U;
                    }
                    Raw rw;
                    wait_vm<RG::NLD * (D - 1)>();
                    read_unit(rw, ring + d * SLOT + RG::ROWB * r + Fmt<T>::BYTES * (u >> 2), sub);
                    wait_lgkm0();
                    issue(d);
                    value(rw, act, n);
                    if ((n & (MX_US - 1)) == MX_US - 1 || n + 1 == wsteps) flush(n & ~(MX_US - 1), c, part);
                    if (++n == wsteps) {
                        n = 0;
                        ++c;
                    }
                }
            }
            // keep the waves of the work-group in step (one barrier per ring turn)
            wg_sync<true>();
        }
        wait_vm<0>();
    }
};

// LDS of an mx launch: the staging area of one position's K chunk (the flush
// area [M][W][64] lives there too: it is used only between chunk set-ups),
// then the weight ring, 16-byte aligned.
__host__ __device__ constexpr size_t mx_ring_offset(int M, int W, int cs) {
    return ((mx_stage_bytes(cs) > (size_t)M * W * 64 * 4 ? mx_stage_bytes(cs) : (size_t)M * W * 64 * 4) + 15) &
           ~(size_t)15;
}

// Ring depth per format and M (slots of 2304 bytes for Q4_K, 3392 for Q6_K):
// what fits 160 KB beside a 14-stripe chunk of activations
template <int T, int M> constexpr int MX_D() { return M <= 2 ? (T == T_Q4_K ? 3 : 2) : 4; }
// work-group size bound: 16 waves (128 VGPRs) for one A set, else 8 (256)
template <int M> constexpr int MX_LB() { return M <= 2 ? 1024 : 512; }

template <int T, int M, int D>
__device__ __forceinline__ void mx_side(const Segs &sg, int64_t rb, int K, int cs, int wg, int nwg,
                                        const float *__restrict__ x, char *smem) {
    typedef MxSide<T, M, D> S;
    const int W = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    char *rings = smem + mx_ring_offset(M, W, cs);
    char *ring = rings + (size_t)wave * D * S::SLOT;
    float *sxl = reinterpret_cast<float *>(rings + (size_t)W * D * S::SLOT + (size_t)wave * S::SXL_BYTES);
    S p(sg, rb, K, cs, wave, lane, wg, nwg, ring, sxl);
    p.issue_first();
    p.setup_chunk(x, K, 0, smem);
    p.run(x, K, smem);
}

// One launch over the segments sb (format TB, the first gb work-groups) and sa
// (format TA, the rest); TA == TB: one format, sa empty.
template <int TA, int TB, int M>
__global__ __launch_bounds__(MX_LB<M>()) void qgemv_mx_kernel(const Segs sa, int64_t rba, const Segs sb, int64_t rbb,
                                                               int gb, int K, int cs, const float *__restrict__ x) {
    extern __shared__ float smem_f[];
    char *smem = reinterpret_cast<char *>(smem_f);
    if ((int)blockIdx.x < gb)
        mx_side<TB, M, MX_D<TB, M>()>(sb, rbb, K, cs, blockIdx.x, gb, x, smem);
    else if constexpr (TA != TB)
        mx_side<TA, M, MX_D<TA, M>()>(sa, rba, K, cs, blockIdx.x - gb, gridDim.x - gb, x, smem);
}

// ---------------------------------------------------------------------------
// Host side

// Work-group shape of an mx launch: cs stripe waves per row slot (a K chunk
// of cs stripes; chunks as even as the wave budget allows) and as many row
// slots as keep one work-group per compute unit busy.
struct MxCfg {
    int cs, W;
    size_t lds;
};
template <int TA, int TB, int M> bool mx_cfg(int K, int64_t steps, MxCfg *c) {
    const int U = K / 64;
    const int ns = (U + MX_US - 1) / MX_US;
    const int maxw = MX_LB<M>() / 64;
    // fewest chunks whose staged activations fit beside the ring
    for (int nch = (ns + maxw - 1) / maxw; nch <= ns; ++nch) {
        c->cs = (ns + nch - 1) / nch;
        int rs = maxw / c->cs;
        const int64_t per = steps / cu_count();
        if (per < rs) rs = per < 1 ? 1 : (int)per;
        c->W = c->cs * rs;
        const size_t ring =
            std::max((size_t)MX_D<TA, M>() * MxRing<TA>::SLOT + MxSide<TA, M, MX_D<TA, M>()>::SXL_BYTES,
                     (size_t)MX_D<TB, M>() * MxRing<TB>::SLOT + MxSide<TB, M, MX_D<TB, M>()>::SXL_BYTES);
        const size_t lds = mx_ring_offset(M, c->W, c->cs) + (size_t)c->W * ring;
        c->lds = lds;
        if (lds <= LDS_MAX) return true;
    }
    return false;
}

// One mx launch over the segments sa (format TA) and sb (format TB; when TA
// == TB every matrix is in sb).  Starts of both are padded to 4 rows.
template <int TA, int TB, int M>
int launch_mx(const Segs &sa, const Segs &sb, int K, const float *x, hipStream_t st) {
    const int64_t rba = Fmt<TA>::BYTES * (int64_t)(K / Fmt<TA>::QK), rbb = Fmt<TB>::BYTES * (int64_t)(K / Fmt<TB>::QK);
    const int64_t steps_a = TA == TB ? 0 : sa.start[sa.n] / MX_G, steps_b = sb.start[sb.n] / MX_G;
    MxCfg c;
    if (!mx_cfg<TA, TB, M>(K, steps_a + steps_b, &c)) return KQ_ERR_ARG;
    const int RS = c.W / c.cs;
    const int64_t need_a = (steps_a + RS - 1) / RS, need_b = (steps_b + RS - 1) / RS;
    const int64_t cap = cu_count();
    int64_t ga = need_a, gb = need_b;
    if (ga + gb > cap) {
        if (TA == TB) {
            gb = cap;
            ga = 0;
        } else {
            // a work-group makes whole row steps; the split that finishes the
            // slower side first, weighting a Q6_K byte (register ring, one
            // step in flight) as 1.3 of a Q4_K byte (ring in LDS)
            const double wa = (TA == T_Q6_K ? 1.3 : 1.0) * rba, wb = (TB == T_Q6_K ? 1.3 : 1.0) * rbb;
            double best = 0;
            for (int64_t b = 1; b < cap && b <= need_b; ++b) {
                const int64_t a = cap - b;
                const double t = std::max((double)((need_a + a - 1) / a) * wa, (double)((need_b + b - 1) / b) * wb);
                if (b == 1 || t < best) {
                    best = t;
                    gb = b;
                }
            }
            ga = cap - gb < need_a ? cap - gb : need_a;
        }
    }
    const int grid = (int)(ga + gb);
    if (grid == 0) return KQ_OK;
    auto kern = qgemv_mx_kernel<TA, TB, M>;
    if (allow_lds(kern, c.lds) != hipSuccess) return KQ_ERR_LAUNCH;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * c.W), c.lds, st, sa, rba, sb, rbb, (int)gb, K, c.cs, x);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_LAUNCH;
}

template <int TA, int TB>
int launch_mx_m(int M, const Segs &sa, const Segs &sb, int K, const float *x, hipStream_t st) {
    switch (M) {
    case 1: return launch_mx<TA, TB, 1>(sa, sb, K, x, st);
    case 2: return launch_mx<TA, TB, 2>(sa, sb, K, x, st);
    case 3: return launch_mx<TA, TB, 3>(sa, sb, K, x, st);
    case 4: return launch_mx<TA, TB, 4>(sa, sb, K, x, st);
    case 5: return launch_mx<TA, TB, 5>(sa, sb, K, x, st);
    case 6: return launch_mx<TA, TB, 6>(sa, sb, K, x, st);
    case 7: return launch_mx<TA, TB, 7>(sa, sb, K, x, st);
    default: return launch_mx<TA, TB, 8>(sa, sb, K, x, st);
    }
}

// Whether a format and row length take the matrix-core path (every call on
// such a matrix does, whatever M, N and grouping: its rows keep one set of
// bits).
template <int T> constexpr bool mx_format() { return MX_FMT<T>(); }
inline bool mx_rows(int K) { return K >= MX_KMIN && K % 1024 == 0 && K <= (1 << 20); }
