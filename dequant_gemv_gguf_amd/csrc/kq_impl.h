// kq_impl.h -- kernels and launchers of the fused GGUF K-quant dequant-GEMV
// library for AMD MI355X (gfx950, CDNA4) whose C ABI is include/kqgemv.h.
// Every translation unit of the library includes this file; the launchers of
// each format and of each mixed pair are instantiated in kq_inst.hip (one
// object per format or pair, compiled in parallel) and declared extern below.
//
// Prior art on the pages: fused dequant-matmul kernels that expand quantized
// weights only in registers (Kortex summary, section Approach; Kortex article,
// section Key components, item 3) and native K-quant kernels for Q2_K..Q6_K,
// Q4_0 and Q8_0 (RunNburn post).  Their designs target other hardware; this
// file is a gfx950 design of the same operation.
//
// Design (memory-bound matvec, one pass over the packed weights):
//  * Weights are read with 128-bit buffer loads (raw buffer resources give
//    hardware bounds checks: a read past the tile returns zeros, never faults).
//    Q6_K, Q3_K, Q8_0 and Q4_0 blocks may start 2 bytes off a dword; their
//    fields are read from the dword-aligned address below and realigned with
//    v_alignbyte.
//  * Each lane owns "units" of 64 weights (32 for Q8_0 and Q4_0) that share their
//    scales; a group of LPR lanes (16, 32 or 64) walks the units of R rows, so
//    one read of the activations serves R rows.  Unit u of a row always goes
//    to lane u % LPR in ascending order, whatever M, R or the K chunk, so the
//    rounding of a row's result does not depend on M (an M = 8 call gives the
//    M = 1 bits on each row).
//  * Activations are staged in LDS per K chunk (padded by 16 B every 64
//    floats so that lanes reading 256-B-strided unit slices hit distinct
//    banks), together with exact-order fp32 sums of every 16 activations for
//    the factored min / offset terms.
//  * Quants are turned into fp16 *subnormal* bit patterns with one mask per
//    two weights (a 4-bit q in the low bits of a half is exactly q * 2^-24; a
//    nibble kept in place is 16q * 2^-24) and multiplied by the fp32
//    activation with v_fma_mix_f32, which widens the half exactly.  The
//    power-of-two factors are folded into the per-sub-block scales.
//  * Per unit and sub-block: acc += (d*sc) * sum(q*x) - (dmin*m) * sum(x)
//    (Q6_K: d*sc*(sum(q*x) - 32*sum(x)); Q8_0: d*(sum((q+128)*x) - 128*sum(x));
//    Q4_0: d*(sum(q*x) - 8*sum(x)); Q3_K: d*sc*(sum((low2 + 4*hbit)*x) -
//    4*sum(x)) with q = low2 - 4 + 4*hbit; Q5_K as Q4_K with a fifth bit).
//  * Lane partials are summed with DPP inside 16-lane rows and lane swizzles
//    across rows; one lane per row group stores y.  No atomics anywhere.
//
// Kernels: qgemv1_kernel (M = 1, persistent, one work-group per compute unit,
// several matrices of one format per launch), qgemv1_dma_kernel (its Q4_K form
// with the weight ring in LDS, filled by buffer-to-LDS loads; qgemv1m_dma_kernel
// the same at M = 2),
// qgemv1_mixed_kernel (the same for two formats side by side), qgemvm_kernel (M = 2..8, persistent),
// qgemv_kernel and qgemv_seg_kernel (non-persistent, activations staged per
// work-group: small launches at M = 1 and rows too long for the persistent
// kernels), qmoe_tok_kernel (routed experts, one work-group per row tile and
// token, with the routing-weighted sum) and qmoe_kernel + moe_combine_kernel
// (routed experts grouped by expert, when a token's activations do not fit
// the former's LDS budget), dequant_kernel.  All follow the same per-row
// summation order, so a row's bits do not depend on which one computed it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kqgemv.h"

#include <algorithm>
#include <atomic>
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>
#include <vector>

namespace kq {

typedef uint32_t u32;
typedef _Float16 hf2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef u32 u4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int WG_THREADS = 256;   // 4 waves of 64
constexpr int WAVES = WG_THREADS / 64;
constexpr u32 OOB = 0x80000000u;  // an offset past every tile: loads return 0

// ---------------------------------------------------------------------------
// Format constants (GGUF convention)

enum {
    T_Q4_0 = KQ_TYPE_Q4_0, T_Q8_0 = KQ_TYPE_Q8_0, T_Q2_K = KQ_TYPE_Q2_K, T_Q3_K = KQ_TYPE_Q3_K,
    T_Q4_K = KQ_TYPE_Q4_K, T_Q5_K = KQ_TYPE_Q5_K, T_Q6_K = KQ_TYPE_Q6_K
};

template <int T> struct Fmt;
template <> struct Fmt<T_Q4_K> { static constexpr int QK = 256, BYTES = 144, UPB = 4; };
template <> struct Fmt<T_Q6_K> { static constexpr int QK = 256, BYTES = 210, UPB = 4; };
template <> struct Fmt<T_Q2_K> { static constexpr int QK = 256, BYTES = 84, UPB = 4; };
template <> struct Fmt<T_Q8_0> { static constexpr int QK = 32, BYTES = 34, UPB = 1; };
template <> struct Fmt<T_Q4_0> { static constexpr int QK = 32, BYTES = 18, UPB = 1; };
template <> struct Fmt<T_Q5_K> { static constexpr int QK = 256, BYTES = 176, UPB = 4; };
template <> struct Fmt<T_Q3_K> { static constexpr int QK = 256, BYTES = 110, UPB = 4; };
// Formats whose units carry the most raw registers (more than 4 bits a weight).
template <int T> constexpr bool BIG_UNIT() { return T == T_Q6_K || T == T_Q5_K || T == T_Q3_K; }

// ---------------------------------------------------------------------------
// Small device helpers

// A raw buffer over [base, base + nbytes).  The range check zeroes every
// dword that is not entirely inside the range, so the size is rounded up to a
// whole dword: a dword holding a valid byte never crosses a page boundary, and
// bytes past the data in it are never used.
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, u32 nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)((nbytes + 3u) & ~3u),
                                             0x00020000);
}
__device__ __forceinline__ u4 ld16(rsrc_t r, u32 off) {
    return __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ u32 ld4(rsrc_t r, u32 off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ u32 realign(u32 hi, u32 lo, u32 sh) {
    return __builtin_amdgcn_alignbyte(hi, lo, sh);
}
__device__ __forceinline__ float half_lo(u32 v) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(v & 0xFFFFu));
}
__device__ __forceinline__ hf2 as_h2(u32 v) { return __builtin_bit_cast(hf2, v); }
__device__ __forceinline__ f4 lds4(const float *p) { return *reinterpret_cast<const f4 *>(p); }

// x element e of a staged chunk lives at e + 4 * (e / 64)
__device__ __forceinline__ int xpad(int e) { return e + ((e >> 6) << 2); }

// Sum across the LPR lanes of a lane group; every lane of the group ends with
// the total.  Order is fixed by lane position only.
__device__ __forceinline__ float dpp_add(float v, int ctrl_sel) {
    int iv = __builtin_bit_cast(int, v);
    int t;
    switch (ctrl_sel) {
    case 0: t = __builtin_amdgcn_update_dpp(0, iv, 0xB1, 0xF, 0xF, false); break;   // quad_perm 1,0,3,2
    case 1: t = __builtin_amdgcn_update_dpp(0, iv, 0x4E, 0xF, 0xF, false); break;   // quad_perm 2,3,0,1
    case 2: t = __builtin_amdgcn_update_dpp(0, iv, 0x141, 0xF, 0xF, false); break;  // row_half_mirror
    default: t = __builtin_amdgcn_update_dpp(0, iv, 0x140, 0xF, 0xF, false); break; // row_mirror
    }
    return v + __builtin_bit_cast(float, t);
}
__device__ __forceinline__ float group_sum(float v, int lpr) {
    v = dpp_add(v, 0);
    v = dpp_add(v, 1);
    v = dpp_add(v, 2);
    v = dpp_add(v, 3);
    if (lpr >= 32) {   // rows of 16 lanes pairwise: lane l gets v[l] + v[l ^ 16]
        const u32 b = __builtin_bit_cast(u32, v);
        const auto p = __builtin_amdgcn_permlane16_swap(b, b, false, false);
        v = __builtin_bit_cast(float, (u32)p[0]) + __builtin_bit_cast(float, (u32)p[1]);
    }
    if (lpr >= 64) {   // halves of 32 lanes: lane l gets v[l] + v[l ^ 32]
        const u32 b = __builtin_bit_cast(u32, v);
        const auto p = __builtin_amdgcn_permlane32_swap(b, b, false, false);
        v = __builtin_bit_cast(float, (u32)p[0]) + __builtin_bit_cast(float, (u32)p[1]);
    }
    return v;
}

// group_sum of N values at once, level by level, so that no DPP read waits on
// the instruction just before it; each value gets exactly group_sum's tree.
template <int N> __device__ __forceinline__ void group_sum_n(float (&v)[N], int lpr) {
#pragma unroll
    for (int lv = 0; lv < 4; ++lv)
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = dpp_add(v[i], lv);
    if (lpr >= 32) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const u32 b = __builtin_bit_cast(u32, v[i]);
            const auto p = __builtin_amdgcn_permlane16_swap(b, b, false, false);
            v[i] = __builtin_bit_cast(float, (u32)p[0]) + __builtin_bit_cast(float, (u32)p[1]);
        }
    }
    if (lpr >= 64) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const u32 b = __builtin_bit_cast(u32, v[i]);
            const auto p = __builtin_amdgcn_permlane32_swap(b, b, false, false);
            v[i] = __builtin_bit_cast(float, (u32)p[0]) + __builtin_bit_cast(float, (u32)p[1]);
        }
    }
}

// group_sum of NV values (a power of two, at most 16) in one pass: a
// butterfly that at each of the first log2(NV) levels halves the values a lane
// holds -- it keeps one half, hands the other to its partner and adds the
// partner's copy of the half it kept -- then sums the last value like
// group_sum.  Every lane ends with the total of value scatter_idx(lane); the
// pairs added at every level are those of group_sum's tree, so each total has
// group_sum's bits.  Lane l keeps the upper half at level k iff bit k of
//   (bit0^bit2, bit1^bit2, bit2^bit3, bit3)
// is set: partners at each level differ in that bit and agree in the earlier
// ones (the partners are l^1, l^2, then the mirrors 7-j and 15-j in 8- and
// 16-lane rows).
__device__ __forceinline__ int scatter_bit(int lane, int k) {
    const int b0 = lane & 1, b1 = (lane >> 1) & 1, b2 = (lane >> 2) & 1, b3 = (lane >> 3) & 1;
    return k == 0 ? (b0 ^ b2) : k == 1 ? (b1 ^ b2) : k == 2 ? (b2 ^ b3) : b3;
}
template <int NV> __device__ __forceinline__ int scatter_idx(int lane) {
    int idx = 0, h = NV;
#pragma unroll
    for (int k = 0; (1 << k) < NV; ++k) {
        h >>= 1;
        idx += scatter_bit(lane, k) * h;
    }
    return idx;
}
__device__ __forceinline__ float dpp_get(float v, int lvl) {
    const int iv = __builtin_bit_cast(int, v);
    int t;
    switch (lvl) {
    case 0: t = __builtin_amdgcn_update_dpp(0, iv, 0xB1, 0xF, 0xF, false); break;
    case 1: t = __builtin_amdgcn_update_dpp(0, iv, 0x4E, 0xF, 0xF, false); break;
    case 2: t = __builtin_amdgcn_update_dpp(0, iv, 0x141, 0xF, 0xF, false); break;
    default: t = __builtin_amdgcn_update_dpp(0, iv, 0x140, 0xF, 0xF, false); break;
    }
    return __builtin_bit_cast(float, t);
}
template <int NV> __device__ __forceinline__ float reduce_scatter(float (&v)[NV], int lane, int lpr) {
    static_assert(NV >= 1 && NV <= 16 && (NV & (NV - 1)) == 0, "NV: power of two <= 16");
    int n = NV;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (n > 1) {
            const bool up = scatter_bit(lane, k);
            const int h = n >> 1;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (j < h) {
                    // both halves' pair sums, then this lane's half: a select
                    // of two array elements would be folded into an indexed
                    // (scratch) load of the array
                    const float lo = v[j] + dpp_get(v[j], k);
                    const float hi = v[j + h] + dpp_get(v[j + h], k);
                    v[j] = up ? hi : lo;
                }
            }
            n = h;
        } else {
            v[0] = dpp_add(v[0], k);
        }
    }
    float r = v[0];
    if (lpr >= 32) {
        const u32 b = __builtin_bit_cast(u32, r);
        const auto p = __builtin_amdgcn_permlane16_swap(b, b, false, false);
        r = __builtin_bit_cast(float, (u32)p[0]) + __builtin_bit_cast(float, (u32)p[1]);
    }
    if (lpr >= 64) {
        const u32 b = __builtin_bit_cast(u32, r);
        const auto p = __builtin_amdgcn_permlane32_swap(b, b, false, false);
        r = __builtin_bit_cast(float, (u32)p[0]) + __builtin_bit_cast(float, (u32)p[1]);
    }
    return r;
}

// ---------------------------------------------------------------------------
// Activation access.  A unit's activations are addressed by their offset from
// the unit's first weight in the unit's own coordinates (Q4_K: 0..63, one
// contiguous run; Q6_K and Q2_K: four runs of 16 at offsets 0, 32, 64, 96;
// Q8_0: 0..31) and its sums of 16 activations by run index.  The two accessors
// below return bit-identical values: the sums are formed by the same
// expression (sum16) whether they are staged in LDS or kept in registers.

__device__ __forceinline__ float sum16(f4 a, f4 b, f4 c, f4 d) {
    return (((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w))) +
           (((c.x + c.y) + (c.z + c.w)) + ((d.x + d.y) + (d.z + d.w)));
}

// Activations of a staged K chunk in LDS: row m at xs + m * XS (16 B of padding
// every 64 floats, see xpad), 16-sums at ss + m * SS.  xo / so locate the unit.
struct XLds {
    static constexpr bool FENCE = true;
    const float *xs, *ss;
    int XS, SS, xo, so, srun;
    __device__ __forceinline__ f4 x4(int m, int off) const { return lds4(xs + m * XS + xo + xpad(off)); }
    __device__ __forceinline__ float sum(int m, int run) const { return ss[m * SS + so + srun * run]; }
};

// One activation row of one unit held in registers (M = 1 kernels).
template <int T> struct XReg {
    static constexpr bool FENCE = false;
    static constexpr bool RUNS32 = (T == T_Q6_K || T == T_Q2_K || T == T_Q3_K);
    static constexpr int NV = (Fmt<T>::QK == 32) ? 8 : 16, NS = NV / 4;
    f4 v[NV];
    float s[NS];
    __device__ __forceinline__ f4 x4(int, int off) const {
        return v[RUNS32 ? ((off >> 5) << 2) + ((off & 31) >> 2) : (off >> 2)];
    }
    __device__ __forceinline__ float sum(int, int run) const { return s[run]; }
    // element offset of the unit's first activation and of run r
    __device__ __forceinline__ void load(const float *x, int e0) {
#pragma unroll
        for (int r = 0; r < NS; ++r) {
            const f4 *p = reinterpret_cast<const f4 *>(x + e0 + (RUNS32 ? 32 : 16) * r);
#pragma unroll
            for (int k = 0; k < 4; ++k) v[4 * r + k] = p[k];
        }
#pragma unroll
        for (int r = 0; r < NS; ++r) s[r] = sum16(v[4 * r], v[4 * r + 1], v[4 * r + 2], v[4 * r + 3]);
    }
};

// ---------------------------------------------------------------------------
// Per-format units.  load_* reads one unit's raw bytes for one row at byte
// offset `off` of a buffer; val_* turns R rows of raw units and M activation
// rows into the unit's contribution v[r][m] to each output, always by the same
// sequence of fp32 operations (so every kernel built on them rounds alike):
//   aq = sum over sub-blocks of (scale * sum_i q_i x_i)     (units of 2^-24)
//   am = sum over sub-blocks of (min   * sum_i x_i)
//   v  = aq * 2^24 - KM * am
// where KM folds a constant quant offset (Q6_K: 32; Q8_0: 128, from reading
// the int8 quants as q + 128).

// With activations in LDS and several activation rows, the compiler would
// otherwise read every row's activations of a unit up front and run out of
// registers: the val_* loops below read one activation row at a time, one step
// ahead of its use, and pin each step's accumulators with an empty asm
// statement that also orders memory accesses, which keeps the step's
// arithmetic and reads in program order.  Register-resident activations need
// no pinning.
template <class XA, int M> __device__ __forceinline__ void pin(float &v) {
    if constexpr (XA::FENCE && M > 1) asm volatile("" : "+v"(v) : : "memory");
}

// acc + w * x for one fp16 half of w (HI: the upper one), widened exactly
// (one rounding: the compiler emits v_fma_mix_f32, or converts the half once
// and reuses it with v_fmac_f32 across activation rows).
template <class XA, int M, bool HI> __device__ __forceinline__ float fmx(hf2 w, float x, float acc) {
    return __builtin_fmaf((float)(HI ? w.y : w.x), x, acc);
}

// Reads of the activations of step t (NV float4 each) kept XP steps ahead of
// their use in a small register ring; register-resident activations are read
// at their use (XP = 0).
constexpr int XPREF = 2;
template <class XA, int M> constexpr int xpref() { return (XA::FENCE && M > 1) ? XPREF : 0; }

// ---- Q4_K: unit (block b, group g) = quant bytes 32g..32g+31, i.e. weights
// 64g..64g+31 (low nibbles, sub-block 2g) and 64g+32..64g+63 (high nibbles,
// sub-block 2g+1); plus the 16-byte header.
struct RawQ4K { u4 h, qa, qb; };

__device__ __forceinline__ void load_unit(RawQ4K &r, rsrc_t rs, u32 off, int g) {
    r.h = ld16(rs, off);
    r.qa = ld16(rs, off + 16 + 32 * g);
    r.qb = ld16(rs, off + 32 + 32 * g);
}

template <int M, int R, class XA>
__device__ __forceinline__ void val_unit(const RawQ4K (&raw)[R], int g, const XA &xa, float (&v)[R][M]) {
    float dsc0[R], dsc1[R], dm0[R], dm1[R];
    const u32 sel = (u32)(2 * g) | ((u32)(2 * g + 1) << 8) | 0x0C0C0000u;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const u32 h0 = raw[r].h.x, h1 = raw[r].h.y, h2 = raw[r].h.z, h3 = raw[r].h.w;
        const float d = half_lo(h0), dmin = half_lo(h0 >> 16);
        const u32 sc_lo = h1 & 0x3F3F3F3Fu, m_lo = h2 & 0x3F3F3F3Fu;
        const u32 sc_hi = (h3 & 0x0F0F0F0Fu) | ((h1 >> 2) & 0x30303030u);
        const u32 m_hi = ((h3 >> 4) & 0x0F0F0F0Fu) | ((h2 >> 2) & 0x30303030u);
        const u32 sc = __builtin_amdgcn_perm(sc_hi, sc_lo, sel);
        const u32 mm = __builtin_amdgcn_perm(m_hi, m_lo, sel);
        dsc0[r] = d * (float)(sc & 0xFFu);
        dsc1[r] = (d * 0.0625f) * (float)((sc >> 8) & 0xFFu);
        dm0[r] = dmin * (float)(mm & 0xFFu);
        dm1[r] = dmin * (float)((mm >> 8) & 0xFFu);
    }
    float slo[R][M], shi[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) slo[r][m] = shi[r][m] = 0.f;
    // step t = (i, m) reads x[4i .. 4i+3] and x[32+4i .. 32+4i+3] of row m
    constexpr int XP = xpref<XA, M>(), NT = 8 * M;
    f4 xb[XP + 1][2];
    auto fetch = [&](int t) {
        const int i = t / M, m = t % M;
        xb[t % (XP + 1)][0] = xa.x4(m, 4 * i);
        xb[t % (XP + 1)][1] = xa.x4(m, 32 + 4 * i);
    };
#pragma unroll
    for (int t = 0; t < XP; ++t)
        if (t < NT) fetch(t);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        hf2 a[R], b[R], c[R], e[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const u32 D = i < 4 ? raw[r].qa[i & 3] : raw[r].qb[i & 3];
            const u32 D8 = D >> 8;
            a[r] = as_h2(D & 0x000F000Fu);
            b[r] = as_h2(D8 & 0x000F000Fu);
            c[r] = as_h2(D & 0x00F000F0u);
            e[r] = as_h2(D8 & 0x00F000F0u);
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int t = i * M + m;
            if (t + XP < NT) fetch(t + XP);
            const f4 cl = xb[t % (XP + 1)][0], ch = xb[t % (XP + 1)][1];
            // the 2R chains of the step advance together (independent FMAs
            // back to back); each chain keeps its own order
#pragma unroll
            for (int r = 0; r < R; ++r) {
                slo[r][m] = fmx<XA, M, false>(a[r], cl.x, slo[r][m]);
                shi[r][m] = fmx<XA, M, false>(c[r], ch.x, shi[r][m]);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                slo[r][m] = fmx<XA, M, false>(b[r], cl.y, slo[r][m]);
                shi[r][m] = fmx<XA, M, false>(e[r], ch.y, shi[r][m]);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                slo[r][m] = fmx<XA, M, true>(a[r], cl.z, slo[r][m]);
                shi[r][m] = fmx<XA, M, true>(c[r], ch.z, shi[r][m]);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                slo[r][m] = fmx<XA, M, true>(b[r], cl.w, slo[r][m]);
                shi[r][m] = fmx<XA, M, true>(e[r], ch.w, shi[r][m]);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                pin<XA, M>(slo[r][m]);
                pin<XA, M>(shi[r][m]);
            }
        }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const float s_lo = xa.sum(m, 0) + xa.sum(m, 1), s_hi = xa.sum(m, 2) + xa.sum(m, 3);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float aq = dsc0[r] * slo[r][m];
            aq = __builtin_fmaf(dsc1[r], shi[r][m], aq);
            float am = dm0[r] * s_lo;
            am = __builtin_fmaf(dm1[r], s_hi, am);
            v[r][m] = __builtin_fmaf(aq, 16777216.0f, -am);
        }
    }
}

// ---- Q6_K: unit (block b, half h, quarter q2) = the 64 weights
// 128h + 32g + 16*q2 + i (g = 0..3, i = 0..15): low bits from bytes
// 64h + 16*q2 + i (g = 0, 2) and 64h + 32 + 16*q2 + i (g = 1, 3), high bits
// from byte 128 + 32h + 16*q2 + i, scales 8h + 2g + q2.  Blocks may start
// 2 bytes off a dword: fields are read dword-aligned and realigned.
// The raw registers hold the dword-aligned loads as they arrive; the
// realignment happens at use, so a prefetch never waits for its data.
struct RawQ6K { u4 a, b, hq; u32 a4, b4, h4, s0, s1, s2, dw, sh; };

__device__ __forceinline__ void load_unit(RawQ6K &r, rsrc_t rs, u32 off, int sub) {
    const int h = sub >> 1, q2 = sub & 1;
    const u32 sh = off & 3u, base = off - sh;
    const u32 oa = base + 64 * h + 16 * q2;
    r.a = ld16(rs, oa);
    r.a4 = ld4(rs, oa + 16);
    r.b = ld16(rs, oa + 32);
    r.b4 = ld4(rs, oa + 48);
    r.hq = ld16(rs, base + 128 + 32 * h + 16 * q2);
    r.h4 = ld4(rs, base + 144 + 32 * h + 16 * q2);
    const u32 so = base + 192 + 8 * h;
    r.s0 = ld4(rs, so);
    r.s1 = ld4(rs, so + 4);
    r.s2 = ld4(rs, so + 8);
    r.dw = ld4(rs, base + 208);
    r.sh = sh;
}

struct Q6KFields { u32 a[4], b[4], hq[4], s0, s1; float d; };

__device__ __forceinline__ Q6KFields fields(const RawQ6K &r) {
    Q6KFields f;
    const u32 sh = r.sh;
    f.a[0] = realign(r.a.y, r.a.x, sh); f.a[1] = realign(r.a.z, r.a.y, sh);
    f.a[2] = realign(r.a.w, r.a.z, sh); f.a[3] = realign(r.a4, r.a.w, sh);
    f.b[0] = realign(r.b.y, r.b.x, sh); f.b[1] = realign(r.b.z, r.b.y, sh);
    f.b[2] = realign(r.b.w, r.b.z, sh); f.b[3] = realign(r.b4, r.b.w, sh);
    f.hq[0] = realign(r.hq.y, r.hq.x, sh); f.hq[1] = realign(r.hq.z, r.hq.y, sh);
    f.hq[2] = realign(r.hq.w, r.hq.z, sh); f.hq[3] = realign(r.h4, r.hq.w, sh);
    f.s0 = realign(r.s1, r.s0, sh);
    f.s1 = realign(r.s2, r.s1, sh);
    f.d = half_lo(r.dw >> (8 * sh));
    return f;
}

template <int M, int R, class XA>
__device__ __forceinline__ void val_unit(const RawQ6K (&rawu)[R], int sub, const XA &xa, float (&v)[R][M]) {
    const int q2 = sub & 1;
    Q6KFields raw[R];
#pragma unroll
    for (int r = 0; r < R; ++r) raw[r] = fields(rawu[r]);
    float dsc[R][4];
    const u32 sel = (u32)q2 | ((u32)(q2 + 2) << 8) | ((u32)(q2 + 4) << 16) | ((u32)(q2 + 6) << 24);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const u32 p = __builtin_amdgcn_perm(raw[r].s1, raw[r].s0, sel);
#pragma unroll
        for (int g = 0; g < 4; ++g) dsc[r][g] = raw[r].d * (float)(int)(signed char)(p >> (8 * g));
    }
    float acc[R][M][4];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int g = 0; g < 4; ++g) acc[r][m][g] = 0.f;
    // step t = (k, m) reads run g at x[32g + 4k .. 32g + 4k + 3] of row m
    constexpr int XP = xpref<XA, M>(), NT = 4 * M;
    f4 xb[XP + 1][4];
    auto fetch = [&](int t) {
        const int k = t / M, m = t % M;
#pragma unroll
        for (int g = 0; g < 4; ++g) xb[t % (XP + 1)][g] = xa.x4(m, 32 * g + 4 * k);
    };
#pragma unroll
    for (int t = 0; t < XP; ++t)
        if (t < NT) fetch(t);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        hf2 w[R][4][2];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const u32 A = raw[r].a[k], B = raw[r].b[k], H = raw[r].hq[k];
            const u32 A8 = A >> 8, B8 = B >> 8;
            const u32 H4l = H << 4, H4r = H >> 4, H2l = H << 2, H6r = H >> 6;
            w[r][0][0] = as_h2((A & 0x000F000Fu) | (H4l & 0x00300030u));
            w[r][0][1] = as_h2((A8 & 0x000F000Fu) | (H4r & 0x00300030u));
            w[r][1][0] = as_h2((B & 0x000F000Fu) | (H2l & 0x00300030u));
            w[r][1][1] = as_h2((B8 & 0x000F000Fu) | (H6r & 0x00300030u));
            w[r][2][0] = as_h2((A & 0x00F000F0u) | (H4l & 0x03000300u));
            w[r][2][1] = as_h2((A8 & 0x00F000F0u) | (H4r & 0x03000300u));
            w[r][3][0] = as_h2((B & 0x00F000F0u) | (H2l & 0x03000300u));
            w[r][3][1] = as_h2((B8 & 0x00F000F0u) | (H6r & 0x03000300u));
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int t = k * M + m;
            if (t + XP < NT) fetch(t + XP);
            const f4 *xv = xb[t % (XP + 1)];
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int g = 0; g < 4; ++g) acc[r][m][g] = fmx<XA, M, false>(w[r][g][0], xv[g].x, acc[r][m][g]);
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int g = 0; g < 4; ++g) acc[r][m][g] = fmx<XA, M, false>(w[r][g][1], xv[g].y, acc[r][m][g]);
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int g = 0; g < 4; ++g) acc[r][m][g] = fmx<XA, M, true>(w[r][g][0], xv[g].z, acc[r][m][g]);
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int g = 0; g < 4; ++g) acc[r][m][g] = fmx<XA, M, true>(w[r][g][1], xv[g].w, acc[r][m][g]);
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int g = 0; g < 4; ++g) pin<XA, M>(acc[r][m][g]);
        }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const float sx[4] = {xa.sum(m, 0), xa.sum(m, 1), xa.sum(m, 2), xa.sum(m, 3)};
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float aq = dsc[r][0] * acc[r][m][0];
            aq = __builtin_fmaf(dsc[r][1], acc[r][m][1], aq);
            aq = __builtin_fmaf(dsc[r][2] * 0.0625f, acc[r][m][2], aq);
            aq = __builtin_fmaf(dsc[r][3] * 0.0625f, acc[r][m][3], aq);
            float am = dsc[r][0] * sx[0];
#pragma unroll
            for (int g = 1; g < 4; ++g) am = __builtin_fmaf(dsc[r][g], sx[g], am);
            v[r][m] = __builtin_fmaf(aq, 16777216.0f, -32.0f * am);
        }
    }
}

// ---- Q2_K: unit (block b, half h, quarter q2) = the 64 weights
// 128h + 32s + 16*q2 + i (s = 0..3, i = 0..15): bits 2s..2s+1 of quant byte
// 32h + 16*q2 + i, scale/min byte 8h + 2s + q2.
struct RawQ2K { u4 q; u32 s0, s1, dd; };

__device__ __forceinline__ void load_unit(RawQ2K &r, rsrc_t rs, u32 off, int sub) {
    const int h = sub >> 1, q2 = sub & 1;
    r.q = ld16(rs, off + 16 + 32 * h + 16 * q2);
    const u4 sc = ld16(rs, off + 8 * h);   // bytes 8h .. 8h+15 (the first 8 are used)
    r.s0 = sc.x;
    r.s1 = sc.y;
    r.dd = ld4(rs, off + 80);
}

template <int M, int R, class XA>
__device__ __forceinline__ void val_unit(const RawQ2K (&raw)[R], int sub, const XA &xa, float (&v)[R][M]) {
    const int q2 = sub & 1;
    float dsc[R][4], dmm[R][4];
    const u32 sel = (u32)q2 | ((u32)(q2 + 2) << 8) | ((u32)(q2 + 4) << 16) | ((u32)(q2 + 6) << 24);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const u32 p = __builtin_amdgcn_perm(raw[r].s1, raw[r].s0, sel);
        const float d = half_lo(raw[r].dd), dmin = half_lo(raw[r].dd >> 16);
        const float dq[4] = {d, d * 0.25f, d * 0.0625f, d * 0.015625f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            dsc[r][s] = dq[s] * (float)((p >> (8 * s)) & 15u);
            dmm[r][s] = dmin * (float)((p >> (8 * s + 4)) & 15u);
        }
    }
    float acc[R][M][4];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int s = 0; s < 4; ++s) acc[r][m][s] = 0.f;
    // step t = (k, m) reads run s at x[32s + 4k .. 32s + 4k + 3] of row m
    constexpr int XP = xpref<XA, M>(), NT = 4 * M;
    f4 xb[XP + 1][4];
    auto fetch = [&](int t) {
        const int k = t / M, m = t % M;
#pragma unroll
        for (int s = 0; s < 4; ++s) xb[t % (XP + 1)][s] = xa.x4(m, 32 * s + 4 * k);
    };
#pragma unroll
    for (int t = 0; t < XP; ++t)
        if (t < NT) fetch(t);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        hf2 we[R][4], wo[R][4];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const u32 D = raw[r].q[k], D8 = D >> 8;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const u32 mask = 0x00030003u << (2 * s);
                we[r][s] = as_h2(D & mask);
                wo[r][s] = as_h2(D8 & mask);
            }
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int t = k * M + m;
            if (t + XP < NT) fetch(t + XP);
            const f4 *xv = xb[t % (XP + 1)];
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int s = 0; s < 4; ++s) acc[r][m][s] = fmx<XA, M, false>(we[r][s], xv[s].x, acc[r][m][s]);
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int s = 0; s < 4; ++s) acc[r][m][s] = fmx<XA, M, false>(wo[r][s], xv[s].y, acc[r][m][s]);
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int s = 0; s < 4; ++s) acc[r][m][s] = fmx<XA, M, true>(we[r][s], xv[s].z, acc[r][m][s]);
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int s = 0; s < 4; ++s) acc[r][m][s] = fmx<XA, M, true>(wo[r][s], xv[s].w, acc[r][m][s]);
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int s = 0; s < 4; ++s) pin<XA, M>(acc[r][m][s]);
        }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const float sx[4] = {xa.sum(m, 0), xa.sum(m, 1), xa.sum(m, 2), xa.sum(m, 3)};
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float aq = dsc[r][0] * acc[r][m][0];
            float am = dmm[r][0] * sx[0];
#pragma unroll
            for (int s = 1; s < 4; ++s) {
                aq = __builtin_fmaf(dsc[r][s], acc[r][m][s], aq);
                am = __builtin_fmaf(dmm[r][s], sx[s], am);
            }
            v[r][m] = __builtin_fmaf(aq, 16777216.0f, -am);
        }
    }
}

// ---- Q8_0: unit = one block of 32 weights; quants read as q + 128.
struct RawQ80 { u4 a, b; u32 c, dw, off; };

__device__ __forceinline__ void load_unit(RawQ80 &r, rsrc_t rs, u32 off, int) {
    const u32 qo = off + 2, qb = qo & ~3u;
    r.a = ld16(rs, qb);
    r.b = ld16(rs, qb + 16);
    r.c = ld4(rs, qb + 32);
    r.dw = ld4(rs, off & ~3u);
    r.off = off;
}

struct Q80Fields { u32 q[8]; float d; };

__device__ __forceinline__ Q80Fields fields(const RawQ80 &r) {
    Q80Fields f;
    const u32 sh = (r.off + 2) & 3u;
    f.q[0] = realign(r.a.y, r.a.x, sh); f.q[1] = realign(r.a.z, r.a.y, sh);
    f.q[2] = realign(r.a.w, r.a.z, sh); f.q[3] = realign(r.b.x, r.a.w, sh);
    f.q[4] = realign(r.b.y, r.b.x, sh); f.q[5] = realign(r.b.z, r.b.y, sh);
    f.q[6] = realign(r.b.w, r.b.z, sh); f.q[7] = realign(r.c, r.b.w, sh);
    f.d = half_lo(r.dw >> (8 * (r.off & 3u)));
    return f;
}

template <int M, int R, class XA>
__device__ __forceinline__ void val_unit(const RawQ80 (&rawu)[R], int, const XA &xa, float (&v)[R][M]) {
    Q80Fields raw[R];
#pragma unroll
    for (int r = 0; r < R; ++r) raw[r] = fields(rawu[r]);
    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.f;
    // step t = (i, m) reads x[4i .. 4i+3] of row m
    constexpr int XP = xpref<XA, M>(), NT = 8 * M;
    f4 xb[XP + 1];
    auto fetch = [&](int t) { xb[t % (XP + 1)] = xa.x4(t % M, 4 * (t / M)); };
#pragma unroll
    for (int t = 0; t < XP; ++t)
        if (t < NT) fetch(t);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        hf2 we[R], wo[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const u32 U = raw[r].q[i] ^ 0x80808080u;
            we[r] = as_h2(U & 0x00FF00FFu);
            wo[r] = as_h2((U >> 8) & 0x00FF00FFu);
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int t = i * M + m;
            if (t + XP < NT) fetch(t + XP);
            const f4 cx = xb[t % (XP + 1)];
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r][m] = fmx<XA, M, false>(we[r], cx.x, acc[r][m]);
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r][m] = fmx<XA, M, false>(wo[r], cx.y, acc[r][m]);
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r][m] = fmx<XA, M, true>(we[r], cx.z, acc[r][m]);
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r][m] = fmx<XA, M, true>(wo[r], cx.w, acc[r][m]);
#pragma unroll
            for (int r = 0; r < R; ++r) pin<XA, M>(acc[r][m]);
        }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const float sx = xa.sum(m, 0) + xa.sum(m, 1);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float aq = raw[r].d * acc[r][m];
            const float am = raw[r].d * sx;
            v[r][m] = __builtin_fmaf(aq, 16777216.0f, -128.0f * am);
        }
    }
}

// ---- Q4_0: unit = one block of 32 weights: weight i < 16 in the low nibble
// of quant byte i, weight 16 + i in its high nibble; w = d*(q - 8).  Blocks of
// 18 B may start 2 bytes off a dword.
struct RawQ40 { u4 a; u32 c, dw, off; };

__device__ __forceinline__ void load_unit(RawQ40 &r, rsrc_t rs, u32 off, int) {
    const u32 qb = (off + 2) & ~3u;
    r.a = ld16(rs, qb);
    r.c = ld4(rs, qb + 16);
    r.dw = ld4(rs, off & ~3u);
    r.off = off;
}

struct Q40Fields { u32 q[4]; float d; };

__device__ __forceinline__ Q40Fields fields(const RawQ40 &r) {
    Q40Fields f;
    const u32 sh = (r.off + 2) & 3u;
    f.q[0] = realign(r.a.y, r.a.x, sh); f.q[1] = realign(r.a.z, r.a.y, sh);
    f.q[2] = realign(r.a.w, r.a.z, sh); f.q[3] = realign(r.c, r.a.w, sh);
    f.d = half_lo(r.dw >> (8 * (r.off & 3u)));
    return f;
}

template <int M, int R, class XA>
__device__ __forceinline__ void val_unit(const RawQ40 (&rawu)[R], int, const XA &xa, float (&v)[R][M]) {
    Q40Fields raw[R];
#pragma unroll
    for (int r = 0; r < R; ++r) raw[r] = fields(rawu[r]);
    float slo[R][M], shi[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) slo[r][m] = shi[r][m] = 0.f;
    // step t = (i, m) reads x[4i .. 4i+3] and x[16+4i .. 16+4i+3] of row m
    constexpr int XP = xpref<XA, M>(), NT = 4 * M;
    f4 xb[XP + 1][2];
    auto fetch = [&](int t) {
        const int i = t / M, m = t % M;
        xb[t % (XP + 1)][0] = xa.x4(m, 4 * i);
        xb[t % (XP + 1)][1] = xa.x4(m, 16 + 4 * i);
    };
#pragma unroll
    for (int t = 0; t < XP; ++t)
        if (t < NT) fetch(t);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        hf2 a[R], b[R], c[R], e[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const u32 D = raw[r].q[i], D8 = D >> 8;
            a[r] = as_h2(D & 0x000F000Fu);
            b[r] = as_h2(D8 & 0x000F000Fu);
            c[r] = as_h2(D & 0x00F000F0u);
            e[r] = as_h2(D8 & 0x00F000F0u);
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int t = i * M + m;
            if (t + XP < NT) fetch(t + XP);
            const f4 cl = xb[t % (XP + 1)][0], ch = xb[t % (XP + 1)][1];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                slo[r][m] = fmx<XA, M, false>(a[r], cl.x, slo[r][m]);
                shi[r][m] = fmx<XA, M, false>(c[r], ch.x, shi[r][m]);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                slo[r][m] = fmx<XA, M, false>(b[r], cl.y, slo[r][m]);
                shi[r][m] = fmx<XA, M, false>(e[r], ch.y, shi[r][m]);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                slo[r][m] = fmx<XA, M, true>(a[r], cl.z, slo[r][m]);
                shi[r][m] = fmx<XA, M, true>(c[r], ch.z, shi[r][m]);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                slo[r][m] = fmx<XA, M, true>(b[r], cl.w, slo[r][m]);
                shi[r][m] = fmx<XA, M, true>(e[r], ch.w, shi[r][m]);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                pin<XA, M>(slo[r][m]);
                pin<XA, M>(shi[r][m]);
            }
        }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const float sx = xa.sum(m, 0) + xa.sum(m, 1);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float aq = raw[r].d * slo[r][m];
            aq = __builtin_fmaf(raw[r].d * 0.0625f, shi[r][m], aq);
            const float am = raw[r].d * sx;
            v[r][m] = __builtin_fmaf(aq, 16777216.0f, -8.0f * am);
        }
    }
}

// ---- Q5_K: unit (block b, group g) = weights 64g .. 64g+63 as in Q4_K; their
// low 4 bits are Q4_K's (quant bytes 48 + 32g .. 48 + 32g + 31), bit 4 of
// weight 64g + 32s + l (s = 0, 1) is bit 2g + s of high-bit byte 16 + l.
struct RawQ5K { u4 h, qa, qb, ha, hb; };

__device__ __forceinline__ void load_unit(RawQ5K &r, rsrc_t rs, u32 off, int g) {
    r.h = ld16(rs, off);
    r.qa = ld16(rs, off + 48 + 32 * g);
    r.qb = ld16(rs, off + 64 + 32 * g);
    r.ha = ld16(rs, off + 16);
    r.hb = ld16(rs, off + 32);
}

template <int M, int R, class XA>
__device__ __forceinline__ void val_unit(const RawQ5K (&raw)[R], int g, const XA &xa, float (&v)[R][M]) {
    float dsc0[R], dsc1[R], dm0[R], dm1[R];
    const u32 sel = (u32)(2 * g) | ((u32)(2 * g + 1) << 8) | 0x0C0C0000u;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const u32 h0 = raw[r].h.x, h1 = raw[r].h.y, h2 = raw[r].h.z, h3 = raw[r].h.w;
        const float d = half_lo(h0), dmin = half_lo(h0 >> 16);
        const u32 sc_lo = h1 & 0x3F3F3F3Fu, m_lo = h2 & 0x3F3F3F3Fu;
        const u32 sc_hi = (h3 & 0x0F0F0F0Fu) | ((h1 >> 2) & 0x30303030u);
        const u32 m_hi = ((h3 >> 4) & 0x0F0F0F0Fu) | ((h2 >> 2) & 0x30303030u);
        const u32 sc = __builtin_amdgcn_perm(sc_hi, sc_lo, sel);
        const u32 mm = __builtin_amdgcn_perm(m_hi, m_lo, sel);
        dsc0[r] = d * (float)(sc & 0xFFu);
        dsc1[r] = (d * 0.0625f) * (float)((sc >> 8) & 0xFFu);
        dm0[r] = dmin * (float)(mm & 0xFFu);
        dm1[r] = dmin * (float)((mm >> 8) & 0xFFu);
    }
    float slo[R][M], shi[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) slo[r][m] = shi[r][m] = 0.f;
    constexpr int XP = xpref<XA, M>(), NT = 8 * M;
    f4 xb[XP + 1][2];
    auto fetch = [&](int t) {
        const int i = t / M, m = t % M;
        xb[t % (XP + 1)][0] = xa.x4(m, 4 * i);
        xb[t % (XP + 1)][1] = xa.x4(m, 32 + 4 * i);
    };
#pragma unroll
    for (int t = 0; t < XP; ++t)
        if (t < NT) fetch(t);
    const u32 s0 = 2 * g, s1 = 2 * g + 1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        hf2 a[R], b[R], c[R], e[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const u32 D = i < 4 ? raw[r].qa[i & 3] : raw[r].qb[i & 3];
            const u32 H = i < 4 ? raw[r].ha[i & 3] : raw[r].hb[i & 3];
            const u32 D8 = D >> 8, hl = H >> s0, hh = H >> s1;
            a[r] = as_h2((D & 0x000F000Fu) | ((hl << 4) & 0x00100010u));
            b[r] = as_h2((D8 & 0x000F000Fu) | ((hl >> 4) & 0x00100010u));
            c[r] = as_h2((D & 0x00F000F0u) | ((hh << 8) & 0x01000100u));
            e[r] = as_h2((D8 & 0x00F000F0u) | (hh & 0x01000100u));
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int t = i * M + m;
            if (t + XP < NT) fetch(t + XP);
            const f4 cl = xb[t % (XP + 1)][0], ch = xb[t % (XP + 1)][1];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                slo[r][m] = fmx<XA, M, false>(a[r], cl.x, slo[r][m]);
                shi[r][m] = fmx<XA, M, false>(c[r], ch.x, shi[r][m]);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                slo[r][m] = fmx<XA, M, false>(b[r], cl.y, slo[r][m]);
                shi[r][m] = fmx<XA, M, false>(e[r], ch.y, shi[r][m]);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                slo[r][m] = fmx<XA, M, true>(a[r], cl.z, slo[r][m]);
                shi[r][m] = fmx<XA, M, true>(c[r], ch.z, shi[r][m]);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                slo[r][m] = fmx<XA, M, true>(b[r], cl.w, slo[r][m]);
                shi[r][m] = fmx<XA, M, true>(e[r], ch.w, shi[r][m]);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                pin<XA, M>(slo[r][m]);
                pin<XA, M>(shi[r][m]);
            }
        }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const float s_lo = xa.sum(m, 0) + xa.sum(m, 1), s_hi = xa.sum(m, 2) + xa.sum(m, 3);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float aq = dsc0[r] * slo[r][m];
            aq = __builtin_fmaf(dsc1[r], shi[r][m], aq);
            float am = dm0[r] * s_lo;
            am = __builtin_fmaf(dm1[r], s_hi, am);
            v[r][m] = __builtin_fmaf(aq, 16777216.0f, -am);
        }
    }
}

// ---- Q3_K: unit (block b, half h, quarter q2) = the 64 weights
// 128h + 32s + 16*q2 + i (s = 0..3, i = 0..15): two low bits from bits
// 2s..2s+1 of byte 32 + 32h + 16*q2 + i, the mask bit (set: +4) is bit 4h + s of
// byte 16*q2 + i, scale 8h + 2s + q2 (6 bits, used as sc - 32); the value
// used is q + 4 in 0..7, the -4 folded into the activation sums.  Blocks of
// 110 B may start 2 bytes off a dword: fields are read dword-aligned and
// realigned at use.
struct RawQ3K { u4 q, mk, s; u32 q4, m4, sh; };

__device__ __forceinline__ void load_unit(RawQ3K &r, rsrc_t rs, u32 off, int sub) {
    const int h = sub >> 1, q2 = sub & 1;
    const u32 sh = off & 3u, base = off - sh;
    r.q = ld16(rs, base + 32 + 32 * h + 16 * q2);
    r.q4 = ld4(rs, base + 48 + 32 * h + 16 * q2);
    r.mk = ld16(rs, base + 16 * q2);
    r.m4 = ld4(rs, base + 16 + 16 * q2);
    r.s = ld16(rs, base + 96);       // scales (12 B) and d, for sh <= 2
    r.sh = sh;
}

struct Q3KFields { u32 q[4], mk[4], s0, s1, s2; float d; };

__device__ __forceinline__ Q3KFields fields(const RawQ3K &r) {
    Q3KFields f;
    const u32 sh = r.sh;
    f.q[0] = realign(r.q.y, r.q.x, sh); f.q[1] = realign(r.q.z, r.q.y, sh);
    f.q[2] = realign(r.q.w, r.q.z, sh); f.q[3] = realign(r.q4, r.q.w, sh);
    f.mk[0] = realign(r.mk.y, r.mk.x, sh); f.mk[1] = realign(r.mk.z, r.mk.y, sh);
    f.mk[2] = realign(r.mk.w, r.mk.z, sh); f.mk[3] = realign(r.m4, r.mk.w, sh);
    f.s0 = realign(r.s.y, r.s.x, sh);
    f.s1 = realign(r.s.z, r.s.y, sh);
    f.s2 = realign(r.s.w, r.s.z, sh);
    f.d = half_lo(r.s.w >> (8 * sh));
    return f;
}

// The unit's four scales minus 32, as d * (sc - 32): scale 8h + 2s + q2 has
// its low 4 bits in byte 2s + q2 (low nibble for h = 0, high for h = 1) and its
// top 2 bits at bit 4h + 2*(s/2) of byte 8 + (2s + q2) % 4.
__device__ __forceinline__ void q3k_scales(const Q3KFields &f, int sub, float (&dsc)[4]) {
    const int h = sub >> 1, q2 = sub & 1;
    const u32 sel = (u32)q2 | ((u32)(q2 + 2) << 8) | ((u32)(q2 + 4) << 16) | ((u32)(q2 + 6) << 24);
    const u32 lo = (__builtin_amdgcn_perm(f.s1, f.s0, sel) >> (4 * h)) & 0x0F0F0F0Fu;
    const u32 tsel = (u32)q2 | ((u32)(q2 + 2) << 8) | ((u32)q2 << 16) | ((u32)(q2 + 2) << 24);
    const u32 t = __builtin_amdgcn_perm(f.s2, f.s2, tsel) >> (4 * h);
    const u32 top = ((t & 0x0000FFFFu) | ((t >> 2) & 0xFFFF0000u)) & 0x03030303u;
    const u32 sc = lo | (top << 4);
#pragma unroll
    for (int s = 0; s < 4; ++s) dsc[s] = f.d * (float)((int)((sc >> (8 * s)) & 0xFFu) - 32);
}

template <int M, int R, class XA>
__device__ __forceinline__ void val_unit(const RawQ3K (&rawu)[R], int sub, const XA &xa, float (&v)[R][M]) {
    const int h = sub >> 1;
    Q3KFields raw[R];
    float dsc[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        raw[r] = fields(rawu[r]);
        q3k_scales(raw[r], sub, dsc[r]);
    }
    float acc[R][M][4];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int s = 0; s < 4; ++s) acc[r][m][s] = 0.f;
    constexpr int XP = xpref<XA, M>(), NT = 4 * M;
    f4 xb[XP + 1][4];
    auto fetch = [&](int t) {
        const int k = t / M, m = t % M;
#pragma unroll
        for (int s = 0; s < 4; ++s) xb[t % (XP + 1)][s] = xa.x4(m, 32 * s + 4 * k);
    };
#pragma unroll
    for (int t = 0; t < XP; ++t)
        if (t < NT) fetch(t);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        hf2 we[R][4], wo[R][4];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const u32 Q = raw[r].q[k], Q8 = Q >> 8;
            const u32 H = raw[r].mk[k] >> (4 * h), H8 = H >> 8;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                we[r][s] = as_h2(((Q >> (2 * s)) & 0x00030003u) | (((H >> s) << 2) & 0x00040004u));
                wo[r][s] = as_h2(((Q8 >> (2 * s)) & 0x00030003u) | (((H8 >> s) << 2) & 0x00040004u));
            }
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int t = k * M + m;
            if (t + XP < NT) fetch(t + XP);
            const f4 *xv = xb[t % (XP + 1)];
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int s = 0; s < 4; ++s) acc[r][m][s] = fmx<XA, M, false>(we[r][s], xv[s].x, acc[r][m][s]);
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int s = 0; s < 4; ++s) acc[r][m][s] = fmx<XA, M, false>(wo[r][s], xv[s].y, acc[r][m][s]);
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int s = 0; s < 4; ++s) acc[r][m][s] = fmx<XA, M, true>(we[r][s], xv[s].z, acc[r][m][s]);
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int s = 0; s < 4; ++s) acc[r][m][s] = fmx<XA, M, true>(wo[r][s], xv[s].w, acc[r][m][s]);
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int s = 0; s < 4; ++s) pin<XA, M>(acc[r][m][s]);
        }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const float sx[4] = {xa.sum(m, 0), xa.sum(m, 1), xa.sum(m, 2), xa.sum(m, 3)};
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float aq = dsc[r][0] * acc[r][m][0];
            float am = dsc[r][0] * sx[0];
#pragma unroll
            for (int s = 1; s < 4; ++s) {
                aq = __builtin_fmaf(dsc[r][s], acc[r][m][s], aq);
                am = __builtin_fmaf(dsc[r][s], sx[s], am);
            }
            v[r][m] = __builtin_fmaf(aq, 16777216.0f, -4.0f * am);
        }
    }
}

template <int T> struct RawOf;
template <> struct RawOf<T_Q4_K> { typedef RawQ4K type; };
template <> struct RawOf<T_Q6_K> { typedef RawQ6K type; };
template <> struct RawOf<T_Q2_K> { typedef RawQ2K type; };
template <> struct RawOf<T_Q8_0> { typedef RawQ80 type; };
template <> struct RawOf<T_Q4_0> { typedef RawQ40 type; };
template <> struct RawOf<T_Q5_K> { typedef RawQ5K type; };
template <> struct RawOf<T_Q3_K> { typedef RawQ3K type; };

// First weight (within its row) of unit u, and the spacing of its 16-sums.
template <int T> __device__ __forceinline__ int unit_e0(int u) {
    typedef Fmt<T> F;
    const int b = u / F::UPB, sub = u - b * F::UPB;
    if constexpr (T == T_Q4_K || T == T_Q5_K) return b * 256 + 64 * sub;
    else if constexpr (Fmt<T>::QK == 32) return b * 32;
    else return b * 256 + 128 * (sub >> 1) + 16 * (sub & 1);
}
template <int T> constexpr int sum_run_stride() { return (T == T_Q6_K || T == T_Q2_K || T == T_Q3_K) ? 2 : 1; }

// ---------------------------------------------------------------------------
// Row-sum structure shared by every kernel.  Units are numbered along the row;
// "stripe" i is units [i*LPR, (i+1)*LPR) with unit i*LPR + l on lane l of a
// lane group.  A row's result is
//     y = ((0 + S_0) + S_1) + ... ,   S_i = group_sum over the stripe's lanes
// of the per-unit values v, with a fixed binary tree (lanes paired by bit 0,
// then bit 1, ... ).  Any kernel that follows it gives the same bits.

// ---------------------------------------------------------------------------
// Activation staging for the LDS kernels: rows xr[0..M) of the chunk
// [c0, c0 + kc) go to LDS with 16 B of padding every 64 floats, and
// ss[m][j] = sum16 of x[c0 + 16j .. +16).  kc is a multiple of 32.

template <int M>
__device__ __forceinline__ void stage_x(float *xs, float *ss, int XS, int SS, const float *const (&xr)[M],
                                        int c0, int kc, int nthreads) {
    const int n16 = kc >> 4;
    for (int idx = threadIdx.x; idx < M * n16; idx += nthreads) {
        const int m = idx / n16, j = idx - m * n16;
        const f4 *src = reinterpret_cast<const f4 *>(xr[m] + c0 + 16 * j);
        const f4 v0 = src[0], v1 = src[1], v2 = src[2], v3 = src[3];
        float *dst = xs + m * XS + xpad(16 * j);
        reinterpret_cast<f4 *>(dst)[0] = v0;
        reinterpret_cast<f4 *>(dst)[1] = v1;
        reinterpret_cast<f4 *>(dst)[2] = v2;
        reinterpret_cast<f4 *>(dst)[3] = v3;
        ss[m * SS + j] = sum16(v0, v1, v2, v3);
    }
}

// LDS row strides (multiples of 4 floats, so every row starts 16-B aligned)
// and the LDS floats needed for M rows and a chunk of kc columns.
__host__ __device__ constexpr int x_stride(int kc) { return (kc + (kc >> 4) + 3) & ~3; }
__host__ __device__ constexpr int s_stride(int kc) { return ((kc >> 4) + 3) & ~3; }
__host__ __device__ constexpr int lds_floats(int M, int kc) { return M * (x_stride(kc) + s_stride(kc)); }

// ---------------------------------------------------------------------------
// LDS kernel body (any M; used for M >= 2, for the routed experts and for very
// long rows).  One work-group of WG_THREADS computes `nrows` rows starting at
// `row0` of one matrix for M activation rows xr[] and writes yr[m][row].
// Each lane group of LPR lanes owns R rows; activations are staged per K chunk.

template <int T, int M, int R>
__device__ __forceinline__ void gemv_tile(float *smem, const uint8_t *W, int64_t row_bytes, int row0, int nrows,
                                          int K, int KC, int lpr, const float *const (&xr)[M],
                                          float *const (&yr)[M]) {
    typedef Fmt<T> F;
    typedef typename RawOf<T>::type Raw;
    const int G = 64 / lpr;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int grp = lane / lpr, slot = lane - grp * lpr;
    const int rfirst = (wave * G + grp) * R;     // first tile-relative row of this group

    const uintptr_t ta = (uintptr_t)(W + (int64_t)row0 * row_bytes);
    const u32 delta = (u32)(ta & 3u);
    const rsrc_t rs = make_rsrc((const void *)(ta - delta), delta + (u32)((int64_t)nrows * row_bytes));
    u32 roff[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int rr = rfirst + r;
        roff[r] = rr < nrows ? delta + (u32)((int64_t)rr * row_bytes) : OOB;
    }

    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.f;

    const int kcmax = KC < K ? KC : K;
    const int XS = x_stride(kcmax);
    const int SS = s_stride(kcmax);
    float *xs = smem;
    float *ss = smem + M * XS;

    for (int c0 = 0; c0 < K; c0 += KC) {
        const int kc = (K - c0) < KC ? (K - c0) : KC;
        if (c0) __syncthreads();
        stage_x<M>(xs, ss, XS, SS, xr, c0, kc, WG_THREADS);
        __syncthreads();
        const int units = (kc / F::QK) * F::UPB;
        const int ub = (c0 / F::QK) * F::UPB;       // units before this chunk
        const int nstripes = (units + lpr - 1) / lpr;
        for (int i = 0; i < nstripes; ++i) {
            const int ul = slot + lpr * i;
            const bool act = ul < units;
            const int uc = act ? ul : 0;
            const int bl = uc / F::UPB, sub = uc - bl * F::UPB;
            const u32 boff = (u32)((ub + uc) / F::UPB) * F::BYTES;
            Raw raw[R];
#pragma unroll
            for (int r = 0; r < R; ++r) load_unit(raw[r], rs, act ? roff[r] + boff : OOB, sub);
            const int e0 = unit_e0<T>(uc);
            const XLds xa{xs, ss, XS, SS, xpad(e0), e0 >> 4, sum_run_stride<T>()};
            float v[R][M];
            val_unit<M, R>(raw, sub, xa, v);
            (void)bl;
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < M; ++m) acc[r][m] += group_sum(act ? v[r][m] : 0.f, lpr);
        }
    }

#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int rr = rfirst + r;
            if (slot == 0 && rr < nrows) yr[m][row0 + rr] = acc[r][m];
        }
}

// ---------------------------------------------------------------------------
// Kernels

template <int T, int M, int R>
__global__ __launch_bounds__(WG_THREADS) void qgemv_kernel(const uint8_t *__restrict__ W, int64_t row_bytes,
                                                           int N, int K, int KC, int lpr,
                                                           const float *__restrict__ x, float *__restrict__ y) {
    extern __shared__ float smem[];
    const int rows_per_wg = WAVES * (64 / lpr) * R;
    const int row0 = blockIdx.x * rows_per_wg;
    const int nrows = (N - row0) < rows_per_wg ? (N - row0) : rows_per_wg;
    const float *xr[M];
    float *yr[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        xr[m] = x + (int64_t)m * K;
        yr[m] = y + (int64_t)m * N;
    }
    gemv_tile<T, M, R>(smem, W, row_bytes, row0, nrows, K, KC, lpr, xr, yr);
}

// Batch-1 kernel.  The row is cut into stripes of 64 units (fewer than 64:
// one stripe of LPR lanes, 64 / LPR rows per wave); a work-group holds RS
// row slots x NS stripes of waves (at most 16 waves), one work-group per
// compute unit, persistent.  The work-group stages the activations and their
// 16-sums once in LDS; every wave then copies the slice its lanes need into
// registers, so the activations cross L2 once per compute unit.  Row slot rs
// of work-group b takes the row steps b*RS + rs, + grid*RS, ... (interleaved,
// every work-group gets the same share).  Each wave keeps the loads of the
// next D steps in flight in a ring of registers; the loop body is
// straight-line: a step's stripe sum is parked in one lane (lane = step mod
// LPR) and every LPR steps the parked sums are flushed -- stored directly when
// the row is one stripe, otherwise added across stripes in stripe order
// through LDS.

// Several matrices with the same format and K that read the same
// activations can be served by one launch: their rows are numbered one after
// another, segment s holding rows [start[s], start[s] + rows[s]).  Starts are
// multiples of the rows one step covers (G), so a step never spans two
// segments; the numbers between a segment's last row and the next start are
// padding that loads and stores nothing.
constexpr int MAX_SEGS = 8;
struct Segs {
    const uint8_t *W[MAX_SEGS];
    float *y[MAX_SEGS];
    int start[MAX_SEGS + 1];
    int rows[MAX_SEGS];
    int n;
};

template <bool MS> __device__ __forceinline__ int seg_of(const Segs &sg, int row) {
    if (!MS) return 0;
    int s = 0;
#pragma unroll
    for (int i = 1; i < MAX_SEGS; ++i) s += (i < sg.n && row >= sg.start[i]) ? 1 : 0;
    return s;
}

// The segment of the rows a wave loads.  A wave's row steps mostly move
// forward, so the cursor keeps the current segment's fields and compares the
// row with the next segment's start; the fields of another segment are read
// only when the row leaves the current one.  (Reading them through a computed
// index at every step puts two dependent scalar-memory loads and their waits
// in front of each step's weight loads.)  `row` is uniform over the wave.
template <bool MS> struct SegCursor {
    const uint8_t *W;
    int s, start, rows, next;
    __device__ __forceinline__ void set(const Segs &sg, int i) {
        s = i;
        W = sg.W[i];
        start = sg.start[i];
        rows = sg.rows[i];
        next = (MS && i + 1 < sg.n) ? sg.start[i + 1] : 0x7fffffff;
    }
    __device__ __forceinline__ void seek(const Segs &sg, int row) {
        if (!MS) return;
        if ((unsigned)(row - start) >= (unsigned)(next - start)) set(sg, seg_of<MS>(sg, row));
    }
};

// Output slot of a row, or NULL for a padding row or a row past the end.
// (m: the activation row; a segment's outputs are [M][rows])
template <bool MS> __device__ __forceinline__ float *out_of(const Segs &sg, int N, int row, int m = 0) {
    if (row >= N) return nullptr;
    const int s = seg_of<MS>(sg, row);
    const int local = row - sg.start[s];
    return local < sg.rows[s] ? sg.y[s] + (int64_t)m * sg.rows[s] + local : nullptr;
}

// Registers <- LDS for one unit's activations (same values as XReg::load).
template <int T>
__device__ __forceinline__ void xreg_from_lds(XReg<T> &xr, const XLds &xa) {
#pragma unroll
    for (int r = 0; r < XReg<T>::NS; ++r) {
#pragma unroll
        for (int k = 0; k < 4; ++k) xr.v[4 * r + k] = xa.x4(0, (XReg<T>::RUNS32 ? 32 : 16) * r + 4 * k);
        xr.s[r] = xa.sum(0, r);
    }
}

// Write the parked sums of steps [b0, b0 + LPR): one stripe -- store; several
// stripes -- add them in stripe order through LDS (barriers: every wave of the
// work-group calls this at the same steps).
// Work-group barrier.  With buffer-to-LDS loads in flight (DMA) it waits only
// for the wave's own LDS accesses: __syncthreads would also wait for every
// outstanding buffer-to-LDS load (the compiler cannot tell that only the
// issuing wave reads their destination) and drain the weight ring.
template <bool DMA> __device__ __forceinline__ void wg_sync() {
    if constexpr (DMA)
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
        __syncthreads();
}

template <bool MS, bool DMA = false>
__device__ __forceinline__ void flush1(float keep, int b0, int wsteps, int first, int rstride, int N, int ns,
                                       int wave, int lane, int rsl, int stripe, int grp, int slot,
                                       float (*part)[64], const Segs &sg, int m = 0) {
    if (ns > 1) {
        part[wave][lane] = keep;
        wg_sync<DMA>();
        float *o = out_of<MS>(sg, N, first + (b0 + lane) * rstride, m);
        if (stripe == 0 && b0 + lane < wsteps && o) {
            float s = 0.f;
            for (int w = 0; w < ns; ++w) s += part[rsl * ns + w][lane];
            *o = s;
        }
        wg_sync<DMA>();
    } else {
        float *o = out_of<MS>(sg, N, first + (b0 + slot) * rstride + grp, m);
        if (b0 + slot < wsteps && o) *o = 0.f + keep;
    }
}

// One batch-1 pass over a set of segments of one format (rows of one or more
// matrices with the same K) on activations already staged in LDS.  Each wave
// owns one stripe of one row slot: its lane's unit never changes, so the
// unit's activations are read from LDS into registers once, and every step
// only streams weights.
template <int T, int D, bool MS, int LP = 0> struct B1Pass {
    typedef Fmt<T> F;
    typedef typename RawOf<T>::type Raw;
    const Segs &sg;
    int64_t row_bytes;
    int N, lpr, ns, wave, lane, rsl, stripe, G, grp, slot, sub, rstride, first, wsteps, uc;
    bool act;
    u32 boff;
    SegCursor<MS> cur;
    Raw ring[D][1];
    int irow;              // first row of the next step to issue
    const uint8_t *iptr;   // its bytes (valid while irow is in the cursor's segment)
    int64_t sbytes;        // bytes between a row slot's consecutive steps
    // lanes per row: LP when fixed at compile time (64: rows of >= 64 units)
    __device__ __forceinline__ int lp() const { return LP ? LP : lpr; }

    // wg / nwg: this work-group's index among the nwg that share the rows
    __device__ __forceinline__ B1Pass(const Segs &s, int64_t rb, int K, int lpr_, int ns_, int wave_, int lane_,
                                      int wg, int nwg)
        : sg(s), row_bytes(rb), lpr(lpr_), ns(ns_), wave(wave_), lane(lane_) {
        N = sg.start[sg.n];
        const int RS = (blockDim.x >> 6) / ns;          // row slots
        rsl = wave / ns;
        stripe = wave - rsl * ns;
        G = 64 / lpr;
        grp = lane / lpr;
        slot = lane - grp * lpr;
        const int units = (K / F::QK) * F::UPB;
        const int u = stripe * 64 + slot;
        act = u < units;
        uc = act ? u : 0;
        sub = uc % F::UPB;
        boff = (u32)(uc / F::UPB) * F::BYTES;
        rstride = nwg * RS * G;
        first = (wg * RS + rsl) * G;
        // steps of the work-group's first row slot; every row slot runs this
        // many (uniform trip count: the loop has barriers), later slots may
        // run past N on empty buffers and store nothing
        const int f0 = wg * RS * G;
        wsteps = f0 < N ? (N - f0 + rstride - 1) / rstride : 0;
        cur.set(sg, 0);
        irow = first;
        iptr = cur.W + (int64_t)first * rb;
        sbytes = (int64_t)rstride * rb;
    }
    // the loads of the wave's next row step (rows irow .. irow + G - 1, one per
    // lane group; steps are issued in order, so the step's address is carried
    // forward).  Never conditional: a step past the last row gets an empty
    // buffer (its loads return zeros), so the loads of every ring slot stay
    // in flight in program order.
    __device__ __forceinline__ void issue(int d) {
        const int row0 = irow;
        if constexpr (MS) {
            if ((unsigned)(row0 - cur.start) >= (unsigned)(cur.next - cur.start)) {
                cur.set(sg, seg_of<MS>(sg, row0));
                iptr = cur.W + (int64_t)(row0 - cur.start) * row_bytes;
            }
        }
        const int local = row0 - cur.start;
        const int left = cur.rows - local;
        const int nr = row0 >= N || left <= 0 ? 0 : (left < G ? left : G);
        const uintptr_t ta = (uintptr_t)(nr ? iptr : cur.W);
        const u32 delta = (u32)(ta & 3u);
        const rsrc_t rs = make_rsrc((const void *)(ta - delta), nr ? delta + (u32)((int64_t)nr * row_bytes) : 0u);
        load_unit(ring[d][0], rs, (act && grp < nr) ? delta + (u32)((int64_t)grp * row_bytes) + boff : OOB, sub);
        irow = row0 + rstride;
        iptr += sbytes;
    }
    __device__ __forceinline__ void issue_first() {
#pragma unroll
        for (int d = 0; d < D; ++d) issue(d);
    }
    __device__ __forceinline__ void flush(float keep, int b0, float (*part)[64]) {
        flush1<MS>(keep, b0, wsteps, first, rstride, N, ns, wave, lane, rsl, stripe, grp, slot, part, sg);
    }
    // the loads of the first D steps must have been issued (issue_first)
    __device__ __forceinline__ void run(const float *xs, const float *ss, int XS, int SS, float (*part)[64]) {
        XReg<T> xa;
        {
            const int e0 = unit_e0<T>(uc);
            const XLds xl{xs, ss, XS, SS, xpad(e0), e0 >> 4, sum_run_stride<T>()};
            xreg_from_lds<T>(xa, xl);
        }
        float keep = 0.f;
        int j = 0;
        for (; j + D <= wsteps; j += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                float v[1][1];
                val_unit<1, 1>(ring[d], sub, xa, v);
                issue(d);
                const float S = group_sum(act ? v[0][0] : 0.f, lp());
                keep = (slot == ((j + d) & (lp() - 1))) ? S : keep;
            }
            if (((j + D) & (lp() - 1)) == 0) flush(keep, j + D - lp(), part);
            // keep the waves of the work-group in step: otherwise the oldest
            // waves race ahead and the work-group ends on a few slow waves
            // with too few loads in flight
            __syncthreads();
        }
#pragma unroll
        for (int d = 0; d < D - 1; ++d) {
            if (j + d < wsteps) {
                float v[1][1];
                val_unit<1, 1>(ring[d], sub, xa, v);
                const float S = group_sum(act ? v[0][0] : 0.f, lp());
                keep = (slot == ((j + d) & (lp() - 1))) ? S : keep;
            }
        }
        if (wsteps & (lp() - 1)) flush(keep, wsteps & ~(lp() - 1), part);
    }
};

// Activation staging of the batch-1 kernels in two halves: x1_load issues the
// activation loads (at most two groups of 16 per thread) as the kernel's first
// memory accesses, so that they wait only for the kernel arguments they use;
// the kernel then sets up its row pass and issues the first row loads, and
// x1_store writes the activations and their 16-sums to LDS -- waiting for the
// activations leaves the row loads in flight.
struct X1 {
    f4 g[2][4];
};
__device__ __forceinline__ X1 x1_load(const float *__restrict__ x, int K, int nthreads) {
    const int n16 = K >> 4;
    X1 r;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int idx = threadIdx.x + it * nthreads;
        const f4 *src = reinterpret_cast<const f4 *>(x + 16 * (idx < n16 ? idx : 0));
#pragma unroll
        for (int k = 0; k < 4; ++k) r.g[it][k] = src[k];
    }
    return r;
}
template <bool DMA>
__device__ __forceinline__ void x1_store(const X1 &r, int K, int nthreads, float *smem, float *xs, float *ss) {
    const int n16 = K >> 4;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        // unconditional, so the loads are not sunk below the row loads:
        // threads without a group write into the (not yet used) flush area
        const int idx = threadIdx.x + it * nthreads;
        const bool ok = idx < n16;
        f4 *dst = reinterpret_cast<f4 *>(ok ? xs + xpad(16 * idx) : smem);
#pragma unroll
        for (int k = 0; k < 4; ++k) dst[k] = r.g[it][k];
        (ok ? ss[idx] : smem[16]) = sum16(r.g[it][0], r.g[it][1], r.g[it][2], r.g[it][3]);
    }
    wg_sync<DMA>();
}

// Batch-1 kernel: one persistent work-group per compute unit, RS row slots of
// ns stripe waves.  LDS: [16][64] flush area, then the staged activations.
template <int T, int D, int LB, bool MS, int LP>
__global__ __launch_bounds__(LB) void qgemv1_kernel(const float *__restrict__ x, int K, int nthreads, const Segs sg,
                                                    int64_t row_bytes, int lpr, int ns) {
    extern __shared__ float smem[];
    float (*part)[64] = reinterpret_cast<float (*)[64]>(smem);
    float *xs = smem + 16 * 64;
    const int XS = x_stride(K), SS = s_stride(K);
    float *ss = xs + XS;
    // wave index as a scalar: everything derived from it (the row of a step and
    // the buffer descriptor of its loads) stays in SGPRs
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    // the activation loads before the pass is set up: they wait only for the
    // kernel arguments they use, not for the pass's segment lookups
    const X1 xr = x1_load(x, K, nthreads);
    __builtin_amdgcn_sched_barrier(0);
    B1Pass<T, D, MS, LP> p(sg, row_bytes, K, lpr, ns, wave, lane, blockIdx.x, gridDim.x);
    p.issue_first();
    __builtin_amdgcn_sched_barrier(0);
    x1_store<false>(xr, K, nthreads, smem, xs, ss);
    p.run(xs, ss, XS, SS, part);
}

// Batch-1 pass with the weight ring in LDS (used for Q4_K).  A wave's row step
// covers 64 units: at most 16 blocks (Q4_K: 2304 contiguous bytes, one stripe
// of a long row or G whole short rows).  The wave copies them with NLD
// buffer-to-LDS loads of 16 bytes per lane (lane i: bytes 1024k + 16i), each
// covering whole 128-byte lines, so they can bypass the caches (non-temporal)
// without a line being fetched twice; each lane then reads its unit's header
// and quant bytes from LDS.  Compared with the register ring of B1Pass this
// frees the ring's registers, and every load instruction is a single
// coalesced 1-KB request.  The compiler does not order LDS reads after these
// loads, so the waits are explicit: before reading slot d a wave lets at most
// NLD(D-1) loads stay outstanding (those of the D-1 later steps; loads
// complete in issue order, and a store issued in between only makes the wait
// stricter), and its reads of a slot complete before the slot is refilled.
// Requires 16-byte aligned matrices and rows.
#define KQ_LDS __attribute__((address_space(3)))

template <int N> __device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int T> struct DmaGeom {
    static constexpr int SPAN = 16 * Fmt<T>::BYTES;          // bytes of 64 units
    static constexpr int NLD = (SPAN + 1023) / 1024;         // 1-KB loads per step
    static constexpr int SLOT = NLD * 1024;                  // bytes per ring slot
};

__device__ __forceinline__ void read_unit(RawQ4K &r, const char *blk, int g) {
    r.h = *reinterpret_cast<const u4 *>(blk);
    r.qa = *reinterpret_cast<const u4 *>(blk + 16 + 32 * g);
    r.qb = *reinterpret_cast<const u4 *>(blk + 32 + 32 * g);
}
// M activation rows held in registers, one XReg each (the LDS-ring pass at
// M = 2: with the weight ring in LDS two rows' activations fit the registers
// of an 8-wave work-group).
template <int T, int M> struct XRegM {
    static constexpr bool FENCE = false;
    XReg<T> r[M];
    __device__ __forceinline__ f4 x4(int m, int off) const { return r[m].x4(0, off); }
    __device__ __forceinline__ float sum(int m, int run) const { return r[m].sum(0, run); }
};

template <int T, int D, bool MS, int M = 1, int LP = 0> struct B1Dma {
    typedef Fmt<T> F;
    typedef DmaGeom<T> GM;
    typedef typename RawOf<T>::type Raw;
    const Segs &sg;
    int64_t row_bytes;
    int N, lpr, ns, wave, lane, rsl, stripe, G, grp, slot, sub, rstride, first, wsteps, uc;
    bool act;
    u32 rbase, span, lofs;
    char *ring;   // this wave's D slots
    SegCursor<MS> cur;
    int irow;              // first row of the next step to issue
    const uint8_t *iptr;   // its bytes (valid while irow is in the cursor's segment)
    int64_t sbytes;        // bytes between a row slot's consecutive steps
    // lanes per row: LP when fixed at compile time (64: rows of >= 64 units)
    __device__ __forceinline__ int lp() const { return LP ? LP : lpr; }

    __device__ __forceinline__ B1Dma(const Segs &s, int64_t rb, int K, int lpr_, int ns_, int wave_, int lane_, int wg,
                                     int nwg, char *ring_)
        : sg(s), row_bytes(rb), lpr(lpr_), ns(ns_), wave(wave_), lane(lane_), ring(ring_) {
        N = sg.start[sg.n];
        const int RS = (blockDim.x >> 6) / ns;
        rsl = wave / ns;
        stripe = wave - rsl * ns;
        G = 64 / lpr;
        grp = lane / lpr;
        slot = lane - grp * lpr;
        const int units = (K / F::QK) * F::UPB;
        const int u = stripe * 64 + slot;
        act = u < units;
        uc = act ? u : 0;
        sub = uc % F::UPB;
        rstride = nwg * RS * G;
        first = (wg * RS + rsl) * G;
        const int f0 = wg * RS * G;
        wsteps = f0 < N ? (N - f0 + rstride - 1) / rstride : 0;
        rbase = (u32)stripe * GM::SPAN;
        const int64_t rest = rb - (int64_t)rbase;
        span = ns > 1 ? (u32)(rest < GM::SPAN ? rest : GM::SPAN) : (u32)(G * rb);
        // a lane's block inside the slot (inactive lanes stay inside the slot)
        lofs = (u32)(grp * (ns > 1 ? 0 : rb)) + (u32)(slot / F::UPB) * F::BYTES;
        cur.set(sg, 0);
        irow = first;
        iptr = cur.W + (int64_t)first * rb;
        sbytes = (int64_t)rstride * rb;
    }
    // the loads of the wave's next row step (steps are issued in order)
    __device__ __forceinline__ void issue(int d) {
        const int row0 = irow;
        if constexpr (MS) {
            if ((unsigned)(row0 - cur.start) >= (unsigned)(cur.next - cur.start)) {
                cur.set(sg, seg_of<MS>(sg, row0));
                iptr = cur.W + (int64_t)(row0 - cur.start) * row_bytes;
            }
        }
        const int local = row0 - cur.start;
        const int left = cur.rows - local;
        const int nr = row0 >= N || left <= 0 ? 0 : (left < G ? left : G);
        const rsrc_t rs = make_rsrc(nr ? iptr : cur.W, (u32)((int64_t)nr * row_bytes));
        irow = row0 + rstride;
        iptr += sbytes;
        char *dst = ring + d * GM::SLOT;
#pragma unroll
        for (int k = 0; k < GM::NLD; ++k) {
            const u32 o = 1024u * k + 16u * lane;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (KQ_LDS void *)(dst + 1024 * k), 16, o < span ? rbase + o : OOB,
                                                     0, 0, 2 /* nt */);
        }
    }
    __device__ __forceinline__ void issue_first() {
#pragma unroll
        for (int d = 0; d < D; ++d) issue(d);
    }
    __device__ __forceinline__ void flush(const float (&keep)[M], int b0, float (*part)[64]) {
#pragma unroll
        for (int m = 0; m < M; ++m)
            flush1<MS, true>(keep[m], b0, wsteps, first, rstride, N, ns, wave, lane, rsl, stripe, grp, slot, part, sg,
                             m);
    }
    // park the step's row sums (one per activation row) in lane `step mod lpr`
    template <class XA> __device__ __forceinline__ void value(const Raw &r, const XA &xa, int step, float (&keep)[M]) const {
        const Raw rr[1] = {r};
        float v[1][M];
        val_unit<M, 1>(rr, sub, xa, v);
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const float S = group_sum(act ? v[0][m] : 0.f, lp());
            keep[m] = (slot == (step & (lp() - 1))) ? S : keep[m];
        }
    }
    // activations of the lane's unit from the staged copy in LDS
    __device__ __forceinline__ void x_from_lds(XReg<T> &xa, const float *xs, const float *ss, int XS, int SS) const {
        const int e0 = unit_e0<T>(uc);
        const XLds xl{xs, ss, XS, SS, xpad(e0), e0 >> 4, sum_run_stride<T>()};
        xreg_from_lds<T>(xa, xl);
    }
    // the loads of the first D steps must have been issued (issue_first)
    template <class XA> __device__ __forceinline__ void run(const XA &xa, float (*part)[64]) {
        float keep[M];
#pragma unroll
        for (int m = 0; m < M; ++m) keep[m] = 0.f;
        int j = 0;
        for (; j + D <= wsteps; j += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                Raw r;
                wait_vm<GM::NLD * (D - 1)>();
                read_unit(r, ring + d * GM::SLOT + lofs, sub);
                wait_lgkm0();
                issue(d);
                value(r, xa, j + d, keep);
            }
            if (((j + D) & (lp() - 1)) == 0) flush(keep, j + D - lp(), part);
            wg_sync<true>();
        }
        wait_vm<0>();
#pragma unroll
        for (int d = 0; d < D - 1; ++d) {
            if (j + d < wsteps) {
                Raw r;
                read_unit(r, ring + d * GM::SLOT + lofs, sub);
                value(r, xa, j + d, keep);
            }
        }
        if (wsteps & (lp() - 1)) flush(keep, wsteps & ~(lp() - 1), part);
    }
};

// LDS of the batch-1 kernels: [16][64] flush area, the staged activations and
// 16-sums, then (ring in LDS) the weight ring, 16-byte aligned.
__host__ __device__ constexpr size_t b1_ring_offset(int K, int M = 1) {
    return ((size_t)(16 * 64 + M * (x_stride(K) + s_stride(K))) * sizeof(float) + 15) & ~(size_t)15;
}

template <int T, int D, int LB, bool MS, int LP>
__global__ __launch_bounds__(LB) void qgemv1_dma_kernel(const float *__restrict__ x, int K, int nthreads,
                                                        const Segs sg, int64_t row_bytes, int lpr, int ns) {
    extern __shared__ float smem[];
    float (*part)[64] = reinterpret_cast<float (*)[64]>(smem);
    float *xs = smem + 16 * 64;
    const int XS = x_stride(K), SS = s_stride(K);
    float *ss = xs + XS;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    char *ring = reinterpret_cast<char *>(smem) + b1_ring_offset(K) + (size_t)wave * D * DmaGeom<T>::SLOT;
    // the activation loads before the pass is set up (as in qgemv1_kernel)
    const X1 xr = x1_load(x, K, nthreads);
    __builtin_amdgcn_sched_barrier(0);
    B1Dma<T, D, MS, 1, LP> p(sg, row_bytes, K, lpr, ns, wave, lane, blockIdx.x, gridDim.x, ring);
    p.issue_first();
    __builtin_amdgcn_sched_barrier(0);
    x1_store<true>(xr, K, nthreads, smem, xs, ss);
    XReg<T> xa;
    p.x_from_lds(xa, xs, ss, XS, SS);
    p.run(xa, part);
}

// x1_load / x1_store for M activation rows (row m at xs + m * (XS + SS), its
// 16-sums right after it), for the M-row LDS-ring kernel.
template <int M> struct XM {
    f4 g[M][2][4];
};
template <int M> __device__ __forceinline__ XM<M> xm_load(const float *__restrict__ x, int K, int nthreads) {
    const int n16 = K >> 4;
    XM<M> r;
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int idx = threadIdx.x + it * nthreads;
            const f4 *src = reinterpret_cast<const f4 *>(x + (int64_t)m * K + 16 * (idx < n16 ? idx : 0));
#pragma unroll
            for (int k = 0; k < 4; ++k) r.g[m][it][k] = src[k];
        }
    return r;
}
template <int M>
__device__ __forceinline__ void xm_store(const XM<M> &r, int K, int nthreads, float *smem, float *xs, int XS, int SS) {
    const int n16 = K >> 4;
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int idx = threadIdx.x + it * nthreads;
            const bool ok = idx < n16;
            float *xm = xs + m * (XS + SS);
            f4 *dst = reinterpret_cast<f4 *>(ok ? xm + xpad(16 * idx) : smem);
#pragma unroll
            for (int k = 0; k < 4; ++k) dst[k] = r.g[m][it][k];
            (ok ? xm[XS + idx] : smem[16]) = sum16(r.g[m][it][0], r.g[m][it][1], r.g[m][it][2], r.g[m][it][3]);
        }
    wg_sync<true>();
}

// The LDS-ring kernel at M > 1 (used for Q4_K at M = 2): 8 waves, both
// activation rows in registers, the same per-row sums as at M = 1.
template <int T, int D, int LB, bool MS, int M, int LP>
__global__ __launch_bounds__(LB) void qgemv1m_dma_kernel(const float *__restrict__ x, int K, int nthreads,
                                                         const Segs sg, int64_t row_bytes, int lpr, int ns) {
    extern __shared__ float smem[];
    float (*part)[64] = reinterpret_cast<float (*)[64]>(smem);
    float *xs = smem + 16 * 64;
    const int XS = x_stride(K), SS = s_stride(K);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    char *ring = reinterpret_cast<char *>(smem) + b1_ring_offset(K, M) + (size_t)wave * D * DmaGeom<T>::SLOT;
    // the activation loads first, then the pass and its first row loads (as
    // in qgemv1_dma_kernel)
    const XM<M> xr = xm_load<M>(x, K, nthreads);
    __builtin_amdgcn_sched_barrier(0);
    B1Dma<T, D, MS, M, LP> p(sg, row_bytes, K, lpr, ns, wave, lane, blockIdx.x, gridDim.x, ring);
    p.issue_first();
    __builtin_amdgcn_sched_barrier(0);
    xm_store<M>(xr, K, nthreads, smem, xs, XS, SS);
    XRegM<T, M> xa;
#pragma unroll
    for (int m = 0; m < M; ++m) p.x_from_lds(xa.r[m], xs + m * (XS + SS), xs + m * (XS + SS) + XS, XS, SS);
    p.run(xa, part);
}

// One side of a mixed launch: this work-group's share of the rows of one
// format (Q4_K through the LDS ring when DMA is set).
template <int T, int D, bool DMA, int LP>
__device__ __forceinline__ void b1_side(const Segs &sg, int64_t rb, int K, int lpr, int ns, int wave, int lane, int wg,
                                        int nwg, const X1 &xr, int nthreads, float *smem) {
    float (*part)[64] = reinterpret_cast<float (*)[64]>(smem);
    float *xs = smem + 16 * 64;
    const int XS = x_stride(K), SS = s_stride(K);
    float *ss = xs + XS;
    if constexpr (DMA && T == T_Q4_K) {
        char *ring = reinterpret_cast<char *>(smem) + b1_ring_offset(K) + (size_t)wave * D * DmaGeom<T>::SLOT;
        B1Dma<T, D, true, 1, LP> p(sg, rb, K, lpr, ns, wave, lane, wg, nwg, ring);
        p.issue_first();
        __builtin_amdgcn_sched_barrier(0);
        x1_store<true>(xr, K, nthreads, smem, xs, ss);
        XReg<T> xa;
        p.x_from_lds(xa, xs, ss, XS, SS);
        p.run(xa, part);
    } else {
        B1Pass<T, D, true, LP> p(sg, rb, K, lpr, ns, wave, lane, wg, nwg);
        p.issue_first();
        __builtin_amdgcn_sched_barrier(0);
        x1_store<false>(xr, K, nthreads, smem, xs, ss);
        p.run(xs, ss, XS, SS, part);
    }
}

template <int TA, int DA, int TB, int DB, int LB, bool DMA, int LP>
__global__ __launch_bounds__(LB) void qgemv1_mixed_kernel(const float *__restrict__ x, int K, int nthreads,
                                                           const Segs sa, int64_t rba, const Segs sb, int64_t rbb,
                                                           int gb, int lpr, int ns) {
    extern __shared__ float smem[];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    // both sides stage the same activations: load them before either side
    // sets up its pass
    const X1 xr = x1_load(x, K, nthreads);
    __builtin_amdgcn_sched_barrier(0);
    if ((int)blockIdx.x < gb)
        b1_side<TB, DB, DMA, LP>(sb, rbb, K, lpr, ns, wave, lane, blockIdx.x, gb, xr, nthreads, smem);
    else
        b1_side<TA, DA, DMA, LP>(sa, rba, K, lpr, ns, wave, lane, blockIdx.x - gb, gridDim.x - gb, xr, nthreads, smem);
}

// Small grouped launches at M = 1 (the non-persistent counterpart of the
// grouped and mixed batch-1 kernels): one 4-wave work-group per row tile of
// one matrix, the tiles of the TB matrices first, then those of the TA
// matrices (TA may equal TB); each tile runs the LDS kernel body.  tiles[s]
// is the first tile of segment s (tiles[n] the total), computed on the host;
// the segment of a tile is found with compares and selects on the kernel
// arguments at fixed offsets (no dependent loads before the weight loads).
struct SegTiles {
    int t[MAX_SEGS + 1];
};
template <int T>
__device__ __forceinline__ void seg_tile(float *smem, const Segs &sg, const SegTiles &st, int64_t row_bytes, int tile,
                                         int rows_per_wg, int K, int lpr, const float *x) {
    const uint8_t *W = sg.W[0];
    float *y = sg.y[0];
    int rows = sg.rows[0], t0 = 0;
#pragma unroll
    for (int i = 1; i < MAX_SEGS; ++i) {
        const bool in = i < sg.n && tile >= st.t[i];
        W = in ? sg.W[i] : W;
        y = in ? sg.y[i] : y;
        rows = in ? sg.rows[i] : rows;
        t0 = in ? st.t[i] : t0;
    }
    const int row0 = (tile - t0) * rows_per_wg;
    const int nrows = (rows - row0) < rows_per_wg ? (rows - row0) : rows_per_wg;
    // settle the tile's matrix here, before the activations are staged: left
    // to itself the compiler reads these arguments only after the staging
    // barrier, in front of the first weight loads
    asm volatile("" ::"s"(W), "s"(y), "s"(row0), "s"(nrows), "s"(row_bytes));
    const float *xr[1] = {x};
    float *yr[1] = {y};
    gemv_tile<T, 1, 1>(smem, W, row_bytes, row0, nrows, K, K, lpr, xr, yr);
}

template <int TA, int TB>
__global__ __launch_bounds__(WG_THREADS) void qgemv_seg_kernel(const Segs sa, const SegTiles ta, int64_t rba,
                                                               const Segs sb, const SegTiles tb, int64_t rbb,
                                                               int tiles_b, int rows_per_wg, int K, int lpr,
                                                               const float *__restrict__ x) {
    extern __shared__ float smem[];
    if constexpr (TA == TB) {
        // one format: every tile is in sb (sa is empty)
        seg_tile<TB>(smem, sb, tb, rbb, blockIdx.x, rows_per_wg, K, lpr, x);
    } else {
        if ((int)blockIdx.x < tiles_b)
            seg_tile<TB>(smem, sb, tb, rbb, blockIdx.x, rows_per_wg, K, lpr, x);
        else
            seg_tile<TA>(smem, sa, ta, rba, blockIdx.x - tiles_b, rows_per_wg, K, lpr, x);
    }
}

// Batch-M kernel (2 <= M <= 8).  Persistent work-groups of NW waves, one per
// compute unit.  Rows are dealt out in row steps of RG = R * G rows (G lane
// groups of LPR lanes per wave, R rows per group, so one read of a unit's
// activations from LDS serves R rows).  The activations of M rows are staged
// per K chunk (a multiple of 4096 columns, so stripes never straddle chunks);
// for each chunk a wave walks its row steps and, within a step, the chunk's
// stripes in order.  The running row sums live in LDS across chunks and take
// the stripe sums in ascending order, so every output gets the M = 1 bits.
// The weight loads run D items ahead through a register ring that does not
// stop at chunk boundaries (the loads do not depend on the activations).
template <bool MS> __device__ __forceinline__ float *out_m(const Segs &sg, int N, int row, int m) {
    if (row >= N) return nullptr;
    const int s = seg_of<MS>(sg, row);
    const int local = row - sg.start[s];
    return local < sg.rows[s] ? sg.y[s] + (int64_t)m * sg.rows[s] + local : nullptr;
}

template <int T, int R, bool MS>
__device__ __forceinline__ void issue_rows(typename RawOf<T>::type (&raw)[R], SegCursor<MS> &cur, const Segs &sg,
                                           int64_t row_bytes, int N, int RG, int row0, bool live, int grp, bool act,
                                           u32 boff, int sub) {
    cur.seek(sg, row0);
    const int local = row0 - cur.start;
    const int left = cur.rows - local;
    const int nr = (!live || row0 >= N || left <= 0) ? 0 : (left < RG ? left : RG);
    const uintptr_t ta = (uintptr_t)(cur.W + (int64_t)(nr ? local : 0) * row_bytes);
    const u32 delta = (u32)(ta & 3u);
    const rsrc_t rs = make_rsrc((const void *)(ta - delta), nr ? delta + (u32)((int64_t)nr * row_bytes) : 0u);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int rr = grp * R + r;
        load_unit(raw[r], rs, (act && rr < nr) ? delta + (u32)((int64_t)rr * row_bytes) + boff : OOB, sub);
    }
}

template <int T, int M, int R, int D, bool MS>
__global__ __launch_bounds__(512) void qgemvm_kernel(const Segs sg, int64_t row_bytes, int K, int KC, int lpr,
                                                     const float *__restrict__ x) {
    typedef Fmt<T> F;
    typedef typename RawOf<T>::type Raw;
    const int N = sg.start[sg.n];
    extern __shared__ float smem[];
    const int NW = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int G = 64 / lpr, grp = lane / lpr, slot = lane - grp * lpr;
    const int RG = R * G;
    const int XS = x_stride(KC), SS = s_stride(KC);
    float *xs = smem, *ss = smem + M * XS, *accl = ss + M * SS;
    const int nsteps = (N + RG - 1) / RG;
    const int per_round = gridDim.x * NW;
    const int f0 = blockIdx.x * NW;
    const int wsteps = f0 < nsteps ? (nsteps - f0 + per_round - 1) / per_round : 0;
    if (wsteps == 0) return;                       // uniform over the work-group
    const int nchunks = (K + KC - 1) / KC;
    const int ub_chunk = (KC / F::QK) * F::UPB;    // units per full chunk
    const int units_last = ((K - (nchunks - 1) * KC) / F::QK) * F::UPB;
    const int ns_full = (ub_chunk + lpr - 1) / lpr, ns_last = (units_last + lpr - 1) / lpr;
    const int total = wsteps * (ns_full * (nchunks - 1) + ns_last);
    const int sub = slot % F::UPB;
    const int accn = wsteps * NW * RG * M;
    for (int i = threadIdx.x; i < accn; i += blockDim.x) accl[i] = 0.f;
    const float *xr[M];
#pragma unroll
    for (int m = 0; m < M; ++m) xr[m] = x + (int64_t)m * K;

    // item cursors (chunk c, row step j, stripe s): one for issue, one for use
    int ic = 0, ij = 0, is = 0, ins = nchunks > 1 ? ns_full : ns_last;
    int cc = 0, cj = 0, cs = 0, cns = ins;
    auto step = [&](int &c, int &j, int &st, int &ns) {
        if (++st == ns) {
            st = 0;
            if (++j == wsteps) {
                j = 0;
                ++c;
                ns = c < nchunks - 1 ? ns_full : ns_last;
            }
        }
    };
    SegCursor<MS> cur;
    cur.set(sg, 0);
    auto issue = [&](Raw (&raw)[R], int c, int j, int st) {
        const int ul = st * lpr + slot;
        const int uc_n = c < nchunks - 1 ? ub_chunk : units_last;
        const bool act = ul < uc_n;
        const int ug = c * ub_chunk + (act ? ul : 0);
        const u32 boff = (u32)(ug / F::UPB) * F::BYTES;
        const int row0 = ((j * gridDim.x + blockIdx.x) * NW + wave) * RG;
        issue_rows<T, R, MS>(raw, cur, sg, row_bytes, N, RG, row0, c < nchunks, grp, act, boff, sub);
    };

    Raw ring[D][R];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        issue(ring[d], ic, ij, is);
        step(ic, ij, is, ins);
    }

    // row sums: each lane carries the running sum of index idx = r * M + m
    // (the butterfly's output slot), for rows grp * R + r of the step
    constexpr int RM = R * M, NV = RM <= 4 ? 4 : (RM <= 8 ? 8 : 16);
    static_assert(RM <= 16, "butterfly row sums hold at most 16 values");
    const int idx = scatter_idx<NV>(lane);
    float t = 0.f;
    auto use = [&](const Raw (&raw)[R]) {
        if (cj == 0 && cs == 0) {                  // first item of chunk cc: stage its activations
            if (cc) __syncthreads();
            const int kc = cc < nchunks - 1 ? KC : K - cc * KC;
            stage_x<M>(xs, ss, XS, SS, xr, cc * KC, kc, blockDim.x);
            __syncthreads();
        }
        float *acc = accl + ((cj * NW + wave) * RG + grp * R) * M;
        if (cs == 0) t = idx < RM ? acc[idx] : 0.f;
        const int ul = cs * lpr + slot;
        const bool act = ul < (cc < nchunks - 1 ? ub_chunk : units_last);
        const int e0 = unit_e0<T>(act ? ul : 0);
        const XLds xa{xs, ss, XS, SS, xpad(e0), e0 >> 4, sum_run_stride<T>()};
        float v[R][M], g[NV];
        val_unit<M, R>(raw, sub, xa, v);
#pragma unroll
        for (int i = 0; i < NV; ++i) g[i] = (i < RM && act) ? v[i / M][i % M] : 0.f;
        float S;
        if constexpr (NV <= 8) {
            // up to 8 values: plain sums side by side (measured faster than
            // the butterfly there), then this lane's index
            group_sum_n<NV>(g, lpr);
            S = g[0];
#pragma unroll
            for (int i = 1; i < NV; ++i) S = idx == i ? g[i] : S;
        } else {
            S = reduce_scatter<NV>(g, lane, lpr);
        }
        t = t + S;
        if (cs == cns - 1 && idx < RM) acc[idx] = t;   // lanes holding one index store the same value
        step(cc, cj, cs, cns);
    };

    int it = 0;
    for (; it + D <= total; it += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            use(ring[d]);
            issue(ring[d], ic, ij, is);
            step(ic, ij, is, ins);
        }
    }
#pragma unroll
    for (int d = 0; d < D - 1; ++d)
        if (it + d < total) use(ring[d]);

    __syncthreads();
    for (int i = threadIdx.x; i < accn; i += blockDim.x) {
        const int m = i % M, rest = i / M;
        const int tt = rest % RG, q = rest / RG;
        const int w = q % NW, j = q / NW;
        float *o = out_m<MS>(sg, N, ((j * gridDim.x + blockIdx.x) * NW + w) * RG + tt, m);
        if (o) *o = accl[i];
    }
}

// Expert tensors of one routed-expert launch: tensors of one format, shape,
// routing and activations (an MoE layer's gate and up projections), each with
// its per-slot outputs.
constexpr int MOE_SETS = 4;
struct MoeSet {
    const uint8_t *W[MOE_SETS];
    float *y[MOE_SETS];
    int n;
};

// Rows per lane group of the routed-expert kernel: one activation read from
// LDS serves that many rows.  Two rows for the formats with large units and
// for one-token calls, four otherwise (measured).
template <int T, int MAXM> constexpr int MOE_ROWS() { return (BIG_UNIT<T>() || MAXM == 1) ? 2 : 4; }

// Routed experts: work-group (row tile, slot s).  Only the lowest slot that
// routes to an expert does the work; it collects every slot that routes to the
// same expert and serves them in batches of up to MAXM activation rows with one
// pass over the expert's weights per batch.  Invalid ids: zero output, flag.
template <int T, int M, int R>
__device__ __forceinline__ void moe_batch(float *smem, const uint8_t *We, int64_t row_bytes, int row0, int nrows,
                                          int K, int KC, int lpr, const int *members, int x_mode, int k,
                                          const float *x, float *y, int N) {
    const float *xr[M];
    float *yr[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const int s = members[m];
        xr[m] = x + (int64_t)(x_mode ? s : s / k) * K;
        yr[m] = y + (int64_t)s * N;
    }
    gemv_tile<T, M, R>(smem, We, row_bytes, row0, nrows, K, KC, lpr, xr, yr);
}

template <int T, int MAXM>
__global__ __launch_bounds__(WG_THREADS) void qmoe_kernel(const MoeSet set, int64_t row_bytes, int E, int N, int K,
                                                          int KC, int lpr, const int32_t *__restrict__ ids,
                                                          int nslots, int k, const float *__restrict__ x,
                                                          int x_mode, int32_t *err_flag) {
    extern __shared__ float smem[];
    __shared__ int members[128];
    __shared__ unsigned long long match[2];
    // grid.y: (expert tensor, slot)
    const int ti = blockIdx.y / nslots, s = blockIdx.y - ti * nslots;
    const uint8_t *__restrict__ W = set.W[ti];
    float *__restrict__ y = set.y[ti];
    constexpr int R = MOE_ROWS<T, MAXM>();
    const int rows_per_wg = WAVES * (64 / lpr) * R;
    const int row0 = blockIdx.x * rows_per_wg;
    const int nrows = (N - row0) < rows_per_wg ? (N - row0) : rows_per_wg;
    const int e = ids[s];
    if (e < 0 || e >= E) {
        for (int i = threadIdx.x; i < nrows; i += WG_THREADS) y[(int64_t)s * N + row0 + i] = 0.f;
        if (err_flag && threadIdx.x == 0 && blockIdx.x == 0) *err_flag = 1;
        return;
    }
    int n = 0;
    if (nslots <= 16) {
        // few slots: a scan of the ids
        for (int t = 0; t < s; ++t)
            if (ids[t] == e) return;           // a lower slot serves this expert
        for (int t = s; t < nslots; ++t)
            if (ids[t] == e) {
                if (threadIdx.x == 0) members[n] = t;
                ++n;
            }
    } else {
        // thread t < nslots (<= 128: the first two waves) compares slot t's
        // id: a lower slot with the same expert serves it; otherwise the
        // matching slots, in ascending order, are the members
        const int tid = threadIdx.x, lane = tid & 63;
        const bool same = tid < nslots && ids[tid] == e;
        if (__syncthreads_or(same && tid < s)) return;     // uniform
        const unsigned long long bal = __ballot(same);
        if (tid < 128 && lane == 0) match[tid >> 6] = bal;
        __syncthreads();
        const unsigned long long below = tid >= 64 ? match[0] : 0ull;
        const int rank = __popcll(below) + __popcll(bal & ((1ull << lane) - 1ull));
        if (same) members[rank] = tid;
        n = __popcll(match[0]) + __popcll(match[1]);
    }
    __syncthreads();
    const uint8_t *We = W + (int64_t)e * N * row_bytes;
    for (int b0 = 0; b0 < n; b0 += MAXM) {
        const int mb = (n - b0) < MAXM ? (n - b0) : MAXM;
        if (b0) __syncthreads();
        switch (mb) {
#define KQ_MOE_CASE(MM) \
    case MM: if constexpr (MM <= MAXM) moe_batch<T, MM, R>(smem, We, row_bytes, row0, nrows, K, KC, lpr, members + b0, x_mode, k, x, y, N); break;
            KQ_MOE_CASE(1) KQ_MOE_CASE(2) KQ_MOE_CASE(3) KQ_MOE_CASE(4)
            KQ_MOE_CASE(5) KQ_MOE_CASE(6) KQ_MOE_CASE(7) KQ_MOE_CASE(8)
#undef KQ_MOE_CASE
        default: break;
        }
    }
}

// Routed experts, token-major: work-group (row tile, token t, expert tensor);
// wave w serves slots w, w + MOEC_WAVES, ... of token t over the tile's rows,
// each row summed in the canonical order.  Per-slot outputs (rw NULL) are
// stored as they are; otherwise they go to LDS and
// y[t][row] = sum_j rw[t][j] * s_j[row], ascending j, one fma per term from
// +0 -- the arithmetic of the separate combine, so the bits are the same.
// An expert routed to several tokens is read once per token (the slot-major
// kernel reads it once per batch of 8), which the full-width grid and, for
// the sum, the saved launch repay.  Invalid ids: the slot gives zero and sets
// the flag.
constexpr int MOEC_WAVES = 8;
constexpr int MOEC_R = 1;          // rows per lane group per step (1: measured best, few VGPRs)
template <int T>
__global__ __launch_bounds__(64 * MOEC_WAVES) void qmoe_tok_kernel(
    const float *__restrict__ x, const int32_t *__restrict__ ids, int K, int k, int x_mode, int T_, const MoeSet set,
    int64_t row_bytes, int E, int N, int lpr, int RT, const float *__restrict__ rw, int32_t *err_flag) {
    // (the arguments the first loads need come first: they are preloaded into
    // SGPRs, so the expert ids and activations are requested at once)
    typedef Fmt<T> F;
    typedef typename RawOf<T>::type Raw;
    extern __shared__ float smem[];
    const int ti = blockIdx.y / T_, t = blockIdx.y - ti * T_;
    const uint8_t *__restrict__ W = set.W[ti];
    float *__restrict__ y = set.y[ti];
    const int row0 = blockIdx.x * RT;
    const int nrows = (N - row0) < RT ? (N - row0) : RT;
    const int XS = x_stride(K), SS = s_stride(K);
    const int nx = x_mode ? k : 1;                 // activation rows staged
    float *xs = smem, *ss = smem + nx * XS, *res = ss + nx * SS;
    // the expert of the wave's first slot, read before the staging so that
    // its latency overlaps the activations' (a vector load: a scalar one
    // would be waited for with the kernel arguments, before the staging)
    const int wave0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const u32 e_first = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(ids, (u32)(T_ * k) * 4u),
                                                             wave0 < k ? (u32)(t * k + wave0) * 4u : OOB, 0, 0);
    {
        const int n16 = K >> 4;
        for (int idx = threadIdx.x; idx < nx * n16; idx += 64 * MOEC_WAVES) {
            const int m = idx / n16, j = idx - m * n16;
            const f4 *src = reinterpret_cast<const f4 *>(x + (int64_t)(x_mode ? t * k + m : t) * K + 16 * j);
            const f4 v0 = src[0], v1 = src[1], v2 = src[2], v3 = src[3];
            f4 *dst = reinterpret_cast<f4 *>(xs + m * XS + xpad(16 * j));
            dst[0] = v0;
            dst[1] = v1;
            dst[2] = v2;
            dst[3] = v3;
            ss[m * SS + j] = sum16(v0, v1, v2, v3);
        }
    }
    __syncthreads();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int G = 64 / lpr, grp = lane / lpr, slot = lane - grp * lpr;
    const int units = (K / F::QK) * F::UPB;
    const int nstripes = (units + lpr - 1) / lpr;
    for (int j = wave; j < k; j += MOEC_WAVES) {
        // slot j's results: LDS for the sum, else its output row
        float *out = rw ? res + j * RT : y + ((int64_t)t * k + j) * N + row0;
        const int e = j == wave ? (int)__builtin_amdgcn_readfirstlane(e_first) : ids[t * k + j];
        if (e < 0 || e >= E) {                     // uniform over the wave
            for (int i = lane; i < nrows; i += 64) out[i] = 0.f;
            if (err_flag && lane == 0) *err_flag = 1;
            continue;
        }
        const float *xj = xs + (x_mode ? j : 0) * XS, *sj = ss + (x_mode ? j : 0) * SS;
        const uintptr_t ta = (uintptr_t)(W + ((int64_t)e * N + row0) * row_bytes);
        const u32 delta = (u32)(ta & 3u);
        const rsrc_t rs = make_rsrc((const void *)(ta - delta), delta + (u32)((int64_t)nrows * row_bytes));
        for (int r0 = 0; r0 < nrows; r0 += G * MOEC_R) {
            u32 roff[MOEC_R];
            float acc[MOEC_R];
#pragma unroll
            for (int r = 0; r < MOEC_R; ++r) {
                const int rr = r0 + grp * MOEC_R + r;
                roff[r] = rr < nrows ? delta + (u32)((int64_t)rr * row_bytes) : OOB;
                acc[r] = 0.f;
            }
            for (int i = 0; i < nstripes; ++i) {
                const int ul = slot + lpr * i;
                const bool act = ul < units;
                const int uc = act ? ul : 0;
                const int sub = uc % F::UPB;
                const u32 boff = (u32)(uc / F::UPB) * F::BYTES;
                Raw raw[MOEC_R];
#pragma unroll
                for (int r = 0; r < MOEC_R; ++r) load_unit(raw[r], rs, act ? roff[r] + boff : OOB, sub);
                const int e0 = unit_e0<T>(uc);
                const XLds xa{xj, sj, XS, SS, xpad(e0), e0 >> 4, sum_run_stride<T>()};
                float v[MOEC_R][1];
                val_unit<1, MOEC_R>(raw, sub, xa, v);
#pragma unroll
                for (int r = 0; r < MOEC_R; ++r) acc[r] += group_sum(act ? v[r][0] : 0.f, lpr);
            }
#pragma unroll
            for (int r = 0; r < MOEC_R; ++r) {
                const int rr = r0 + grp * MOEC_R + r;
                if (slot == 0 && rr < nrows) out[rr] = acc[r];
            }
        }
    }
    if (!rw) return;                               // uniform
    __syncthreads();
    for (int i = threadIdx.x; i < nrows; i += blockDim.x) {
        float a = 0.f;
        for (int j = 0; j < k; ++j) a = __builtin_fmaf(rw[t * k + j], res[j * RT + i], a);
        y[(int64_t)t * N + row0 + i] = a;
    }
}

// ---------------------------------------------------------------------------
// Standalone dequantization, one unit per thread.  Each weight is the exact
// product(s) with a single rounding at the subtraction; + 0.0f maps -0 to +0.

template <int T>
__global__ __launch_bounds__(WG_THREADS) void dequant_kernel(const uint8_t *__restrict__ src, int64_t nunits,
                                                             float *__restrict__ dst) {
    typedef Fmt<T> F;
    const int64_t ufirst = (int64_t)blockIdx.x * WG_THREADS;
    const int64_t u = ufirst + threadIdx.x;
    const int64_t bfirst = ufirst / F::UPB;
    const int64_t blast = (ufirst + WG_THREADS + F::UPB - 1) / F::UPB;
    const int64_t nblocks = nunits / F::UPB;
    const int64_t bend = blast < nblocks ? blast : nblocks;
    const uintptr_t ta = (uintptr_t)(src + bfirst * F::BYTES);
    const u32 delta = (u32)(ta & 3u);
    const rsrc_t rs = make_rsrc((const void *)(ta - delta), delta + (u32)((bend - bfirst) * F::BYTES));
    // each wave's 64 units are a contiguous run of 64 * UW outputs: they are
    // written to LDS first and stored from there with contiguous 16-B lanes
    // (a lane's own unit would be 64 separate cache lines per store)
    constexpr int UW = F::QK / F::UPB;              // weights per unit
    __shared__ f4 win4[WG_THREADS / 64][16 * UW];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t u0 = ufirst + 64 * wave;
    if (u0 >= nunits) return;                        // uniform over the wave
    float *win = reinterpret_cast<float *>(win4[wave]);
    if (u < nunits) {
        const int64_t b = u / F::UPB;
        const int sub = (int)(u - b * F::UPB);
        const u32 off = delta + (u32)((b - bfirst) * F::BYTES);
        float *out = win + (b * F::QK - u0 * UW);
        if constexpr (T == T_Q4_K) {
            RawQ4K r;
            load_unit(r, rs, off, sub);
            const u32 h0 = r.h.x, h1 = r.h.y, h2 = r.h.z, h3 = r.h.w;
            const float d = half_lo(h0), dmin = half_lo(h0 >> 16);
            const u32 sc_lo = h1 & 0x3F3F3F3Fu, m_lo = h2 & 0x3F3F3F3Fu;
            const u32 sc_hi = (h3 & 0x0F0F0F0Fu) | ((h1 >> 2) & 0x30303030u);
            const u32 m_hi = ((h3 >> 4) & 0x0F0F0F0Fu) | ((h2 >> 2) & 0x30303030u);
            const u32 sel = (u32)(2 * sub) | ((u32)(2 * sub + 1) << 8) | 0x0C0C0000u;
            const u32 sc = __builtin_amdgcn_perm(sc_hi, sc_lo, sel), mm = __builtin_amdgcn_perm(m_hi, m_lo, sel);
            const float ds0 = d * (float)(sc & 0xFFu), ds1 = d * (float)((sc >> 8) & 0xFFu);
            const float dm0 = dmin * (float)(mm & 0xFFu), dm1 = dmin * (float)((mm >> 8) & 0xFFu);
            float lo[32], hi[32];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const u32 D = i < 4 ? r.qa[i & 3] : r.qb[i & 3];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const u32 byte = (D >> (8 * j)) & 0xFFu;
                    lo[4 * i + j] = __builtin_fmaf(ds0, (float)(byte & 15u), -dm0) + 0.0f;
                    hi[4 * i + j] = __builtin_fmaf(ds1, (float)(byte >> 4), -dm1) + 0.0f;
                }
            }
            f4 *o4 = reinterpret_cast<f4 *>(out + 64 * sub);
#pragma unroll
            for (int i = 0; i < 8; ++i) o4[i] = f4{lo[4 * i], lo[4 * i + 1], lo[4 * i + 2], lo[4 * i + 3]};
#pragma unroll
            for (int i = 0; i < 8; ++i) o4[8 + i] = f4{hi[4 * i], hi[4 * i + 1], hi[4 * i + 2], hi[4 * i + 3]};
        } else if constexpr (T == T_Q6_K) {
            const int h = sub >> 1, q2 = sub & 1;
            RawQ6K ru;
            load_unit(ru, rs, off, sub);
            const Q6KFields r = fields(ru);
            const u32 sel = (u32)q2 | ((u32)(q2 + 2) << 8) | ((u32)(q2 + 4) << 16) | ((u32)(q2 + 6) << 24);
            const u32 p = __builtin_amdgcn_perm(r.s1, r.s0, sel);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float dsc = r.d * (float)(int)(signed char)(p >> (8 * g));
                float w[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const u32 lowb = (g & 1) ? r.b[i >> 2] : r.a[i >> 2];
                    const u32 byte = (lowb >> (8 * (i & 3))) & 0xFFu;
                    const u32 lo4 = (g < 2) ? (byte & 15u) : (byte >> 4);
                    const u32 hi2 = (r.hq[i >> 2] >> (8 * (i & 3) + 2 * g)) & 3u;
                    w[i] = dsc * (float)((int)(lo4 | (hi2 << 4)) - 32) + 0.0f;
                }
                f4 *o4 = reinterpret_cast<f4 *>(out + 128 * h + 32 * g + 16 * q2);
#pragma unroll
                for (int i = 0; i < 4; ++i) o4[i] = f4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
            }
        } else if constexpr (T == T_Q2_K) {
            const int h = sub >> 1, q2 = sub & 1;
            RawQ2K r;
            load_unit(r, rs, off, sub);
            const u32 sel = (u32)q2 | ((u32)(q2 + 2) << 8) | ((u32)(q2 + 4) << 16) | ((u32)(q2 + 6) << 24);
            const u32 p = __builtin_amdgcn_perm(r.s1, r.s0, sel);
            const float d = half_lo(r.dd), dmin = half_lo(r.dd >> 16);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float dsc = d * (float)((p >> (8 * s)) & 15u);
                const float dm = dmin * (float)((p >> (8 * s + 4)) & 15u);
                float w[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const u32 q = (r.q[i >> 2] >> (8 * (i & 3) + 2 * s)) & 3u;
                    w[i] = __builtin_fmaf(dsc, (float)q, -dm) + 0.0f;
                }
                f4 *o4 = reinterpret_cast<f4 *>(out + 128 * h + 32 * s + 16 * q2);
#pragma unroll
                for (int i = 0; i < 4; ++i) o4[i] = f4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
            }
        } else if constexpr (T == T_Q4_0) {
            RawQ40 ru;
            load_unit(ru, rs, off, 0);
            const Q40Fields r = fields(ru);
            float w[32];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const u32 byte = (r.q[i >> 2] >> (8 * (i & 3))) & 0xFFu;
                w[i] = r.d * (float)((int)(byte & 15u) - 8) + 0.0f;
                w[16 + i] = r.d * (float)((int)(byte >> 4) - 8) + 0.0f;
            }
            f4 *o4 = reinterpret_cast<f4 *>(out);
#pragma unroll
            for (int i = 0; i < 8; ++i) o4[i] = f4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
        } else if constexpr (T == T_Q5_K) {
            RawQ5K r;
            load_unit(r, rs, off, sub);
            const u32 h0 = r.h.x, h1 = r.h.y, h2 = r.h.z, h3 = r.h.w;
            const float d = half_lo(h0), dmin = half_lo(h0 >> 16);
            const u32 sc_lo = h1 & 0x3F3F3F3Fu, m_lo = h2 & 0x3F3F3F3Fu;
            const u32 sc_hi = (h3 & 0x0F0F0F0Fu) | ((h1 >> 2) & 0x30303030u);
            const u32 m_hi = ((h3 >> 4) & 0x0F0F0F0Fu) | ((h2 >> 2) & 0x30303030u);
            const u32 sel = (u32)(2 * sub) | ((u32)(2 * sub + 1) << 8) | 0x0C0C0000u;
            const u32 sc = __builtin_amdgcn_perm(sc_hi, sc_lo, sel), mm = __builtin_amdgcn_perm(m_hi, m_lo, sel);
            const float ds0 = d * (float)(sc & 0xFFu), ds1 = d * (float)((sc >> 8) & 0xFFu);
            const float dm0 = dmin * (float)(mm & 0xFFu), dm1 = dmin * (float)((mm >> 8) & 0xFFu);
            float lo[32], hi[32];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const u32 D = i < 4 ? r.qa[i & 3] : r.qb[i & 3];
                const u32 H = i < 4 ? r.ha[i & 3] : r.hb[i & 3];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const u32 byte = (D >> (8 * j)) & 0xFFu, hb = (H >> (8 * j)) & 0xFFu;
                    const u32 ql = (byte & 15u) | (((hb >> (2 * sub)) & 1u) << 4);
                    const u32 qh = (byte >> 4) | (((hb >> (2 * sub + 1)) & 1u) << 4);
                    lo[4 * i + j] = __builtin_fmaf(ds0, (float)ql, -dm0) + 0.0f;
                    hi[4 * i + j] = __builtin_fmaf(ds1, (float)qh, -dm1) + 0.0f;
                }
            }
            f4 *o4 = reinterpret_cast<f4 *>(out + 64 * sub);
#pragma unroll
            for (int i = 0; i < 8; ++i) o4[i] = f4{lo[4 * i], lo[4 * i + 1], lo[4 * i + 2], lo[4 * i + 3]};
#pragma unroll
            for (int i = 0; i < 8; ++i) o4[8 + i] = f4{hi[4 * i], hi[4 * i + 1], hi[4 * i + 2], hi[4 * i + 3]};
        } else if constexpr (T == T_Q3_K) {
            const int h = sub >> 1, q2 = sub & 1;
            RawQ3K ru;
            load_unit(ru, rs, off, sub);
            const Q3KFields r = fields(ru);
            float dsc[4];
            q3k_scales(r, sub, dsc);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                float w[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const u32 q = (r.q[i >> 2] >> (8 * (i & 3) + 2 * s)) & 3u;
                    const u32 hb = (r.mk[i >> 2] >> (8 * (i & 3) + 4 * h + s)) & 1u;
                    w[i] = dsc[s] * (float)((int)(q | (hb << 2)) - 4) + 0.0f;
                }
                f4 *o4 = reinterpret_cast<f4 *>(out + 128 * h + 32 * s + 16 * q2);
#pragma unroll
                for (int i = 0; i < 4; ++i) o4[i] = f4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
            }
        } else {
            RawQ80 ru;
            load_unit(ru, rs, off, 0);
            const Q80Fields r = fields(ru);
            float w[32];
#pragma unroll
            for (int i = 0; i < 32; ++i) w[i] = r.d * (float)(int)(signed char)(r.q[i >> 2] >> (8 * (i & 3))) + 0.0f;
            f4 *o4 = reinterpret_cast<f4 *>(out);
#pragma unroll
            for (int i = 0; i < 8; ++i) o4[i] = f4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int64_t n4 = ((nunits - u0 < 64 ? nunits - u0 : 64) * UW) >> 2;
    f4 *dst4 = reinterpret_cast<f4 *>(dst + u0 * UW);
#pragma unroll
    for (int i = 0; i < UW / 4; ++i) {
        const int q = 64 * i + lane;
        if (q < n4) dst4[q] = win4[wave][q];
    }
}

// ---------------------------------------------------------------------------
// Host side

inline int fmt_of(int type, int *qk, int *bytes, int *upb) {
    switch (type) {
    case KQ_TYPE_Q4_K: *qk = 256; *bytes = 144; *upb = 4; return 0;
    case KQ_TYPE_Q6_K: *qk = 256; *bytes = 210; *upb = 4; return 0;
    case KQ_TYPE_Q2_K: *qk = 256; *bytes = 84; *upb = 4; return 0;
    case KQ_TYPE_Q8_0: *qk = 32; *bytes = 34; *upb = 1; return 0;
    case KQ_TYPE_Q4_0: *qk = 32; *bytes = 18; *upb = 1; return 0;
    case KQ_TYPE_Q5_K: *qk = 256; *bytes = 176; *upb = 4; return 0;
    case KQ_TYPE_Q3_K: *qk = 256; *bytes = 110; *upb = 4; return 0;
    default: return KQ_ERR_TYPE;
    }
}

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Calls fn(TypeTag<T>{}) with the format of a valid type id.
template <int T> using TypeTag = std::integral_constant<int, T>;
template <class Fn> int with_type(int type, Fn &&fn) {
    switch (type) {
    case KQ_TYPE_Q4_K: return fn(TypeTag<T_Q4_K>{});
    case KQ_TYPE_Q6_K: return fn(TypeTag<T_Q6_K>{});
    case KQ_TYPE_Q2_K: return fn(TypeTag<T_Q2_K>{});
    case KQ_TYPE_Q3_K: return fn(TypeTag<T_Q3_K>{});
    case KQ_TYPE_Q5_K: return fn(TypeTag<T_Q5_K>{});
    case KQ_TYPE_Q4_0: return fn(TypeTag<T_Q4_0>{});
    default: return fn(TypeTag<T_Q8_0>{});
    }
}

// Bytes per row of K weights of a valid type (K a multiple of the block).
inline int64_t kq_row_bytes_(int type, int64_t K) {
    int qk, nb, upb;
    fmt_of(type, &qk, &nb, &upb);
    return (K / qk) * nb;
}

// K chunk staged in LDS per M: a multiple of 4096 so that the lane owning a
// unit never depends on the chunking (units per 4096 columns are a multiple of
// 64 for every format).
inline int chunk_for(int M) { return M == 1 ? 8192 : 4096; }

// Lanes per row: enough that a row of fewer than 64 units fits one stripe.
inline int lanes_per_row(int units) { return units > 32 ? 64 : (units > 16 ? 32 : 16); }

// Lets kernel k use `bytes` of dynamic LDS on the current device.  The limit
// is only ever raised, under a lock: with calls from several host threads it
// never drops below what a launch in flight on another thread needs.
inline std::mutex &lds_limit_mutex() {
    static std::mutex mu;
    return mu;
}
template <typename Kern>
hipError_t allow_lds(Kern k, size_t bytes) {
    if (bytes <= 65536) return hipSuccess;
    static std::map<std::pair<const void *, int>, size_t> limit;   // (kernel, device) -> bytes allowed
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    const void *f = reinterpret_cast<const void *>(k);
    std::lock_guard<std::mutex> lock(lds_limit_mutex());
    size_t &cur = limit[{f, dev}];
    if (bytes <= cur) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess) cur = bytes;
    return e;
}

template <int T, int M, int R>
int launch_qgemv_t(const void *W, int64_t row_bytes, int N, int K, const float *x, float *y, hipStream_t st,
                   int lpr) {
    const int KC = chunk_for(M);
    const int kc = KC < K ? KC : K;
    const size_t lds = (size_t)lds_floats(M, kc) * sizeof(float);
    const int rows_per_wg = WAVES * (64 / lpr) * R;
    const int grid = (N + rows_per_wg - 1) / rows_per_wg;
    auto kern = qgemv_kernel<T, M, R>;
    if (allow_lds(kern, lds) != hipSuccess) return KQ_ERR_LAUNCH;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(WG_THREADS), lds, st, (const uint8_t *)W, row_bytes, N, K, KC, lpr,
                       x, y);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_LAUNCH;
}

// Launch of qgemv_seg_kernel over the segments sa (format TA) and sb (format
// TB) at M = 1; both formats have the same units per row (the same lpr).
template <int TA, int TB>
int launch_seg_small(const Segs &sa, int64_t rba, const Segs &sb, int64_t rbb, int K, const float *x,
                     hipStream_t st) {
    const int lpr = lanes_per_row((K / Fmt<TA>::QK) * Fmt<TA>::UPB);
    const int rows_per_wg = WAVES * (64 / lpr);
    SegTiles ta = {}, tb = {};
    for (int i = 0; i < sa.n; ++i) ta.t[i + 1] = ta.t[i] + (sa.rows[i] + rows_per_wg - 1) / rows_per_wg;
    for (int i = 0; i < sb.n; ++i) tb.t[i + 1] = tb.t[i] + (sb.rows[i] + rows_per_wg - 1) / rows_per_wg;
    const int64_t grid = (int64_t)ta.t[sa.n] + tb.t[sb.n];
    if (grid == 0) return KQ_OK;
    const size_t lds = (size_t)lds_floats(1, K) * sizeof(float);
    auto kern = qgemv_seg_kernel<TA, TB>;
    if (allow_lds(kern, lds) != hipSuccess) return KQ_ERR_LAUNCH;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(WG_THREADS), lds, st, sa, ta, rba, sb, tb, rbb, tb.t[sb.n],
                       rows_per_wg, K, lpr, x);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_LAUNCH;
}

// Compute units of the current device (cached per device).
inline int cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    int n = dev < 64 ? cache[dev].load(std::memory_order_relaxed) : 0;
    if (!n) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Batch-1 configurations: a wide one (work-groups up to 16 waves, 4 per SIMD,
// 128 VGPRs) and a narrow one (up to 8 waves, 2 per SIMD, 256 VGPRs) whose
// larger register budget pays for a deeper prefetch ring.  The formats whose
// units carry the most raw registers (Q6_K, Q5_K, Q3_K: more than 4 bits a
// weight) and the 32-weight formats (Q8_0, Q4_0: a scale per 32) take the
// narrow one when it still holds at least two row slots (32-weight formats:
// one), which measured faster for Q6_K and Q8_0; with long rows the wide
// one's extra waves win.  Q4_K and Q2_K (ring of 4) and Q3_K take the narrow
// one only for launches of at most 8 row steps per wide row slot (an 8B
// model's projections), where having every step's loads in flight early
// matters more than the wide one's extra waves (Q3_K 28672 x 8192: +12 %
// wide; Q2_K 14336 x 4096: +11 % narrow; Q5_K and Q6_K measured better narrow
// throughout); rows of two or more stripes only up to 3 row steps outside a
// two-format launch (8192 x 8192 Q4_K: 10.6 -> 10.1 us wide, Q2_K 9.6 -> 9.0,
// since the activations load first).
// PREFETCH is the number of row steps each wave keeps in flight; it must
// divide every lanes-per-row value (16, 32, 64).
template <int T, bool WIDE> constexpr int PREFETCH() {
    return WIDE ? (BIG_UNIT<T>() ? 1 : 2) : (Fmt<T>::QK == 32 || T == T_Q4_K || T == T_Q2_K ? 4 : 2);
}
template <int T> constexpr int NARROW_MAX_STRIPES() {
    return BIG_UNIT<T>() ? 4 : (Fmt<T>::QK == 32 ? 8 : (T == T_Q4_K || T == T_Q2_K ? 2 : 0));
}
// formats that take the narrow configuration only for short launches
template <int T> constexpr bool NARROW_SHORT_ONLY() { return T == T_Q4_K || T == T_Q3_K || T == T_Q2_K; }
constexpr int64_t SHORT_LAUNCH_STEPS = 8, SHORT_MULTI_STRIPE_STEPS = 3;

struct B1Cfg {
    int lpr, ns, rs;
    size_t lds;
    bool wide;
};

// Small launches of short rows at M = 1 go to the non-persistent LDS kernel
// (one matrix) or its grouped form qgemv_seg_kernel (several, of one or two
// formats): many 4-wave work-groups, each issuing all its loads at once,
// reach the first bytes sooner than the persistent kernel's per-CU ring
// (4096 x 4096 Q4_K 6.3 -> 5.0 us, 1024 x 4096 5.1 -> 4.0 us, Q2_K 4096 x 4096
// 5.9 -> 4.6 us; an 8B layer's k+v+q 8.5 -> 7.2 us, three 2048 x 4096 Q4_K
// 7.0 -> 6.1 us); the two are even near 28 MB (12288 x 4096 Q4_K, 4096 x 8192
// Q6_K), and the persistent kernels win for larger launches and longer rows
// (8192 x 8192 Q4_K 11.5 vs 13.6 us; 1024 x 16384 7.1 vs 8.6 us).
constexpr int64_t SMALL_LAUNCH_BYTES = 20 << 20;
inline bool small_launch(int K, int64_t bytes) { return K <= 8192 && bytes <= SMALL_LAUNCH_BYTES; }
template <int T> constexpr int64_t rba_of(int K) { return Fmt<T>::BYTES * (int64_t)(K / Fmt<T>::QK); }

// Batch-1 configuration for a launch over `rows` rows of K columns; false:
// use the LDS kernel.
template <int T> bool batch1_cfg(int K, int64_t rows, B1Cfg *c, bool mixed = false) {
    const int units = (K / Fmt<T>::QK) * Fmt<T>::UPB;
    c->lpr = lanes_per_row(units);
    c->ns = units > 64 ? (units + 63) / 64 : 1;
    c->lds = (size_t)(16 * 64 + x_stride(K) + s_stride(K)) * sizeof(float);
    c->wide = c->ns > NARROW_MAX_STRIPES<T>();
    if (NARROW_SHORT_ONLY<T>() && !c->wide) {
        // row steps per row slot of the wide configuration
        const int64_t slots = (rows + 64 / c->lpr - 1) / (64 / c->lpr);
        const int64_t per_round = (int64_t)cu_count() * (16 / c->ns);
        const int64_t steps = (slots + per_round - 1) / per_round;
        // rows of two or more stripes take the wide configuration from
        // SHORT_MULTI_STRIPE_STEPS on, except in a two-format launch
        c->wide = steps > SHORT_LAUNCH_STEPS || (!mixed && c->ns >= 2 && steps > SHORT_MULTI_STRIPE_STEPS);
    }
    const int maxw = c->wide ? 16 : 8;
    if (c->ns > maxw || c->lds > 150 * 1024) return false;
    c->rs = maxw / c->ns;
    // the prologue stages at most two groups of 16 activations per thread
    if (K / 16 > 2 * 64 * c->ns * c->rs) return false;
    return true;
}

template <int T, bool WIDE>
int launch_qgemv1_cfg(const B1Cfg &c, const Segs &sg, int64_t row_bytes, int K, const float *x, hipStream_t st) {
    const int nt = 64 * c.ns * c.rs;
    const int G = 64 / c.lpr;
    constexpr int D = PREFETCH<T, WIDE>(), LB = WIDE ? 1024 : 512;
    // rows of 64 units or more (lpr 64) get the kernel with the lane count fixed
    auto kern = sg.n > 1 ? (c.lpr == 64 ? qgemv1_kernel<T, D, LB, true, 64> : qgemv1_kernel<T, D, LB, true, 0>)
                         : (c.lpr == 64 ? qgemv1_kernel<T, D, LB, false, 64> : qgemv1_kernel<T, D, LB, false, 0>);
    if (allow_lds(kern, c.lds) != hipSuccess) return KQ_ERR_LAUNCH;
    const int64_t slots = ((int64_t)sg.start[sg.n] + G - 1) / G;
    const int64_t need = (slots + c.rs - 1) / c.rs;
    const int64_t cap = cu_count();
    const int grid = (int)(need < cap ? need : cap);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(nt), c.lds, st, x, K, nt, sg, row_bytes, c.lpr, c.ns);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_LAUNCH;
}

// Batch-1 launches with the weight ring in LDS (qgemv1_dma_kernel), for Q4_K:
// the same work-group shapes and ring depths as the register ring (2 steps
// with 16 waves, 4 with 8); needs 16-byte aligned matrices and rows and the
// ring's LDS beside the staged activations.  (The same pass for Q6_K, with
// each lane's activations loaded from global memory to make room for the
// ring, measured 3-10 % slower than its register ring.)
constexpr size_t LDS_MAX = 160 * 1024;
template <int T> constexpr bool DMA_FMT() { return T == T_Q4_K; }
template <bool WIDE> constexpr int DMA_DEPTH() { return WIDE ? 2 : 4; }
template <int T> size_t dma_lds(const B1Cfg &c, int K) {
    return b1_ring_offset(K) +
           (size_t)(c.ns * c.rs) * (c.wide ? DMA_DEPTH<true>() : DMA_DEPTH<false>()) * DmaGeom<T>::SLOT;
}
template <int T> bool dma_ok(const B1Cfg &c, const Segs &sg, int64_t row_bytes, int K) {
    if (row_bytes % 16 || dma_lds<T>(c, K) > LDS_MAX) return false;
    for (int i = 0; i < sg.n; ++i)
        if ((uintptr_t)sg.W[i] % 16) return false;
    return true;
}
template <int T, bool WIDE>
int launch_qgemv1_dma(const B1Cfg &c, const Segs &sg, int64_t row_bytes, int K, const float *x, hipStream_t st) {
    constexpr int D = DMA_DEPTH<WIDE>(), LB = WIDE ? 1024 : 512;
    const int nt = 64 * c.ns * c.rs;
    const int G = 64 / c.lpr;
    const size_t lds = dma_lds<T>(c, K);
    // rows of 64 units or more (lpr 64) get the kernel with the lane count fixed
    auto kern = sg.n > 1 ? (c.lpr == 64 ? qgemv1_dma_kernel<T, D, LB, true, 64> : qgemv1_dma_kernel<T, D, LB, true, 0>)
                         : (c.lpr == 64 ? qgemv1_dma_kernel<T, D, LB, false, 64> : qgemv1_dma_kernel<T, D, LB, false, 0>);
    if (allow_lds(kern, lds) != hipSuccess) return KQ_ERR_LAUNCH;
    const int64_t slots = ((int64_t)sg.start[sg.n] + G - 1) / G;
    const int64_t need = (slots + c.rs - 1) / c.rs;
    const int64_t cap = cu_count();
    const int grid = (int)(need < cap ? need : cap);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(nt), lds, st, x, K, nt, sg, row_bytes, c.lpr, c.ns);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_LAUNCH;
}

// Batch-1 launch over one or more segments (same format and K): one lane per
// unit, stripes of 64 units, one work-group per compute unit (persistent).
template <int T>
int launch_qgemv1(const B1Cfg &c, const Segs &sg, int64_t row_bytes, int K, const float *x, hipStream_t st) {
    if constexpr (DMA_FMT<T>()) {
        if (dma_ok<T>(c, sg, row_bytes, K))
            return c.wide ? launch_qgemv1_dma<T, true>(c, sg, row_bytes, K, x, st)
                          : launch_qgemv1_dma<T, false>(c, sg, row_bytes, K, x, st);
    }
    if constexpr (NARROW_MAX_STRIPES<T>() > 0) {
        if (!c.wide) return launch_qgemv1_cfg<T, false>(c, sg, row_bytes, K, x, st);
    }
    return launch_qgemv1_cfg<T, true>(c, sg, row_bytes, K, x, st);
}

template <int T>
int launch_qgemv1_single(const void *W, int64_t row_bytes, int N, int K, const float *x, float *y, hipStream_t st) {
    B1Cfg c;
    if (small_launch(K, (int64_t)N * row_bytes) || !batch1_cfg<T>(K, N, &c))
        return launch_qgemv_t<T, 1, 1>(W, row_bytes, N, K, x, y, st, lanes_per_row((K / Fmt<T>::QK) * Fmt<T>::UPB));
    Segs sg = {};
    sg.W[0] = (const uint8_t *)W;
    sg.y[0] = y;
    sg.start[0] = 0;
    sg.start[1] = N;
    sg.rows[0] = N;
    sg.n = 1;
    return launch_qgemv1<T>(c, sg, row_bytes, K, x, st);
}

// Batch-M configuration: rows per lane group (R: each activation read from
// LDS serves R rows) and ring depth (D) per format and M, chosen by
// measurement among the settings that fit the 256-VGPR budget of 8-wave
// work-groups without spilling.  R = 2 keeps R * M <= 16 for the butterfly
// row sums.
template <int T, int M> constexpr int MROWS() { return 2; }
template <int T, int M> constexpr int MRING() { return (BIG_UNIT<T>() && M > 4) ? 1 : 2; }

// Batch-M launch over one or more segments (starts padded to the row step).
// Returns KQ_ERR_ARG when the activations of one 4096-column chunk do not fit
// in LDS next to the row sums (then the caller uses the LDS kernel).
// Q4_K at M = 2 on the LDS-ring kernel (8 waves, a ring of 2 steps) for rows of
// 64 units or more in 1 or 2 stripes (K <= 8192; longer rows leave no LDS
// for the ring beside two staged activation rows): it beats the batch-M
// kernel on short and long launches alike (70B wk + wq 20.3 -> 17.3 us, w1
// 28672 x 8192 36.2 -> 31.7 us, w1 + w3 69.3 -> 63.4 us); with 3 stripes (6
// waves busy) or short rows it does not.  KQ_ERR_ARG when the shape does not
// take it.
template <int T, int M>
int launch_qgemvm_dma(const Segs &sg, int64_t row_bytes, int K, const float *x, hipStream_t st) {
    constexpr int D = 2, LB = 512;
    const int units = (K / Fmt<T>::QK) * Fmt<T>::UPB;
    const int lpr = lanes_per_row(units);
    const int ns = units > 64 ? (units + 63) / 64 : 1;
    if (lpr != 64 || ns > 2) return KQ_ERR_ARG;
    const int rs = 8 / ns;
    if (K / 16 > 2 * 64 * ns * rs) return KQ_ERR_ARG;
    const size_t lds = b1_ring_offset(K, M) + (size_t)(ns * rs) * D * DmaGeom<T>::SLOT;
    if (row_bytes % 16 || lds > LDS_MAX) return KQ_ERR_ARG;
    for (int i = 0; i < sg.n; ++i)
        if ((uintptr_t)sg.W[i] % 16) return KQ_ERR_ARG;
    const int G = 64 / lpr;
    const int64_t slots = ((int64_t)sg.start[sg.n] + G - 1) / G;
    const int64_t need = (slots + rs - 1) / rs;
    const int64_t cap = cu_count();
    const int grid = (int)(need < cap ? need : cap);
    if (grid == 0) return KQ_OK;
    auto kern = sg.n > 1 ? qgemv1m_dma_kernel<T, D, LB, true, M, 64> : qgemv1m_dma_kernel<T, D, LB, false, M, 64>;
    if (allow_lds(kern, lds) != hipSuccess) return KQ_ERR_LAUNCH;
    const int nt = 64 * ns * rs;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(nt), lds, st, x, K, nt, sg, row_bytes, lpr, ns);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_LAUNCH;
}

template <int T, int M>
int launch_qgemvm(const Segs &sg, int64_t row_bytes, int K, const float *x, hipStream_t st) {
    if constexpr (T == T_Q4_K && M == 2) {
        const int r = launch_qgemvm_dma<T, M>(sg, row_bytes, K, x, st);
        if (r != KQ_ERR_ARG) return r;
    }
    constexpr int R = MROWS<T, M>(), D = MRING<T, M>(), NW = 8;
    const int units = (K / Fmt<T>::QK) * Fmt<T>::UPB;
    const int lpr = lanes_per_row(units);
    const int RG = R * (64 / lpr);
    const int N = sg.start[sg.n];
    const int64_t nsteps = ((int64_t)N + RG - 1) / RG;
    const int64_t need = (nsteps + NW - 1) / NW;
    const int64_t cap = cu_count();
    const int grid = (int)(need < cap ? need : cap);
    if (grid == 0) return KQ_OK;
    const int64_t wsteps = (nsteps + (int64_t)grid * NW - 1) / ((int64_t)grid * NW);
    const size_t acc = (size_t)wsteps * NW * RG * M * sizeof(float);
    auto bytes = [&](int kc) { return (size_t)M * (x_stride(kc) + s_stride(kc)) * sizeof(float) + acc; };
    int KC = K;
    if (bytes(K) > LDS_MAX) {
        KC = (K / 4096) * 4096;
        while (KC > 4096 && bytes(KC) > LDS_MAX) KC -= 4096;
        if (KC < 4096 || bytes(KC) > LDS_MAX) return KQ_ERR_ARG;
    }
    const size_t lds = bytes(KC);
    auto kern = sg.n > 1 ? qgemvm_kernel<T, M, R, D, true> : qgemvm_kernel<T, M, R, D, false>;
    if (allow_lds(kern, lds) != hipSuccess) return KQ_ERR_LAUNCH;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * NW), lds, st, sg, row_bytes, K, KC, lpr, x);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_LAUNCH;
}

template <int T, int M>
int launch_qgemvm_single(const void *W, int64_t row_bytes, int N, int K, const float *x, float *y, hipStream_t st) {
    Segs sg = {};
    sg.W[0] = (const uint8_t *)W;
    sg.y[0] = y;
    sg.start[0] = 0;
    sg.start[1] = N;
    sg.rows[0] = N;
    sg.n = 1;
    const int r = launch_qgemvm<T, M>(sg, row_bytes, K, x, st);
    if (r != KQ_ERR_ARG) return r;
    const int lpr = lanes_per_row((K / Fmt<T>::QK) * Fmt<T>::UPB);
    return launch_qgemv_t<T, M, 1>(W, row_bytes, N, K, x, y, st, lpr);
}

template <int T>
int launch_qgemv_m(int M, const void *W, int64_t row_bytes, int N, int K, const float *x, float *y,
                   hipStream_t st) {
    switch (M) {
    case 1: return launch_qgemv1_single<T>(W, row_bytes, N, K, x, y, st);
    case 2: return launch_qgemvm_single<T, 2>(W, row_bytes, N, K, x, y, st);
    case 3: return launch_qgemvm_single<T, 3>(W, row_bytes, N, K, x, y, st);
    case 4: return launch_qgemvm_single<T, 4>(W, row_bytes, N, K, x, y, st);
    case 5: return launch_qgemvm_single<T, 5>(W, row_bytes, N, K, x, y, st);
    case 6: return launch_qgemvm_single<T, 6>(W, row_bytes, N, K, x, y, st);
    case 7: return launch_qgemvm_single<T, 7>(W, row_bytes, N, K, x, y, st);
    default: return launch_qgemvm_single<T, 8>(W, row_bytes, N, K, x, y, st);
    }
}

// Segments for the matrices ids[*pos ..] (their rows numbered one after the
// other, each start padded to a multiple of `pad` rows): at most MAX_SEGS, and
// fewer than 2^31 numbered rows.  Advances *pos; false when none is left.
inline bool next_segs(const std::vector<int> &ids, size_t *pos, const void *const *W, const int64_t *N,
                      float *const *y, int64_t pad, Segs *sg) {
    *sg = Segs{};
    int64_t at = 0;
    while (*pos < ids.size() && sg->n < MAX_SEGS) {
        const int i = ids[*pos];
        const int64_t next = at + (N[i] + pad - 1) / pad * pad;
        if (next >= ((int64_t)1 << 31)) break;
        sg->W[sg->n] = (const uint8_t *)W[i];
        sg->y[sg->n] = y[i];
        sg->start[sg->n] = (int)at;
        sg->rows[sg->n] = (int)N[i];
        ++sg->n;
        at = next;
        ++*pos;
    }
    sg->start[sg->n] = (int)at;
    return sg->n > 0;
}

// Products y[i] = W[i] . x of one format and K for the matrices ids, M rows.
template <int T>
int launch_group(int M, const std::vector<int> &ids, const void *const *W, const int64_t *N, int64_t row_bytes,
                 int K, const float *x, float *const *y, hipStream_t st) {
    size_t pos = 0;
    Segs sg;
    if (M == 1) {
        B1Cfg c;
        int64_t rows = 0;
        for (int i : ids) rows += N[i];
        if (small_launch(K, rows * row_bytes)) {
            if (ids.size() == 1)
                return launch_qgemv_t<T, 1, 1>(W[ids[0]], row_bytes, (int)N[ids[0]], K, x, y[ids[0]], st,
                                               lanes_per_row((K / Fmt<T>::QK) * Fmt<T>::UPB));
            while (next_segs(ids, &pos, W, N, y, 1, &sg)) {
                const int r = launch_seg_small<T, T>(Segs{}, row_bytes, sg, row_bytes, K, x, st);
                if (r) return r;
            }
            return KQ_OK;
        }
        if (!batch1_cfg<T>(K, rows, &c)) {
            const int lpr = lanes_per_row((K / Fmt<T>::QK) * Fmt<T>::UPB);
            for (int i : ids) {
                const int r = launch_qgemv_t<T, 1, 1>(W[i], row_bytes, (int)N[i], K, x, y[i], st, lpr);
                if (r) return r;
            }
            return KQ_OK;
        }
        while (next_segs(ids, &pos, W, N, y, 64 / c.lpr, &sg)) {
            const int r = launch_qgemv1<T>(c, sg, row_bytes, K, x, st);
            if (r) return r;
        }
        return KQ_OK;
    }
    const int lpr = lanes_per_row((K / Fmt<T>::QK) * Fmt<T>::UPB);
    const int64_t pad = 2 * (64 / lpr);          // the batch-M row step (MROWS = 2)
    while (next_segs(ids, &pos, W, N, y, pad, &sg)) {
        int r;
        switch (M) {
        case 2: r = launch_qgemvm<T, 2>(sg, row_bytes, K, x, st); break;
        case 3: r = launch_qgemvm<T, 3>(sg, row_bytes, K, x, st); break;
        case 4: r = launch_qgemvm<T, 4>(sg, row_bytes, K, x, st); break;
        case 5: r = launch_qgemvm<T, 5>(sg, row_bytes, K, x, st); break;
        case 6: r = launch_qgemvm<T, 6>(sg, row_bytes, K, x, st); break;
        case 7: r = launch_qgemvm<T, 7>(sg, row_bytes, K, x, st); break;
        default: r = launch_qgemvm<T, 8>(sg, row_bytes, K, x, st); break;
        }
        if (r == KQ_ERR_ARG) {                     // activations too large for LDS: one call each
            for (int s = 0; s < sg.n; ++s) {
                r = launch_qgemv_m<T>(M, sg.W[s], row_bytes, sg.rows[s], K, x, sg.y[s], st);
                if (r) return r;
            }
        } else if (r) {
            return r;
        }
    }
    return KQ_OK;
}

// Batch-1 configuration of the 16-wave kernel whatever the format prefers
// (the two passes of a mixed launch share the work-group shape).
template <int T> bool batch1_wide_cfg(int K, B1Cfg *c) {
    if (!batch1_cfg<T>(K, 0, c)) return false;
    if (c->wide) return true;
    c->wide = true;
    if (c->ns > 16) return false;
    c->rs = 16 / c->ns;
    return K / 16 <= 2 * 64 * c->ns * c->rs;
}

// Two K-quant formats (type ids TA < TB) with the same K in one launch: up to
// MAX_SEGS matrices of each; returns how many of each it served.
template <int TA, int TB>
int launch_mixed(const std::vector<int> &ia, size_t *pa, const std::vector<int> &ib, size_t *pb,
                 const void *const *W, const int64_t *N, int K, const float *x, float *const *y, hipStream_t st) {
    B1Cfg ca, cb;
    if (!batch1_wide_cfg<TA>(K, &ca) || !batch1_wide_cfg<TB>(K, &cb) || ca.lpr != cb.lpr || ca.ns != cb.ns ||
        ca.rs != cb.rs)
        return KQ_ERR_ARG;
    const int G = 64 / ca.lpr;
    Segs sa, sb;
    const size_t pa0 = *pa, pb0 = *pb;
    next_segs(ia, pa, W, N, y, G, &sa);
    next_segs(ib, pb, W, N, y, G, &sb);
    int64_t bytes = 0;
    for (int i = 0; i < sa.n; ++i) bytes += sa.rows[i] * rba_of<TA>(K);
    for (int i = 0; i < sb.n; ++i) bytes += sb.rows[i] * rba_of<TB>(K);
    if (small_launch(K, bytes)) return launch_seg_small<TA, TB>(sa, rba_of<TA>(K), sb, rba_of<TB>(K), K, x, st);
    // the 8-wave configuration when each format would take it for its own rows
    // (short launches of Q4_K, Q3_K and Q2_K; rows of few stripes otherwise);
    // else the formats go to launches of their own: two formats' code in one
    // 16-wave kernel needs more than the 128 registers a lane has there (it
    // spilled 44-116 bytes a lane)
    B1Cfg na, nb;
    const bool narrow = batch1_cfg<TA>(K, sa.start[sa.n], &na, true) && batch1_cfg<TB>(K, sb.start[sb.n], &nb, true) &&
                        !na.wide && !nb.wide && na.rs == nb.rs;
    if (!narrow) {
        *pa = pa0;
        *pb = pb0;
        return KQ_ERR_ARG;
    }
    ca = na;
    const int64_t rba = Fmt<TA>::BYTES * (int64_t)(K / Fmt<TA>::QK), rbb = Fmt<TB>::BYTES * (int64_t)(K / Fmt<TB>::QK);
    // work-groups each format needs for one step per row slot; when both do
    // not fit one per compute unit, the units are split so that the slowest
    // work-group finishes first: a work-group makes a whole number of row
    // steps, each costing its format's row bytes weighted by the format's
    // relative time per byte, and ties go to the split closer to proportional.
    // The large-unit formats keep two row steps in flight (weight 1.1).
    const int64_t need_a = (((int64_t)sa.start[sa.n] + G - 1) / G + ca.rs - 1) / ca.rs;
    const int64_t need_b = (((int64_t)sb.start[sb.n] + G - 1) / G + ca.rs - 1) / ca.rs;
    const int64_t cap = cu_count();
    int64_t ga = need_a, gb = need_b;
    if (ga + gb > cap) {
        const double big = 1.1;
        const double wa = (BIG_UNIT<TA>() ? big : 1.0) * rba, wb = (BIG_UNIT<TB>() ? big : 1.0) * rbb;
        double best = 0, best_even = 0;
        for (int64_t b = 1; b < cap && b <= need_b; ++b) {
            const int64_t a = cap - b;
            const double t = std::max((double)((need_a + a - 1) / a) * wa, (double)((need_b + b - 1) / b) * wb);
            const double even = std::max((double)need_a / a * wa, (double)need_b / b * wb);
            if (b == 1 || t < best || (t == best && even < best_even)) {
                best = t;
                best_even = even;
                gb = b;
            }
        }
        ga = cap - gb < need_a ? cap - gb : need_a;
    }
    const int grid = (int)(ga + gb);
    if (grid == 0) return KQ_OK;
    size_t lds = ca.lds > cb.lds ? ca.lds : cb.lds;
    // rows of 64 units or more (lpr 64) get the kernels with the lane count fixed
    const bool l64 = ca.lpr == 64;
    auto kern = l64 ? qgemv1_mixed_kernel<TA, PREFETCH<TA, false>(), TB, PREFETCH<TB, false>(), 512, false, 64>
                    : qgemv1_mixed_kernel<TA, PREFETCH<TA, false>(), TB, PREFETCH<TB, false>(), 512, false, 0>;
    if constexpr (TA == T_Q4_K || TB == T_Q4_K) {
        // the Q4_K side through the LDS ring
        B1Cfg cq = ca;
        cq.wide = false;
        if (dma_ok<T_Q4_K>(cq, TA == T_Q4_K ? sa : sb, TA == T_Q4_K ? rba : rbb, K)) {
            lds = std::max(lds, dma_lds<T_Q4_K>(cq, K));
            kern = l64 ? qgemv1_mixed_kernel<TA, PREFETCH<TA, false>(), TB, PREFETCH<TB, false>(), 512, true, 64>
                       : qgemv1_mixed_kernel<TA, PREFETCH<TA, false>(), TB, PREFETCH<TB, false>(), 512, true, 0>;
        }
    }
    if (allow_lds(kern, lds) != hipSuccess) return KQ_ERR_LAUNCH;
    const int nt = 64 * ca.ns * ca.rs;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(nt), lds, st, x, K, nt, sa, rba, sb, rbb, (int)gb, ca.lpr, ca.ns);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_LAUNCH;
}

template <int T, int MAXM>
int launch_qmoe_t(const MoeSet &set, int64_t row_bytes, int E, int N, int K, const int32_t *ids, int T_, int k,
                  const float *x, int x_mode, int32_t *err, hipStream_t st) {
    const int units = (K / Fmt<T>::QK) * Fmt<T>::UPB;
    const int lpr = lanes_per_row(units);
    const int KC = chunk_for(MAXM);
    const int kc = KC < K ? KC : K;
    const size_t lds = (size_t)lds_floats(MAXM, kc) * sizeof(float);
    const int rows_per_wg = WAVES * (64 / lpr) * MOE_ROWS<T, MAXM>();
    dim3 grid((N + rows_per_wg - 1) / rows_per_wg, T_ * k * set.n);
    auto kern = qmoe_kernel<T, MAXM>;
    if (allow_lds(kern, lds) != hipSuccess) return KQ_ERR_LAUNCH;
    hipLaunchKernelGGL(kern, grid, dim3(WG_THREADS), lds, st, set, row_bytes, E, N, K, KC, lpr, ids, T_ * k, k, x,
                       x_mode, err);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_LAUNCH;
}

template <int T>
int launch_qmoe_m(int maxm, const MoeSet &set, int64_t row_bytes, int E, int N, int K, const int32_t *ids, int T_,
                  int k, const float *x, int x_mode, int32_t *err, hipStream_t st) {
    switch (maxm) {
    case 1: return launch_qmoe_t<T, 1>(set, row_bytes, E, N, K, ids, T_, k, x, x_mode, err, st);
    case 2: return launch_qmoe_t<T, 2>(set, row_bytes, E, N, K, ids, T_, k, x, x_mode, err, st);
    case 3: case 4: return launch_qmoe_t<T, 4>(set, row_bytes, E, N, K, ids, T_, k, x, x_mode, err, st);
    default: return launch_qmoe_t<T, 8>(set, row_bytes, E, N, K, ids, T_, k, x, x_mode, err, st);
    }
}

// The token-major routed-expert kernel (qmoe_tok_kernel) for T tokens and
// set.n expert tensors, when the activation rows a work-group stages (and the
// slot sums of a row tile, with rw) fit its LDS budget; KQ_ERR_ARG otherwise
// (the caller then uses the slot-major kernel).  Row tiles of G * MOEC_R * S rows,
// S as large as keeps at least two work-groups per compute unit.
constexpr size_t MOEC_LDS_MAX = 64 * 1024;
template <int T>
int launch_qmoe_tok_t(const MoeSet &set, int64_t row_bytes, int E, int N, int K, const int32_t *ids, const float *rw,
                      int T_, int k, const float *x, int x_mode, int32_t *err, hipStream_t st) {
    const int units = (K / Fmt<T>::QK) * Fmt<T>::UPB;
    const int lpr = lanes_per_row(units);
    const int step = (64 / lpr) * MOEC_R;
    const int64_t per_tile = (int64_t)T_ * set.n;
    int S = 1;
    while (S < 4 && (int64_t)((N + 2 * S * step - 1) / (2 * S * step)) * per_tile >= 2 * cu_count()) S *= 2;
    const int RT = S * step;
    const int nx = x_mode ? k : 1;
    const size_t lds = ((size_t)nx * (x_stride(K) + s_stride(K)) + (rw ? (size_t)k * RT : 0)) * sizeof(float);
    if (lds > MOEC_LDS_MAX) return KQ_ERR_ARG;
    auto kern = qmoe_tok_kernel<T>;
    if (allow_lds(kern, lds) != hipSuccess) return KQ_ERR_LAUNCH;
    hipLaunchKernelGGL(kern, dim3((N + RT - 1) / RT, (unsigned)per_tile), dim3(64 * MOEC_WAVES), lds, st, x, ids, K,
                       k, x_mode, T_, set, row_bytes, E, N, lpr, RT, rw, err);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_LAUNCH;
}

template <int T>
int launch_dequant_t(const void *src, int64_t n, float *dst, hipStream_t st) {
    const int64_t nunits = (n / Fmt<T>::QK) * Fmt<T>::UPB;
    const int64_t grid = (nunits + WG_THREADS - 1) / WG_THREADS;
    hipLaunchKernelGGL(dequant_kernel<T>, dim3((unsigned)grid), dim3(WG_THREADS), 0, st, (const uint8_t *)src,
                       nunits, dst);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_LAUNCH;
}

// ---------------------------------------------------------------------------
// Instantiation.  kq_inst.hip instantiates the launchers of one format (or one
// mixed pair) per object; every other unit sees only these declarations.
#define KQ_TYPE_LAUNCHERS(X, T)                                                                                  \
    X int launch_group<T>(int, const std::vector<int> &, const void *const *, const int64_t *, int64_t, int,      \
                          const float *, float *const *, hipStream_t);                                          \
    X int launch_qgemv_m<T>(int, const void *, int64_t, int, int, const float *, float *, hipStream_t);          \
    X int launch_qmoe_m<T>(int, const MoeSet &, int64_t, int, int, int, const int32_t *, int, int, const float *, \
                           int, int32_t *, hipStream_t);                                                        \
    X int launch_qmoe_tok_t<T>(const MoeSet &, int64_t, int, int, int, const int32_t *, const float *, int, int,    \
                               const float *, int, int32_t *, hipStream_t);                                        \
    X int launch_dequant_t<T>(const void *, int64_t, float *, hipStream_t);
#define KQ_MIXED_LAUNCHER(X, A, B)                                                                               \
    X int launch_mixed<A, B>(const std::vector<int> &, size_t *, const std::vector<int> &, size_t *,              \
                             const void *const *, const int64_t *, int, const float *, float *const *, hipStream_t);

// The matrix-core GEMV of the verify pass (kq_mc.hip): the grouped call once
// its arguments are checked (Q4_K and Q6_K matrices only).
int mc_run(int count, const int *types, const void *const *W, const int64_t *N, int K, const float *x, int M,
           float *const *y, hipStream_t st);

KQ_TYPE_LAUNCHERS(extern template, T_Q4_0)
KQ_TYPE_LAUNCHERS(extern template, T_Q8_0)
KQ_TYPE_LAUNCHERS(extern template, T_Q2_K)
KQ_TYPE_LAUNCHERS(extern template, T_Q3_K)
KQ_TYPE_LAUNCHERS(extern template, T_Q4_K)
KQ_TYPE_LAUNCHERS(extern template, T_Q5_K)
KQ_TYPE_LAUNCHERS(extern template, T_Q6_K)
// the ten K-quant pairs (lower type id first)
KQ_MIXED_LAUNCHER(extern template, T_Q2_K, T_Q3_K)
KQ_MIXED_LAUNCHER(extern template, T_Q2_K, T_Q4_K)
KQ_MIXED_LAUNCHER(extern template, T_Q2_K, T_Q5_K)
KQ_MIXED_LAUNCHER(extern template, T_Q2_K, T_Q6_K)
KQ_MIXED_LAUNCHER(extern template, T_Q3_K, T_Q4_K)
KQ_MIXED_LAUNCHER(extern template, T_Q3_K, T_Q5_K)
KQ_MIXED_LAUNCHER(extern template, T_Q3_K, T_Q6_K)
KQ_MIXED_LAUNCHER(extern template, T_Q4_K, T_Q5_K)
KQ_MIXED_LAUNCHER(extern template, T_Q4_K, T_Q6_K)
KQ_MIXED_LAUNCHER(extern template, T_Q5_K, T_Q6_K)

} // namespace kq
