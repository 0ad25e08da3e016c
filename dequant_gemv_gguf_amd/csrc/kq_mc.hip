// kq_mc.hip -- the matrix-core form of the fused dequant-GEMV for the few
// positions of a speculative-verify pass (Kortex summary, "Out-of-core LLM
// inference engine written from scratch in Rust", section Approach: the draft
// tokens are checked in one pass over the weights), for Q4_K and Q6_K rows.
// Entry points kq_qgemv_mc / kq_qgemv_mc_multi in include/kqgemv.h.
//
// At M positions the vector kernels spend M fused multiply-adds per weight on
// the vector ALU; here the multiply-accumulate goes to the matrix cores and
// the vector ALU keeps only the unpack and the scales:
//
//  * A 16-row tile of W is the B operand (16 columns) of the 16x16x32 f16
//    instruction (Q4_K: one 32-weight sub-block per instruction) or of the
//    16x16x16 f16 one (Q6_K: one 16-weight sub-block).  Lane l holds row
//    l % 16 of the tile at the k positions of lane group g = l / 16; the
//    quants are fp16 subnormal patterns (q * 2^-24, or 16q * 2^-24 for a
//    nibble left in place), made with one mask per two weights, as in the
//    vector kernels.  Q6_K subtracts its offset 32 on the patterns (exact).
//  * The A operand (16 rows) is the activations: row 2p + l holds limb l
//    (high, low fp16) of position p, so M = 8 fills it.  Per 256 columns and
//    position the activations are scaled by 2^e so that their largest
//    magnitude lies in [2^14, 2^15), then split x * 2^e = hi + lo (about 21
//    bits); the scale is undone exactly on the block's sum.  Each wave makes
//    the operands of the blocks it serves from the activations it copies into
//    LDS (the 32-column sums of Q4_K's min term come from one more matrix
//    instruction per sub-block).
//  * Slot s of lane group g is column 16 * (s / 4) + 4g + (0, 2, 1, 3)[s % 4]
//    of a 32-column sub-block: the byte order that the masks produce from a
//    dword of quants, and a layout in which the first and last four slots
//    are each one Q6_K scale group (the 16x16x16 instruction takes either
//    half).
//  * Output element r of lane (n, g) is row n of the tile at A row 4g + r:
//    the lane sums the two limbs of positions 2g and 2g + 1 and applies its
//    own row's sub-block scale (and, Q4_K, min).  Each output element depends
//    only on its own A row, so a position's result does not depend on M.
//
// Work: one persistent work-group of 8 waves per compute unit holds up to 16
// row tiles (interleaved over the grid); wave w takes the 256-column blocks
// b = w (mod 8) of every tile, keeps one block's activation operands in
// registers for all its tiles (the next block's are loaded meanwhile) and the
// next (tile, block) weights in flight; per-tile sums of the 8 waves are added
// in wave order through LDS at the end.  Rows are summed as
//   y = sum over waves w (ascending) of sum over the wave's blocks (ascending)
//       of [u * (sum over sub-blocks of scale * (dot_hi + dot_lo)) - min terms]
// with u = 2^(24 - e) -- a fixed order for given K, whatever N, M, tiling or
// grouping; it is not the vector kernels' order, so these results are within
// the GEMV tolerance of those, not bit-identical to them.
#include "kq_impl.h"

namespace kq {
namespace mc {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));

constexpr int THREADS = 512;                  // 8 waves
constexpr int TW_MAX = 16;                    // row tiles per work-group

// Matrices of one format served by one launch.
struct McSegs {
    const uint8_t *W[MAX_SEGS];
    float *y[MAX_SEGS];
    int rows[MAX_SEGS];
    int tstart[MAX_SEGS + 1];   // first tile of each matrix; tstart[n] = tiles
    int n;
};

// One block's activation operands as a lane uses them.
struct BlkX {
    h8 a[8];
    f4 sx[4];    // Q4_K: 32-column sums of positions 2g, 2g + 1, by sub-block
    f2 u;        // 2^(24 - e) of positions 2g, 2g + 1
};

struct Q4Raw { u4 h; u32 q[8]; };
struct Q6Raw { u32 ql[8], qh[4]; u4 sc; u32 dw; };
template <int T> struct McRaw;
template <> struct McRaw<T_Q4_K> { typedef Q4Raw type; };
template <> struct McRaw<T_Q6_K> { typedef Q6Raw type; };

// LDS staging of one (tile, block) item: the 16 rows' blocks copied by NLD
// buffer-to-LDS loads of 16 bytes per lane (1 KB per instruction), row r at
// r * RS.  Q4_K blocks (144 B) are 16-byte aligned and copied exactly; a
// Q6_K block (210 B, 2-byte aligned) is copied as the 14 aligned 16-byte
// pieces that cover it, its first byte `delta` bytes into the row.
// The last of the NLD loads runs on its first REM lanes only (a lane that is
// switched off writes nothing to LDS), so the slots hold exactly the pieces.
// The loads go through the caches as usual (no non-temporal hint): a block's
// first and last 128-byte lines are shared with the blocks beside it, which
// other waves read a little later, and kept in the caches they are fetched
// from memory again less often.
template <int T> struct Geo;
// NP of the PC pieces of a row are read.
template <> struct Geo<T_Q4_K> { static constexpr int RS = 144, PC = 9, NP = 9, NLD = 3, REM = 16, SLOT = 2304, D = 4; };
// (Q6_K rows take 15 pieces in LDS, the last one not read: a row stride of
// 240 bytes spreads the 16 rows' fields over the LDS banks two lanes a bank)
template <> struct Geo<T_Q6_K> { static constexpr int RS = 240, PC = 15, NP = 14, NLD = 4, REM = 48, SLOT = 3840, D = 3; };
constexpr int BLD = 8, BSLOT = BLD * 1024;   // a block's activations: one 1-KB load per position

#define MC_LDS __attribute__((address_space(3)))

// The buffers over a work-group's tiles, looked up once: lane i holds tile
// wg + i * nwg's (i < tw) -- its rows' first byte aligned down to 16 bytes
// (lo, hi), that byte's offset dt in the buffer, the rows it has (nr, at most
// 16) and the buffer's size.  An item reads its tile's entries with one
// lane-select each, instead of finding the tile's matrix among the segments.
struct TileTab {
    u32 lo, hi, dt, size;
    int nr;
};
__device__ __forceinline__ TileTab tile_tab(const McSegs &sg, int64_t row_bytes, int wg, int nwg, int tw, int lane) {
    const int t = wg + (lane < tw ? lane : 0) * nwg;   // (lanes past the tiles: a valid tile, unused)
    int s = 0;
#pragma unroll
    for (int i = 1; i < MAX_SEGS; ++i) s += (i < sg.n && t >= sg.tstart[i]) ? 1 : 0;
    int ts = 0, rows = 0;
    const uint8_t *W = sg.W[0];
#pragma unroll
    for (int i = 0; i < MAX_SEGS; ++i)
        if (s == i) {
            ts = sg.tstart[i];
            rows = sg.rows[i];
            W = sg.W[i];
        }
    const int row0 = (t - ts) * 16;
    const int left = rows - row0;
    TileTab tt;
    tt.nr = (lane >= tw || left <= 0) ? 0 : (left < 16 ? left : 16);
    const uint64_t base = (uint64_t)(uintptr_t)(W + (int64_t)row0 * row_bytes);
    tt.dt = (u32)(base & 15u);
    tt.lo = (u32)(base & ~(uint64_t)15);
    tt.hi = (u32)(base >> 32);
    tt.size = tt.nr ? tt.dt + (u32)(tt.nr * row_bytes) : 0u;
    return tt;
}

// Copies item (the work-group's tile i, block b) into an LDS slot (every lane
// takes part; the NLD loads are issued whatever `ok`, so the wait counts
// below hold; a missing item reads nothing).  i is uniform over the wave.
template <int T>
__device__ __forceinline__ void issue_item(const TileTab &tt, int64_t row_bytes, int i, int b, bool ok, char *slot,
                                           int lane) {
    typedef Geo<T> G;
    // (every value uniform: kept in scalar registers, so the loads need no
    // loop over distinct descriptors)
    const int nr = ok ? __builtin_amdgcn_readlane(tt.nr, i) : 0;
    const u32 dt = (u32)__builtin_amdgcn_readlane((int)tt.dt, i);
    const u32 lo = (u32)__builtin_amdgcn_readlane((int)tt.lo, i);
    const u32 hi = (u32)__builtin_amdgcn_readlane((int)tt.hi, i);
    const u32 size = ok ? (u32)__builtin_amdgcn_readlane((int)tt.size, i) : 0u;
    const rsrc_t rs = make_rsrc((const void *)(uintptr_t)(((uint64_t)hi << 32) | lo), size);
#pragma unroll
    for (int k = 0; k < G::NLD; ++k) {
        const int p = 64 * k + lane;
        const int r = p / G::PC, pc = p - r * G::PC;
        const u32 first = dt + (u32)(r * row_bytes) + (u32)b * Fmt<T>::BYTES;
        const u32 o = (r < nr && pc < G::NP) ? (first & ~15u) + 16u * pc : OOB;
        if (k < G::NLD - 1 || lane < G::REM)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (MC_LDS void *)(slot + 1024 * k), 16, o, 0, 0, 0);
    }
}

// Copies the activations of block b (columns 256b .. 256b + 255 of the M
// rows of x) into an LDS slot, row p at p * 1 KB; rows p >= M are not read
// (the copy writes zeros), so every block issues the same BLD loads.
__device__ __forceinline__ void issue_blk(rsrc_t xr, int K, int b, bool ok, int M, char *slot, int lane) {
#pragma unroll
    for (int p = 0; p < BLD; ++p)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (MC_LDS void *)(slot + 1024 * p), 16,
                                                 (ok && p < M) ? 4u * ((u32)p * K + 256u * b) + 16u * lane : OOB, 0,
                                                 0, 0);
}

// two floats to fp16, rounded toward zero, in one instruction
__device__ __forceinline__ hf2 pkrtz(float a, float b) {
    return __builtin_bit_cast(hf2, __builtin_amdgcn_cvt_pkrtz(a, b));
}
__device__ __forceinline__ float swap1(float v) {   // lane l ^ 1
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ u32 swap1u(u32 v) {
    return (u32)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ float max_lanes16_32(float v) {   // max over lanes l, l ^ 16, l ^ 32, l ^ 48
    {
        const u32 b = __builtin_bit_cast(u32, v);
        const auto p = __builtin_amdgcn_permlane16_swap(b, b, false, false);
        v = fmaxf(__builtin_bit_cast(float, (u32)p[0]), __builtin_bit_cast(float, (u32)p[1]));
    }
    {
        const u32 b = __builtin_bit_cast(u32, v);
        const auto p = __builtin_amdgcn_permlane32_swap(b, b, false, false);
        v = fmaxf(__builtin_bit_cast(float, (u32)p[0]), __builtin_bit_cast(float, (u32)p[1]));
    }
    return v;
}

// The block's matrix operands from its activations in LDS.  Lane (i, g)
// (i = 2p + limb) reads the four activations of position p at the columns of
// its lane group in one 16-column half of every sub-block (limb 0 the first,
// limb 1 the second), splits them into both limbs, and swaps with lane i ^ 1
// the limb the other one needs.  Scale: the largest magnitude of position
// p's 256 activations (over the 8 lanes that hold them) times 2^e in
// [2^14, 2^15).  The 32-column sums (Q4_K) come from one more matrix
// instruction per sub-block with all-ones weights.
template <int T> __device__ __forceinline__ void conv_blk(BlkX &bx, const f4 (&v)[8], int lane) {
    const int limb = lane & 1;
    float m = 0.f;
#pragma unroll
    for (int J = 0; J < 8; ++J)
        m = fmaxf(m, fmaxf(fmaxf(fabsf(v[J].x), fabsf(v[J].y)), fmaxf(fabsf(v[J].z), fabsf(v[J].w))));
    m = fmaxf(m, swap1(m));
    m = max_lanes16_32(m);
    const int E = (int)(__builtin_bit_cast(u32, m) >> 23);
    int e = m == 0.f ? 0 : 141 - E;
    e = e < -100 ? -100 : (e > 126 ? 126 : e);
    const float s = __builtin_bit_cast(float, (u32)(e + 127) << 23);
    const float u24 = __builtin_bit_cast(float, (u32)(151 - e) << 23);
#pragma unroll
    for (int J = 0; J < 8; ++J) {
        const float a0 = v[J].x * s, a1 = v[J].y * s, a2 = v[J].z * s, a3 = v[J].w * s;
        // slots (0, 1), (2, 3) of a half hold columns (0, 2), (1, 3)
        const hf2 h01 = pkrtz(a0, a2), h23 = pkrtz(a1, a3);
        const hf2 l01 = pkrtz(a0 - (float)h01.x, a2 - (float)h01.y);
        const hf2 l23 = pkrtz(a1 - (float)h23.x, a3 - (float)h23.y);
        const u32 H01 = __builtin_bit_cast(u32, h01), H23 = __builtin_bit_cast(u32, h23);
        const u32 L01 = __builtin_bit_cast(u32, l01), L23 = __builtin_bit_cast(u32, l23);
        const u32 r0 = swap1u(limb ? H01 : L01), r1 = swap1u(limb ? H23 : L23);
        const u4 w = limb ? (u4){r0, r1, L01, L23} : (u4){H01, H23, r0, r1};
        bx.a[J] = __builtin_bit_cast(h8, w);
    }
    // the unscale factors of positions 2g, 2g + 1 (lanes 4g and 4g + 2 hold them)
    const int g = lane >> 4;
    const float ua = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * (4 * g), __builtin_bit_cast(int, u24)));
    const float ub =
        __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * (4 * g + 2), __builtin_bit_cast(int, u24)));
    bx.u = (f2){ua, ub};
    if constexpr (T == T_Q4_K) {
        const u4 ones = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
        const float ka = ua * 0x1p-24f, kb = ub * 0x1p-24f;
        f4 D[8];
#pragma unroll
        for (int J = 0; J < 8; ++J)
            D[J] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bx.a[J], __builtin_bit_cast(h8, ones),
                                                          (f4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int c = 0; c < 4; ++c)
            bx.sx[c] = (f4){(D[2 * c][0] + D[2 * c][1]) * ka, (D[2 * c][2] + D[2 * c][3]) * kb,
                            (D[2 * c + 1][0] + D[2 * c + 1][1]) * ka, (D[2 * c + 1][2] + D[2 * c + 1][3]) * kb};
    }
}

// Lane (n, g)'s fields of its row's block from the item's LDS slot.
__device__ __forceinline__ void read_raw(Q4Raw &r, const char *slot, int n, int g, u32) {
    const char *row = slot + n * Geo<T_Q4_K>::RS;
    r.h = *reinterpret_cast<const u4 *>(row);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        r.q[2 * c] = *reinterpret_cast<const u32 *>(row + 16 + 32 * c + 4 * g);
        r.q[2 * c + 1] = *reinterpret_cast<const u32 *>(row + 32 + 32 * c + 4 * g);
    }
}
// A row's block starts `delta` bytes into its LDS row (delta even, possibly
// not a multiple of 4): each field is read as the two aligned dwords around
// it and realigned.  d (bytes 208-209) is the half of the dword at 208 that
// the block's alignment selects.
__device__ __forceinline__ void read_raw(Q6Raw &r, const char *slot, int n, int g, u32 delta) {
    const char *row = slot + n * Geo<T_Q6_K>::RS + (delta & ~3u);
    const u32 sh = delta & 3u;
    auto fld = [&](int off) {
        return realign(*reinterpret_cast<const u32 *>(row + off + 4), *reinterpret_cast<const u32 *>(row + off), sh);
    };
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
            const int base = 64 * hh + 16 * q2 + 4 * g;
            r.ql[(hh * 2 + q2) * 2] = fld(base);
            r.ql[(hh * 2 + q2) * 2 + 1] = fld(base + 32);
            r.qh[hh * 2 + q2] = fld(128 + 32 * hh + 16 * q2 + 4 * g);
        }
    r.sc = (u4){fld(192), fld(196), fld(200), fld(204)};
    r.dw = *reinterpret_cast<const u32 *>(row + 208) >> (8 * sh);
}

__device__ __forceinline__ f4 mma32(h8 a, u4 b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(h8, b), (f4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
}
__device__ __forceinline__ f4 mma16(h4 a, hf2 b0, hf2 b1) {
    const h4 b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3);
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, (f4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
}

// The block's contribution to positions 2g, 2g + 1 of lane n's row.
__device__ __forceinline__ f2 item_value(const Q4Raw &r, const BlkX &bx) {
    const u32 h0 = r.h.x, h1 = r.h.y, h2 = r.h.z, h3 = r.h.w;
    const float d = half_lo(h0), dmin = half_lo(h0 >> 16);
    const u32 sc_lo = h1 & 0x3F3F3F3Fu, m_lo = h2 & 0x3F3F3F3Fu;
    const u32 sc_hi = (h3 & 0x0F0F0F0Fu) | ((h1 >> 2) & 0x30303030u);
    const u32 m_hi = ((h3 >> 4) & 0x0F0F0F0Fu) | ((h2 >> 2) & 0x30303030u);
    float aq0 = 0.f, aq1 = 0.f, am0 = 0.f, am1 = 0.f;
#pragma unroll
    for (int J = 0; J < 8; ++J) {
        const u32 D0 = r.q[2 * (J >> 1)], D1 = r.q[2 * (J >> 1) + 1];
        const u32 msk = (J & 1) ? 0x00F000F0u : 0x000F000Fu;
        const u4 bw = {D0 & msk, (D0 >> 8) & msk, D1 & msk, (D1 >> 8) & msk};
        const f4 D = mma32(bx.a[J], bw);
        const u32 scw = J < 4 ? sc_lo : sc_hi, mw = J < 4 ? m_lo : m_hi;
        const float sc = (float)((scw >> (8 * (J & 3))) & 0xFFu), mn = (float)((mw >> (8 * (J & 3))) & 0xFFu);
        const float dsc = ((J & 1) ? d * 0.0625f : d) * sc;
        const float dm = dmin * mn;
        aq0 = __builtin_fmaf(dsc, D[0] + D[1], aq0);
        aq1 = __builtin_fmaf(dsc, D[2] + D[3], aq1);
        const f4 sxv = bx.sx[J >> 1];
        am0 = __builtin_fmaf(dm, (J & 1) ? sxv.z : sxv.x, am0);
        am1 = __builtin_fmaf(dm, (J & 1) ? sxv.w : sxv.y, am1);
    }
    return (f2){__builtin_fmaf(aq0, bx.u.x, -am0), __builtin_fmaf(aq1, bx.u.y, -am1)};
}

__device__ __forceinline__ f2 item_value(const Q6Raw &r, const BlkX &bx) {
    const float d = half_lo(r.dw);
    const hf2 off_lo = {(_Float16)(32.f / 16777216.f), (_Float16)(32.f / 16777216.f)};
    const hf2 off_hi = {(_Float16)(512.f / 16777216.f), (_Float16)(512.f / 16777216.f)};
    float aq0 = 0.f, aq1 = 0.f;
    // per half of the block: its 8 sub-blocks' products (independent
    // instructions back to back), then their scales
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        f4 D[8];
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
            const u32 A = r.ql[(hh * 2 + q2) * 2], B = r.ql[(hh * 2 + q2) * 2 + 1], H = r.qh[hh * 2 + q2];
            const u32 A8 = A >> 8, B8 = B >> 8;
            const u32 H4l = H << 4, H4r = H >> 4, H2l = H << 2, H6r = H >> 6;
            u32 w[4][2];
            w[0][0] = (A & 0x000F000Fu) | (H4l & 0x00300030u);
            w[0][1] = (A8 & 0x000F000Fu) | (H4r & 0x00300030u);
            w[1][0] = (B & 0x000F000Fu) | (H2l & 0x00300030u);
            w[1][1] = (B8 & 0x000F000Fu) | (H6r & 0x00300030u);
            w[2][0] = (A & 0x00F000F0u) | (H4l & 0x03000300u);
            w[2][1] = (A8 & 0x00F000F0u) | (H4r & 0x03000300u);
            w[3][0] = (B & 0x00F000F0u) | (H2l & 0x03000300u);
            w[3][1] = (B8 & 0x00F000F0u) | (H6r & 0x03000300u);
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                const hf2 off = gg < 2 ? off_lo : off_hi;
                const hf2 b0 = __builtin_bit_cast(hf2, w[gg][0]) - off;
                const hf2 b1 = __builtin_bit_cast(hf2, w[gg][1]) - off;
                const h8 a8 = bx.a[4 * hh + gg];
                const h4 a = q2 ? __builtin_shufflevector(a8, a8, 4, 5, 6, 7) : __builtin_shufflevector(a8, a8, 0, 1, 2, 3);
                D[2 * gg + q2] = mma16(a, b0, b1);
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int j16 = 8 * hh + j;   // scale index 8h + 2g + q2
            const u32 scw = r.sc[j16 >> 2];
            const float sc = (float)(int)(signed char)(scw >> (8 * (j16 & 3)));
            const float dsc = ((j >> 1) < 2 ? d : d * 0.0625f) * sc;
            aq0 = __builtin_fmaf(dsc, D[j][0] + D[j][1], aq0);
            aq1 = __builtin_fmaf(dsc, D[j][2] + D[j][3], aq1);
        }
    }
    return (f2){aq0 * bx.u.x, aq1 * bx.u.y};
}

// One work-group's share (work-group wg of the nwg that serve sg): TWC is the
// most tiles a work-group of the launch holds (the tile loop is unrolled that
// far).  smem: per wave D item slots and a block slot; at the end the sums.
template <int T, int TWC>
__device__ __forceinline__ void mc_body(const float *__restrict__ x, int K, int M, const McSegs &sg,
                                        int64_t row_bytes, int wg, int nwg, char *smem) {
    typedef Geo<T> G;
    typedef typename McRaw<T>::type Raw;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int n = lane & 15, g = lane >> 4;
    const int tiles = sg.tstart[sg.n];
    const int tw = wg < tiles ? (tiles - wg + nwg - 1) / nwg : 0;
    const int nb = K >> 8;
    const int nbw = wave < nb ? (nb - wave + 7) / 8 : 0;
    char *ring = smem + wave * (G::D * G::SLOT + BSLOT);
    char *bslot = ring + G::D * G::SLOT;
    const rsrc_t xr = make_rsrc(x, 4u * (u32)M * (u32)K);
    const TileTab tt = tile_tab(sg, row_bytes, wg, nwg, tw, lane);

    f2 acc[TWC];
#pragma unroll
    for (int i = 0; i < TWC; ++i) acc[i] = (f2){0.f, 0.f};

    // Every item issues the item D - 1 ahead (past the end: nothing read, the
    // same number of loads), so before computing an item at most (D - 1) NLD
    // later loads may be outstanding (loads complete in issue order; in a
    // block's first D - 1 items this also waits for part of the next block's
    // activations, issued in between -- counting those loads too measured no
    // faster); a block's operands were issued one block (tw items) before
    // they are read.
    int iti = 0, ibi = 0, islot = 0, cslot = 0;
    auto issue = [&]() {
        issue_item<T>(tt, row_bytes, iti, wave + 8 * ibi, ibi < nbw, ring + islot * G::SLOT, lane);
        if (++iti == tw) {
            iti = 0;
            ++ibi;
        }
        if (++islot == G::D) islot = 0;
    };
    issue_blk(xr, K, wave, nbw > 0, M, bslot, lane);
#pragma unroll
    for (int d = 0; d < G::D - 1; ++d) issue();
    for (int bi = 0; bi < nbw; ++bi) {
        // (the block's copy was followed by min(tw, D - 1) items' loads at least)
        if (tw >= G::D - 1)
            wait_vm<(G::D - 1) * G::NLD>();
        else if (tw >= 2)
            wait_vm<2 * G::NLD>();
        else
            wait_vm<G::NLD>();
        f4 xv[8];
        {
            const int p = (lane & 15) >> 1, limb = lane & 1, gg = lane >> 4;
#pragma unroll
            for (int J = 0; J < 8; ++J)
                xv[J] = *reinterpret_cast<const f4 *>(bslot + 1024 * p + 4 * (32 * J + 16 * limb + 4 * gg));
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        issue_blk(xr, K, wave + 8 * (bi + 1), bi + 1 < nbw, M, bslot, lane);
        BlkX cx;
        conv_blk<T>(cx, xv, lane);
        const int b = wave + 8 * bi;
#pragma unroll
        for (int ti = 0; ti < TWC; ++ti) {
            if (ti < tw) {
                // the slot refilled now held the previous item: its reads are done
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                issue();
                wait_vm<(G::D - 1) * G::NLD>();
                // (a tile's first row starts 16-byte aligned: 16 rows into a
                // 16-byte aligned matrix)
                const u32 delta = T == T_Q6_K ? ((u32)(n * row_bytes) + (u32)b * Fmt<T>::BYTES) & 15u : 0u;
                Raw r;
                read_raw(r, ring + cslot * G::SLOT, n, g, delta);
                if (++cslot == G::D) cslot = 0;
                acc[ti] += item_value(r, cx);
            }
        }
    }
    // every copy into LDS has landed before the slots are reused for the sums
    wait_vm<0>();
    __syncthreads();
    f2 *part = reinterpret_cast<f2 *>(smem);   // [tile][wave][lane]
#pragma unroll
    for (int ti = 0; ti < TWC; ++ti)
        if (ti < tw) part[(ti * 8 + wave) * 64 + lane] = acc[ti];
    __syncthreads();
    // per-tile sums of the eight waves, added in wave order
    for (int ti = wave; ti < tw; ti += 8) {
        f2 s = (f2){0.f, 0.f};
#pragma unroll
        for (int w = 0; w < 8; ++w) s += part[(ti * 8 + w) * 64 + lane];
        const int t = wg + ti * nwg;
        int sgi = 0;
#pragma unroll
        for (int i = 1; i < MAX_SEGS; ++i) sgi += (i < sg.n && t >= sg.tstart[i]) ? 1 : 0;
        const int row = (t - sg.tstart[sgi]) * 16 + n;
        if (row < sg.rows[sgi]) {
            float *y = sg.y[sgi];
            const int64_t rows = sg.rows[sgi];
            if (2 * g < M) y[(int64_t)(2 * g) * rows + row] = s.x;
            if (2 * g + 1 < M) y[(int64_t)(2 * g + 1) * rows + row] = s.y;
        }
    }
}

template <int T, int TWC>
__global__ __launch_bounds__(THREADS) void mc_kernel(const float *__restrict__ x, int K, int M, const McSegs sg,
                                                     int64_t row_bytes) {
    extern __shared__ __align__(16) char smem[];
    mc_body<T, TWC>(x, K, M, sg, row_bytes, blockIdx.x, gridDim.x, smem);
}

// Q4_K and Q6_K matrices in one launch (a layer's k and q beside v): the
// first gb work-groups serve the Q6_K tiles, the others the Q4_K tiles.
template <int TWA, int TWB>
__global__ __launch_bounds__(THREADS) void mc_mixed_kernel(const float *__restrict__ x, int K, int M,
                                                           const McSegs sa, int64_t rba, const McSegs sb,
                                                           int64_t rbb, int gb) {
    extern __shared__ __align__(16) char smem[];
    if ((int)blockIdx.x < gb)
        mc_body<T_Q6_K, TWB>(x, K, M, sb, rbb, blockIdx.x, gb, smem);
    else
        mc_body<T_Q4_K, TWA>(x, K, M, sa, rba, blockIdx.x - gb, gridDim.x - gb, smem);
}

template <int T> constexpr size_t ring_lds() { return (size_t)8 * (Geo<T>::D * Geo<T>::SLOT + BSLOT); }

// The split of the grid between the Q6_K (gb work-groups) and Q4_K tiles for
// which the slowest work-group finishes first; a Q6_K tile is taken to cost
// 1.8 Q4_K tiles (its bytes and its slower unpack).  0: none fits.
inline int mixed_split(int64_t ta, int64_t tb, int G, int64_t *twa, int64_t *twb) {
    int best = 0;
    double bc = 0;
    for (int gb = 1; gb < G; ++gb) {
        if (gb > tb || G - gb > ta) continue;
        const int64_t b = (tb + gb - 1) / gb, a = (ta + G - gb - 1) / (G - gb);
        if (a > TW_MAX || b > TW_MAX) continue;
        const double c = std::max(1.8 * (double)b, (double)a);
        if (!best || c < bc) {
            best = gb;
            bc = c;
            *twa = a;
            *twb = b;
        }
    }
    return best;
}

template <int TWA, int TWB>
int launch_mixed_tw(const McSegs &sa, int64_t rba, const McSegs &sb, int64_t rbb, int K, int M, const float *x,
                    int gb, int G, size_t lds, hipStream_t st) {
    auto kern = mc_mixed_kernel<TWA, TWB>;
    if (allow_lds(kern, lds) != hipSuccess) return KQ_ERR_LAUNCH;
    hipLaunchKernelGGL(kern, dim3((unsigned)G), dim3(THREADS), lds, st, x, K, M, sa, rba, sb, rbb, gb);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_LAUNCH;
}

// KQ_ERR_ARG when the two do not share one launch well (then separately).
inline int launch_mc_mixed(const McSegs &sa, int64_t rba, const McSegs &sb, int64_t rbb, int K, int M,
                           const float *x, hipStream_t st) {
    const int G = cu_count();
    int64_t twa = 0, twb = 0;
    const int gb = mixed_split(sa.tstart[sa.n], sb.tstart[sb.n], G, &twa, &twb);
    if (!gb) return KQ_ERR_ARG;
    const size_t lds = std::max({ring_lds<T_Q4_K>(), ring_lds<T_Q6_K>(), (size_t)std::max(twa, twb) * 8 * 64 * sizeof(f2)});
    if (twa <= 4)
        return twb <= 2 ? launch_mixed_tw<4, 2>(sa, rba, sb, rbb, K, M, x, gb, G, lds, st)
                        : launch_mixed_tw<4, TW_MAX>(sa, rba, sb, rbb, K, M, x, gb, G, lds, st);
    return twb <= 2 ? launch_mixed_tw<TW_MAX, 2>(sa, rba, sb, rbb, K, M, x, gb, G, lds, st)
                    : launch_mixed_tw<TW_MAX, TW_MAX>(sa, rba, sb, rbb, K, M, x, gb, G, lds, st);
}

template <int T>
int launch_mc(const McSegs &sg, int64_t row_bytes, int K, int M, const float *x, hipStream_t st) {
    const int64_t tiles = sg.tstart[sg.n];
    if (tiles == 0) return KQ_OK;
    int64_t nwg = std::min<int64_t>(tiles, cu_count());
    nwg = std::max<int64_t>(nwg, (tiles + TW_MAX - 1) / TW_MAX);
    const int64_t tw = (tiles + nwg - 1) / nwg;
    const size_t lds = std::max<size_t>(ring_lds<T>(), (size_t)tw * 8 * 64 * sizeof(f2));
    auto run = [&](auto kern) {
        if (allow_lds(kern, lds) != hipSuccess) return KQ_ERR_LAUNCH;
        hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(THREADS), lds, st, x, K, M, sg, row_bytes);
        return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_LAUNCH;
    };
    if (tw <= 2) return run(mc_kernel<T, 2>);
    if (tw <= 4) return run(mc_kernel<T, 4>);
    if (tw <= 8) return run(mc_kernel<T, 8>);
    return run(mc_kernel<T, TW_MAX>);
}

} // namespace mc

// The grouped matrix-core GEMV once its arguments are checked: one
// preparation launch for x, then the matrices: Q4_K and Q6_K ones together in
// one launch when each format has at most 8 and the grid splits well between
// them, otherwise one launch per format and up to 8 matrices.
int mc_run(int count, const int *types, const void *const *W, const int64_t *N, int K, const float *x, int M,
           float *const *y, hipStream_t st) {
    std::vector<int> by[2];
    for (int i = 0; i < count; ++i) {
        if (N[i] == 0) continue;
        by[types[i] == KQ_TYPE_Q4_K ? 0 : 1].push_back(i);
    }
    const int64_t rb[2] = {kq_row_bytes_(KQ_TYPE_Q4_K, K), kq_row_bytes_(KQ_TYPE_Q6_K, K)};
    auto segs = [&](int f, size_t from, size_t to) {
        mc::McSegs sg = {};
        for (size_t j = from; j < to; ++j) {
            const int i = by[f][j];
            sg.W[sg.n] = static_cast<const uint8_t *>(W[i]);
            sg.y[sg.n] = y[i];
            sg.rows[sg.n] = (int)N[i];
            sg.tstart[sg.n + 1] = sg.tstart[sg.n] + (int)((N[i] + 15) / 16);
            ++sg.n;
        }
        return sg;
    };
    if (!by[0].empty() && !by[1].empty() && by[0].size() <= (size_t)MAX_SEGS && by[1].size() <= (size_t)MAX_SEGS) {
        const int r = mc::launch_mc_mixed(segs(0, 0, by[0].size()), rb[0], segs(1, 0, by[1].size()), rb[1], K, M,
                                          x, st);
        if (r != KQ_ERR_ARG) return r;
    }
    for (int f = 0; f < 2; ++f)
        for (size_t j = 0; j < by[f].size(); j += MAX_SEGS) {
            const mc::McSegs sg = segs(f, j, std::min(by[f].size(), j + MAX_SEGS));
            const int r = f == 0 ? mc::launch_mc<T_Q4_K>(sg, rb[0], K, M, x, st)
                                 : mc::launch_mc<T_Q6_K>(sg, rb[1], K, M, x, st);
            if (r) return r;
        }
    return KQ_OK;
}

} // namespace kq
