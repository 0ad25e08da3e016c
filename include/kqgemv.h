/*
 * kqgemv.h -- C ABI of the fused GGUF K-quant dequant-GEMV library for AMD
 * Instinct MI355X (gfx950).
 *
 * What the calls compute.  Decode-time LLM engines spend their time streaming
 * quantized weights through a matrix-vector product; the weights are expanded
 * to real values only inside the product, in registers, never written back
 * (Kortex: "Out-of-core LLM inference engine written from scratch in Rust",
 * section Approach, and "Kortex: Streaming 70B Models on Consumer GPUs",
 * section Key components, item 3).  The block formats are the GGUF K-quants
 * the RunNburn post lists native kernels for ("RunNburn - Run a 295B Moe from
 * a 98GB GGUF on a 64GB RAM Desktop"): Q2_K, Q3_K, Q4_K, Q5_K, Q6_K, Q4_0 and
 * Q8_0.  A
 * speculative-verify pass runs several positions through one pass of the
 * weights (Kortex summary, section Approach): here M <= 8 activation rows.  The
 * MoE variant applies the experts each token selected (the RunNburn post).
 *
 * Block formats (GGUF convention; the pages name the formats but print no
 * layout, so this is a reading):
 *   Q4_K  256 weights / 144 B   w = d*sc*q - dmin*m   (6-bit sc, m per 32)
 *   Q6_K  256 weights / 210 B   w = d*sc*(q - 32)     (int8 sc per 16)
 *   Q2_K  256 weights /  84 B   w = d*sc*q - dmin*m   (4-bit sc, m per 16)
 *   Q8_0   32 weights /  34 B   w = d*q
 *   Q4_0   32 weights /  18 B   w = d*(q - 8)        (4-bit q)
 *   Q5_K  256 weights / 176 B   w = d*sc*q - dmin*m   (5-bit q, Q4_K's scales)
 *   Q3_K  256 weights / 110 B   w = d*(sc - 32)*q     (q in -4..3, 6-bit sc per 16)
 * d and dmin are IEEE fp16 (subnormals honoured).  A weight matrix W of N rows
 * and K columns is N consecutive rows of K/QK blocks each (K fastest).  MoE
 * expert tensors are E such matrices back to back.
 *
 * Conventions shared by every call:
 *  - All data pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or synchronises.  Outputs are overwritten, never
 *    accumulated.
 *  - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *    Every call is asynchronous on that stream.
 *  - Argument errors are returned synchronously as a negative kq_status before
 *    any HIP call is made.  A call that would launch on a device other than a
 *    gfx950 returns KQ_ERR_DEVICE.  A failed launch returns KQ_ERR_LAUNCH.
 *    Faults in a kernel surface at the caller's next synchronisation.
 *  - The library holds no per-call state (only caches of each device's compute
 *    unit count and of the LDS limits granted to its kernels); calls are
 *    reentrant and thread-safe.
 *  - Alignment: W, W_exps and src 16 B; x, y, dst, workspace 16 B; ids,
 *    route_w, err_flag 4 B.  Rows of Q6_K, Q3_K, Q8_0 and Q4_0 matrices may
 *    start at any even byte offset (e.g. 630-byte rows); that is handled
 *    inside.
 */
#ifndef KQGEMV_H
#define KQGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* GGUF tensor type ids of the supported block formats. */
typedef enum kq_type {
    KQ_TYPE_Q4_0 = 2,
    KQ_TYPE_Q8_0 = 8,
    KQ_TYPE_Q2_K = 10,
    KQ_TYPE_Q3_K = 11,
    KQ_TYPE_Q4_K = 12,
    KQ_TYPE_Q5_K = 13,
    KQ_TYPE_Q6_K = 14
} kq_type;

typedef enum kq_status {
    KQ_OK = 0,
    KQ_ERR_TYPE = -1,     /* unknown or unsupported quant type              */
    KQ_ERR_SHAPE = -2,    /* K not a positive multiple of the block size,
                             N < 0, or a size beyond the documented limits   */
    KQ_ERR_M = -3,        /* M (or T) outside 1..8                          */
    KQ_ERR_NULL = -4,     /* a required pointer is NULL                     */
    KQ_ERR_ALIGN = -5,    /* a pointer violates its alignment requirement   */
    KQ_ERR_ARG = -6,      /* any other invalid argument (x_mode, k, E)      */
    KQ_ERR_LAUNCH = -7,   /* the HIP launch itself failed                   */
    KQ_ERR_DEVICE = -8,   /* the current device is not a gfx950 (checked once
                             per device by the first call that would launch) */
    KQ_ERR_IO = -9,       /* a file could not be opened or mapped (kqgguf.h) */
    KQ_ERR_FORMAT = -10   /* a malformed or unsupported file (kqgguf.h)     */
} kq_status;

/* Library version, major*10000 + minor*100 + patch. */
int kq_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char *kq_status_string(int status);

/* Weights per block and bytes per block of `type`.  Returns KQ_OK or
 * KQ_ERR_TYPE / KQ_ERR_NULL.  Host-only, no HIP call. */
int kq_block_info(int type, int *block_elems, int *block_bytes);

/* Bytes of one row of K weights of `type`, or a negative kq_status when K is
 * not a positive multiple of the block size.  Host-only, no HIP call. */
int64_t kq_row_bytes(int type, int64_t K);

/* Standalone dequantization: dst[i] = fp32 weight i of the packed blocks at
 * src, for i in [0, n_elems).  This is the expansion the fused GEMV below
 * does only in registers (Kortex article, section Key components, item 3),
 * written out to memory: for checking the formats and for callers that need
 * dense weights.  n_elems must be a multiple of the block size (0 is allowed
 * and launches nothing).  Every value is the correctly rounded fp32 of the
 * exact weight (the products are exact, one rounding at the final
 * subtraction); an exact zero is written as +0.  src: n_elems/QK blocks. */
int kq_dequant(int type, const void *src, int64_t n_elems, float *dst, void *stream);

/* Fused dequant-GEMV: y[m][o] = sum_i w[o][i] * x[m][i] for m < M, o < N --
 * the decode-time matrix-vector product over quantized weights that the
 * Kortex summary ("Out-of-core LLM inference engine written from scratch in
 * Rust", section Approach) runs in fused dequant-matmul kernels; M > 1 rows
 * are the several positions one speculative-verify pass runs through the
 * weights (same section).
 *   W  N x K matrix of `type` blocks (row-major, K fastest), 16-B aligned.
 *   x  M rows of K fp32, contiguous (row stride K).
 *   y  M rows of N fp32, contiguous (row stride N), overwritten.
 * 1 <= M <= 8; K a positive multiple of the block size, K <= 2^20;
 * 0 <= N < 2^31 (N == 0 launches nothing).  The weights are expanded only in
 * registers.  Accumulation is fp32; for every output the error against the
 * exact sum is far below 1e-4 * sum_i |w*x| + 1e-6.  Row m of the result does
 * not depend on M or on the other rows of x (bit-identical to an M = 1 call on
 * that row), and reruns are bit-identical (no atomics). */
int kq_qgemv(int type, const void *W, int64_t N, int64_t K,
             const float *x, int M, float *y, void *stream);

/* Grouped fused dequant-GEMV: the `count` products y[i] = W[i] . x of
 * matrices that share K and the activations (a layer's q, k and v
 * projections, or its gate and up projections), served by as few launches as
 * possible: at M == 1, up to 8 matrices of one format per launch, and two
 * K-quant formats (Q2_K..Q6_K) together in one launch (their rows have
 * the same number of units); at M > 1, up to 8 matrices of one format per
 * launch.  The fused kernels of the Kortex pages ("Out-of-core LLM inference
 * engine written from scratch in Rust", section Approach) run one layer's
 * projections in one pass; this is that grouping for matrices with the same
 * input.
 *   types  host array of `count` kq_type values, one per matrix.
 *   W      host array of `count` device pointers; matrix i has N[i] rows of
 *          types[i] blocks (layout and alignment as for kq_qgemv).
 *   N      host array of `count` row counts (0 allowed: that matrix is skipped).
 *   x      M rows of K fp32 shared by every matrix.
 *   y      host array of `count` device pointers, y[i] is M rows of N[i] fp32.
 * count >= 0 (0 launches nothing).  Every argument is checked before anything
 * is launched; the limits are those of kq_qgemv (K must suit every type).
 * Each y[i] is bit-identical to kq_qgemv(types[i], W[i], N[i], K, x, M, y[i],
 * stream).  The y[i] must not overlap each other or any W[i] or x. */
int kq_qgemv_multi(int count, const int *types, const void *const *W,
                   const int64_t *N, int64_t K, const float *x, int M,
                   float *const *y, void *stream);

/* Matrix-core fused dequant-GEMV for the few positions of a speculative-verify
 * pass (Kortex summary, "Out-of-core LLM inference engine written from scratch
 * in Rust", section Approach: several positions run through the weights in one
 * pass), for Q4_K and Q6_K matrices: the products and sums go to the 16x16
 * f16 matrix instructions, the vector unit only unpacks quants, splits the
 * activations and applies scales, so the cost per weight hardly grows with M
 * (at 70B shapes 1.06x as fast as kq_qgemv_multi at M = 2, 2.6x at M = 8).
 * Same operation, arguments and limits as kq_qgemv_multi; types must be
 * KQ_TYPE_Q4_K or KQ_TYPE_Q6_K (else KQ_ERR_TYPE).  Every argument is checked
 * before anything is launched.  Accuracy: every output is within
 * 1e-4 * sum_i |w*x| + 1e-6 of the exact sum for finite x with |x| < 2^116
 * (activations enter as two fp16 limbs, about 21 bits, scaled per 256
 * columns; products and sums in fp32).  Row m of the result does not depend
 * on M or on the other rows of x, and reruns are bit-identical, but the
 * summation order is not that of kq_qgemv: results are not bit-identical to
 * kq_qgemv's.  Q4_K and Q6_K matrices (up to 8 of each) share one launch when
 * the grid splits well between them, else one launch per format and up to 8
 * matrices. */
int kq_qgemv_mc_multi(int count, const int *types, const void *const *W,
                      const int64_t *N, int64_t K, const float *x, int M,
                      float *const *y, void *stream);

/* kq_qgemv_mc_multi for one matrix. */
int kq_qgemv_mc(int type, const void *W, int64_t N, int64_t K, const float *x,
                int M, float *y, void *stream);

/* Workspace bytes kq_qmoe_gemv needs for T tokens, k slots and N rows when a
 * routing-weighted combine is requested (T*k*N*4); 0 on invalid sizes. */
size_t kq_qmoe_workspace_bytes(int T, int k, int64_t N);

/* Routed-expert GEMV over a stacked expert tensor: only the experts each
 * token selected are read (the RunNburn post: only a token's chosen experts
 * are fetched, and the router's choices are not altered).
 *   W_exps  E matrices of N x K `type` blocks, expert-major, 16-B aligned.
 *   ids     [T][k] int32 expert ids (device memory; never read by the host).
 *   x       x_mode 0: [T][K] fp32, one activation row per token, shared by
 *           its k slots (gate/up projections); x_mode 1: [T][k][K], one row
 *           per slot (down projection).
 *   route_w NULL: y is [T][k][N], y[t][j] = W_exps[ids[t][j]] . x_(t,j).
 *           non-NULL: [T][k] fp32 routing weights, y is [T][N],
 *           y[t] = sum_j route_w[t][j] * W_exps[ids[t][j]] . x_(t,j), summed
 *           in ascending j, one fused multiply-add per term starting from
 *           +0; `workspace` must then hold kq_qmoe_workspace_bytes(T, k, N)
 *           bytes (its contents are scratch).  When a token's activation
 *           rows fit the kernel's LDS budget (below) the products and the sum
 *           run in one launch and the workspace is not touched; otherwise the
 *           per-slot results go through the workspace to a second launch.
 *           Either way the result has the same bits.
 *   err_flag NULL or a device int32 the kernel sets to 1 (plain store) when
 *           an id is outside [0, E); such a slot contributes zero.  It is
 *           never cleared by the library.
 * 1 <= T <= 8, 1 <= k <= 16, k <= E.  When a token's activation rows (k rows
 * with x_mode 1, one with x_mode 0) and, with route_w, the per-slot sums of a
 * row tile fit the kernel's 64 KB LDS budget (about 14,000 activations: k = 16
 * rows of K = 768, or one row of K = 12288), each token's slots are served
 * together, an expert routed to several tokens being read once per token;
 * otherwise slots that route to the same expert are served by one pass over
 * that expert's weights (up to 8 slots per pass).
 * Results per slot are bit-identical to kq_qgemv with M = 1 on the expert's
 * matrix and that slot's activation row. */
int kq_qmoe_gemv(int type, const void *W_exps, int64_t E, int64_t N, int64_t K,
                 const int32_t *ids, const float *route_w, int T, int k,
                 const float *x, int x_mode, float *y, float *workspace,
                 int32_t *err_flag, void *stream);

/* Scratch bytes kq_qmoe_gemv_noalloc holds per device (4 MiB). */
#define KQ_NOALLOC_SCRATCH_BYTES (4u << 20)

/* kq_qmoe_gemv without the workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Arguments, results and errors are those
 * of kq_qmoe_gemv; when a routing-weighted sum needs per-slot scratch it
 * uses a static device array of KQ_NOALLOC_SCRATCH_BYTES that the library
 * holds on every device it runs on until the process ends (its address is
 * looked up on the first call on a device: KQ_ERR_DEVICE if that fails).
 * With route_w non-NULL, T*k*N*4 (kq_qmoe_workspace_bytes) above that size
 * is refused with KQ_ERR_SHAPE before any HIP call.  The call allocates and
 * frees nothing.  Every call on a device shares that device's array and
 * overwrites what it uses before reading it; calls that overlap on one device
 * (other streams or host threads) race on it and must be serialised by the
 * caller. */
int kq_qmoe_gemv_noalloc(int type, const void *W_exps, int64_t E, int64_t N, int64_t K,
                         const int32_t *ids, const float *route_w, int T, int k,
                         const float *x, int x_mode, float *y, int32_t *err_flag, void *stream);

/* Grouped routed-expert GEMV: `count` (1..4) stacked expert tensors of one
 * format and shape that share the routing and the activations -- an MoE
 * layer's gate and up projections -- in one launch, per-slot outputs only:
 *   y[i][t][j] = W_exps[i][ids[t][j]] . x_(t,j)   (layouts as kq_qmoe_gemv).
 *   W_exps, y: host arrays of `count` device pointers (16-B aligned).
 * The fused projections of the Kortex pages ("Out-of-core LLM inference engine
 * written from scratch in Rust", section Approach) run a layer's matrices in
 * one pass; this is that grouping for the experts a token selected (the
 * RunNburn post).  Limits and errors as for kq_qmoe_gemv; each y[i] is
 * bit-identical to kq_qmoe_gemv(type, W_exps[i], ..., route_w = NULL, ...). */
int kq_qmoe_gemv_multi(int count, int type, const void *const *W_exps, int64_t E, int64_t N, int64_t K,
                       const int32_t *ids, int T, int k, const float *x, int x_mode, float *const *y,
                       int32_t *err_flag, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KQGEMV_H */
