/*
 * kqprobe.h -- measurement kernels beside the dequant-GEMV library (not part
 * of its computation): the ceilings and fixed costs its kernels are judged
 * against on MI355X (gfx950).
 *
 * Token generation is bound by memory bandwidth, not compute (Kortex:
 * "Kortex: Streaming 70B Models on Consumer GPUs", the paragraph before
 * Table 1), so the GEMV kernels are measured against how fast this GPU can
 * read HBM at all.  These calls give that number for the load forms the
 * kernels use, the floor of one kernel launch, and what a grid-wide barrier
 * between dependent phases of one persistent launch costs compared with a
 * launch per phase.
 *
 * Conventions: device pointers owned by the caller; `stream` is a hipStream_t
 * as void* (NULL: the null stream); calls are asynchronous and return 0 or a
 * negative kq_status (kqgemv.h) -- argument errors before any HIP call,
 * KQ_ERR_LAUNCH when a launch fails.  Nothing is allocated.
 */
#ifndef KQPROBE_H
#define KQPROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` of src once, in spans of 3 KB (a Q4_K batch-1 row step's
 * bytes, rounded up to whole 1-KB requests) dealt out round robin to the
 * `waves` waves of `nwg` persistent work-groups, each wave keeping `depth`
 * spans in flight.
 *   mode 0: 16-byte non-temporal loads into registers;
 *   mode 1: buffer-to-LDS loads of 16 bytes a lane (one 1-KB request per
 *           instruction), non-temporal, into a per-wave LDS ring.
 * sink: nwg * waves * 64 uint32 (each lane's XOR of what it read, so the loads
 * are not optimised away).  src and sink 16-B aligned; bytes a multiple of 16,
 * at most 4 GiB - 4 KiB; 1 <= nwg <= 65535, waves in {4, 8, 16}, depth in
 * 1..4 (mode 1: waves * depth * 3 KB <= 160 KB). */
int kqp_read_stream(const void *src, uint64_t bytes, int mode, int nwg, int waves, int depth, uint32_t *sink,
                    void *stream);

/* An empty kernel of nwg work-groups of `threads` threads (64..1024). */
int kqp_empty(int nwg, int threads, void *stream);

/* `nphases` dependent phases, each reading `phase_bytes` at
 * src + p * phase_stride as kqp_read_stream mode 1 does (16 waves, ring of 2),
 * after reading an `xbytes` slice (the activations a GEMV phase stages) at
 * x into LDS.
 *   persistent 1: one cooperative launch of nwg = compute units work-groups
 *     with a grid-wide barrier between phases (an atomic arrival count);
 *     prefetch bit 0: each work-group issues the next phase's first ring
 *     loads before it waits at the barrier (the weights do not depend on the
 *     previous phase); bit 1: no cache maintenance at the barrier (the
 *     activations are read at device scope) instead of an agent-scope
 *     release and acquire by every work-group.  ctr: 2 uint32 of device
 *     memory; ctr[0] is 0 on entry and 0 again when the kernel ends.  A wait
 *     longer than ~0.2 s gives up and sets ctr[1] to a nonzero value (the
 *     caller clears it).
 *   persistent 0: one ordinary launch per phase (ctr unused, may be NULL).
 * phase_bytes a multiple of 16, at most 4 GiB - 4 KiB; xbytes a multiple of
 * 16, at most 48 KiB; nphases >= 1. */
int kqp_phased_stream(const void *src, uint64_t phase_stride, uint64_t phase_bytes, int nphases, const float *x,
                      int xbytes, int persistent, int prefetch, uint32_t *ctr, uint32_t *sink, void *stream);

/* One wave of the 4x4x4 (16 blocks) f16 matrix instruction,
 * D = A . B + C: lane l passes a[4l..4l+3], b[4l..4l+3] (fp16) and
 * c[4l..4l+3] (fp32) and receives d[4l..4l+3] -- for reading the
 * instruction's lane layout and rounding on the host.  a, b: 256 halves,
 * 8-B aligned; c, d: 256 floats, 16-B aligned. */
int kqp_mfma4(const void *a, const void *b, const float *c, float *d, void *stream);

/* The 16x16x32 (k32 != 0) or 16x16x16 (k32 == 0) f16 matrix instruction on
 * one wave: lane l passes a[l] (8 halves; the first 4 for 16x16x16), b[l]
 * likewise and c[l] (4 floats), and receives d[l] (4 floats).  a, b: 64 x 8
 * fp16; c, d: 64 x 4 fp32; all 16-byte aligned device memory. */
int kqp_mfma16(const void *a, const void *b, const float *c, float *d, int k32, void *stream);

/* Issue rate of the same instruction: nwg work-groups of `waves` waves, each
 * wave `chains` (1, 2, 4 or 8) independent accumulators advanced `iters`
 * times.  sink: nwg * waves * 64 uint32. */
int kqp_mfma4_rate(int nwg, int waves, int chains, int iters, uint32_t *sink, void *stream);

/* The batch-1 GEMV of `count` matrices of `type` (KQ_TYPE_Q4_K or
 * KQ_TYPE_Q6_K) sharing x (kq_qgemv_multi at M = 1, K a multiple of 256 with
 * rows of at least 64 units), run by the library's persistent batch-1 kernel
 * for that format (Q4_K: the weight ring in LDS; Q6_K: the register ring) in
 * the library's launch shape, with timestamps: for each work-group
 * g < *groups, stamps[8 g + 0..3] are the 100 MHz constant-clock times at
 * which its first wave started, finished staging the activations, held its
 * unit's activations in registers (Q6_K: the same as the previous, the load
 * is part of its pass), and (all waves) finished; stamps[8 g + 4] its XCD,
 * stamps[8 g + 5] its hardware id register.  y[i] receives the products (the
 * same bits as kq_qgemv_multi).  stamps: max_groups * 8 uint64 of device
 * memory; *groups (host) is set to the grid size.  KQ_ERR_SHAPE for shapes the
 * library does not serve with those kernels; KQ_ERR_ARG for another type or
 * when the grid exceeds max_groups. */
int kqp_stamped_qgemv1(int type, int count, const void *const *W, const int64_t *N, int64_t K, const float *x,
                       float *const *y, uint64_t *stamps, int max_groups, int *groups, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KQPROBE_H */
