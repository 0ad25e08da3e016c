/*
 * kqstream.h -- host-streamed GEMV in libkqgemv.so: weights that live in host
 * memory are copied through a ring of device slots, each copy overlapping the
 * GEMV of the previous slot.
 *
 * What it computes.  The Kortex summary ("Kortex: Out-of-core LLM inference
 * engine written from scratch in Rust", section Approach) streams layer
 * weights that do not fit in device memory through a ring of VRAM slots while
 * the GPU computes the layers already copied; the RunNburn post pulls the
 * selected experts' weights on demand.  Each call here is one step of such a
 * schedule: the matrices of one group (sharing K and x) are copied from host
 * memory into the next slot of the ring on a copy stream, and the same grouped
 * GEMV as kq_qgemv_multi then runs on the caller's stream once the copy has
 * landed.  The results are bit-identical to kq_qgemv_multi on device-resident
 * copies of the same bytes.
 *
 * Ordering.  Copy i waits (on the copy stream) until the GEMV that last read
 * its slot has finished; GEMV i waits (on the caller's stream) for copy i.
 * With nslots >= 2, the copy of the next group overlaps the GEMV of this one.
 * The host source must be page-locked (hipHostMalloc, or a pinned torch
 * tensor) for the copy to be asynchronous; pageable memory works but the
 * runtime then copies it synchronously.  The bound is the host-to-device link,
 * not HBM.
 *
 * Ownership.  The slots are device memory owned by the caller (`slots`:
 * nslots * slot_bytes bytes, 256-B aligned); the streamer owns a copy stream
 * and two events per slot.  A streamer is used from one host thread at a time.
 * The host buffers of a call must stay valid and unchanged until its copy has
 * run (kq_streamer_sync waits for every copy issued so far).
 */
#ifndef KQSTREAM_H
#define KQSTREAM_H

#include <stddef.h>
#include <stdint.h>

#include "kqgemv.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kq_streamer kq_streamer;

/* A ring of nslots (1..64) slots of slot_bytes (a positive multiple of 256)
 * each, at the device address `slots` (256-B aligned), serving GEMVs issued on
 * `stream` (hipStream_t as void*; NULL = null stream).  Returns KQ_OK,
 * KQ_ERR_NULL, KQ_ERR_ALIGN, KQ_ERR_ARG (nslots or slot_bytes out of range)
 * or KQ_ERR_LAUNCH (stream or event creation failed). */
int kq_streamer_create(void *slots, size_t slot_bytes, int nslots, void *stream, kq_streamer **out);

/* Waits for the work the streamer issued, then frees its stream and events.
 * NULL is a no-op. */
void kq_streamer_destroy(kq_streamer *s);

/* Blocks until every copy issued so far has completed (the host buffers may
 * then be reused).  KQ_ERR_LAUNCH if the runtime reports an error. */
int kq_streamer_sync(kq_streamer *s);

/* y[i] = W[i] . x for the `count` matrices of one group (arguments as for
 * kq_qgemv_multi, except that W[i] are HOST addresses of N[i] rows of types[i]
 * blocks).  The matrices are placed one after the other in the next slot, each
 * at a 256-B boundary; their total must fit in slot_bytes (KQ_ERR_SHAPE
 * otherwise).  Every argument is checked before anything is issued. */
int kq_stream_qgemv_multi(kq_streamer *s, int count, const int *types, const void *const *W,
                          const int64_t *N, int64_t K, const float *x, int M, float *const *y);

/* One matrix: kq_stream_qgemv_multi with count = 1. */
int kq_stream_qgemv(kq_streamer *s, int type, const void *W, int64_t N, int64_t K, const float *x, int M,
                    float *y);

#ifdef __cplusplus
}
#endif

#endif /* KQSTREAM_H */
