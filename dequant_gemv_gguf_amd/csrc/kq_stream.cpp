// kq_stream.cpp -- host-streamed GEMV of libkqgemv.so (C ABI in
// include/kqstream.h): a ring of caller-owned device slots; the matrices of a
// call are copied from host memory into the next slot on the streamer's copy
// stream, and the grouped GEMV runs on the caller's stream once they have
// landed (the Kortex summary, section Approach: weights move through a ring of
// VRAM slots while the GPU computes the layers already there).
#include <hip/hip_runtime_api.h>

#include <stdint.h>

#include <new>

#include "kqstream.h"

extern "C" int kq_multi_check(int count, const int *types, const void *const *W, const int64_t *N, int64_t K,
                              const float *x, int M, float *const *y);

namespace {

constexpr int MAX_SLOTS = 64;
constexpr int MAX_COUNT = 64;                // matrices per call
constexpr uint64_t SLOT_ALIGN = 256;

} // namespace

struct kq_streamer {
    uint8_t *slots = nullptr;
    size_t slot_bytes = 0;
    int nslots = 0;
    hipStream_t stream = nullptr;   // the caller's (GEMV) stream
    hipStream_t copy = nullptr;     // the streamer's copy stream
    hipEvent_t copied[MAX_SLOTS] = {};
    hipEvent_t freed[MAX_SLOTS] = {};
    bool used[MAX_SLOTS] = {};
    int next = 0;
};

extern "C" {

void kq_streamer_destroy(kq_streamer *s) {
    if (!s) return;
    // nothing to report at teardown: wait for the streamer's work, then free
    if (s->copy) (void)hipStreamSynchronize(s->copy);
    for (int i = 0; i < MAX_SLOTS; ++i) {
        if (s->freed[i]) {
            (void)hipEventSynchronize(s->freed[i]);
            (void)hipEventDestroy(s->freed[i]);
        }
        if (s->copied[i]) (void)hipEventDestroy(s->copied[i]);
    }
    if (s->copy) (void)hipStreamDestroy(s->copy);
    delete s;
}

int kq_streamer_create(void *slots, size_t slot_bytes, int nslots, void *stream, kq_streamer **out) {
    if (!out) return KQ_ERR_NULL;
    *out = nullptr;
    if (!slots) return KQ_ERR_NULL;
    if (((uintptr_t)slots & (SLOT_ALIGN - 1)) != 0) return KQ_ERR_ALIGN;
    if (nslots < 1 || nslots > MAX_SLOTS || slot_bytes == 0 || slot_bytes % SLOT_ALIGN != 0) return KQ_ERR_ARG;
    kq_streamer *s = new (std::nothrow) kq_streamer;
    if (!s) return KQ_ERR_LAUNCH;
    s->slots = (uint8_t *)slots;
    s->slot_bytes = slot_bytes;
    s->nslots = nslots;
    s->stream = (hipStream_t)stream;
    bool ok = hipStreamCreateWithFlags(&s->copy, hipStreamNonBlocking) == hipSuccess;
    for (int i = 0; ok && i < nslots; ++i) {
        ok = hipEventCreateWithFlags(&s->copied[i], hipEventDisableTiming) == hipSuccess &&
             hipEventCreateWithFlags(&s->freed[i], hipEventDisableTiming) == hipSuccess;
    }
    if (!ok) {
        kq_streamer_destroy(s);
        return KQ_ERR_LAUNCH;
    }
    *out = s;
    return KQ_OK;
}

int kq_streamer_sync(kq_streamer *s) {
    if (!s) return KQ_ERR_NULL;
    return hipStreamSynchronize(s->copy) == hipSuccess ? KQ_OK : KQ_ERR_LAUNCH;
}

int kq_stream_qgemv_multi(kq_streamer *s, int count, const int *types, const void *const *W, const int64_t *N,
                          int64_t K, const float *x, int M, float *const *y) {
    if (!s) return KQ_ERR_NULL;
    if (count < 0 || count > MAX_COUNT) return KQ_ERR_ARG;
    if (count == 0) return KQ_OK;
    if (!types || !W || !N || !y) return KQ_ERR_NULL;
    // place the matrices in the next slot, then check every argument as the
    // grouped call will, on the slot addresses, before anything is issued
    const int slot = s->next;
    uint8_t *base = s->slots + (size_t)slot * s->slot_bytes;
    const void *dev[MAX_COUNT];
    uint64_t bytes[MAX_COUNT];
    uint64_t at = 0;
    for (int i = 0; i < count; ++i) {
        const int64_t rb = kq_row_bytes(types[i], K);
        if (rb < 0) return (int)rb;
        if (N[i] < 0 || N[i] >= ((int64_t)1 << 31)) return KQ_ERR_SHAPE;
        bytes[i] = (uint64_t)N[i] * (uint64_t)rb;
        at = (at + SLOT_ALIGN - 1) / SLOT_ALIGN * SLOT_ALIGN;
        dev[i] = base + at;
        if (bytes[i] && !W[i]) return KQ_ERR_NULL;
        at += bytes[i];
        if (at > s->slot_bytes) return KQ_ERR_SHAPE;
    }
    const int chk = kq_multi_check(count, types, dev, N, K, x, M, y);
    if (chk) return chk;
    // copy: after the last GEMV that read this slot
    if (s->used[slot] && hipStreamWaitEvent(s->copy, s->freed[slot], 0) != hipSuccess) return KQ_ERR_LAUNCH;
    for (int i = 0; i < count; ++i) {
        if (!bytes[i]) continue;
        if (hipMemcpyAsync(const_cast<void *>(dev[i]), W[i], (size_t)bytes[i], hipMemcpyHostToDevice, s->copy) !=
            hipSuccess)
            return KQ_ERR_LAUNCH;
    }
    if (hipEventRecord(s->copied[slot], s->copy) != hipSuccess) return KQ_ERR_LAUNCH;
    // GEMV: after the copy, on the caller's stream
    if (hipStreamWaitEvent(s->stream, s->copied[slot], 0) != hipSuccess) return KQ_ERR_LAUNCH;
    const int r = kq_qgemv_multi(count, types, dev, N, K, x, M, y, (void *)s->stream);
    if (hipEventRecord(s->freed[slot], s->stream) != hipSuccess) return KQ_ERR_LAUNCH;
    s->used[slot] = true;
    s->next = (slot + 1) % s->nslots;
    return r;
}

int kq_stream_qgemv(kq_streamer *s, int type, const void *W, int64_t N, int64_t K, const float *x, int M,
                    float *y) {
    return kq_stream_qgemv_multi(s, 1, &type, &W, &N, K, x, M, &y);
}

} // extern "C"
