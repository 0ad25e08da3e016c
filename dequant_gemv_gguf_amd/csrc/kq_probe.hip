// kq_probe.hip -- measurement kernels declared in include/kqprobe.h: the HBM
// read-stream ceiling for the load forms the GEMV kernels use, the floor of a
// kernel launch, and a grid-wide barrier between dependent phases of one
// persistent launch against a launch per phase.  They compute nothing of the
// dequant-GEMV; the benchmark runs them to place the GEMV kernels' rates.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kqgemv.h"
#include "kqprobe.h"

namespace kqp {

typedef uint32_t u32;
typedef u32 u4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;
#define KQP_LDS __attribute__((address_space(3)))

constexpr int SPAN = 3072;            // bytes of one wave step
constexpr int NLD = SPAN / 1024;      // 1-KB requests per step
constexpr u32 OOB = 0x80000000u;      // past every buffer: loads return 0
constexpr uint64_t MAX_BYTES = (1ull << 32) - 4096;
constexpr int PH_WAVES = 16, PH_DEPTH = 2, PH_XMAX = 48 * 1024;
constexpr int64_t SPIN_TICKS = 20000000;   // 0.2 s of the 100 MHz constant clock

__device__ __forceinline__ rsrc_t mk(const void *p, u32 n) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)n, 0x00020000);
}
template <int N> __device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// work-group barrier that waits only for LDS accesses (buffer-to-LDS loads in
// flight stay in flight)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Steps of wave gw among nw waves over nspans spans (uniform over the wave).
__device__ __forceinline__ u32 wave_steps(uint64_t nspans, u32 gw, u32 nw) {
    return nspans > gw ? (u32)((nspans - gw + nw - 1) / nw) : 0u;
}
__device__ __forceinline__ u32 step_off(u32 gw, u32 nw, u32 j) { return (u32)(((uint64_t)gw + (uint64_t)j * nw) * SPAN); }

// ---- read stream into registers (mode 0)
template <int D>
__global__ __launch_bounds__(1024) void stream_reg_kernel(const uint8_t *src, u32 bytes, u32 *sink) {
    const int waves = blockDim.x >> 6;
    const u32 wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const u32 nw = gridDim.x * waves, gw = blockIdx.x * waves + wave;
    const u32 steps = wave_steps(((uint64_t)bytes + SPAN - 1) / SPAN, gw, nw);
    const rsrc_t rs = mk(src, bytes);
    u4 ring[D][NLD];
    u32 acc = 0;
    auto issue = [&](int d, u32 j) {
#pragma unroll
        for (int k = 0; k < NLD; ++k)
            ring[d][k] = __builtin_bit_cast(
                u4, __builtin_amdgcn_raw_buffer_load_b128(rs, j < steps ? step_off(gw, nw, j) + 1024u * k + 16u * lane : OOB,
                                                          0, 2 /* nt */));
    };
#pragma unroll
    for (int d = 0; d < D; ++d) issue(d, d);
    u32 j = 0;
    for (; j < steps; j += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
#pragma unroll
            for (int k = 0; k < NLD; ++k) acc ^= ring[d][k].x ^ ring[d][k].y ^ ring[d][k].z ^ ring[d][k].w;
            issue(d, j + d + D);
        }
    }
#pragma unroll
    for (int d = 0; d < D; ++d)
#pragma unroll
        for (int k = 0; k < NLD; ++k) acc ^= ring[d][k].x;
    sink[(blockIdx.x * waves + wave) * 64 + lane] = acc;
}

// ---- read stream through a per-wave LDS ring (mode 1): the weight stream of
// the Q4_K batch-1 kernels without their arithmetic.  Before reading slot d a
// wave lets the NLD (D - 1) loads of its later slots stay outstanding; its
// reads of the slot complete before the slot is refilled.
template <int D> struct LdsRing {
    char *ring;
    rsrc_t rs;
    u32 gw, nw, steps, lane;
    __device__ __forceinline__ void issue(int d, u32 j) {
        char *dst = ring + d * SPAN;
#pragma unroll
        for (int k = 0; k < NLD; ++k)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (KQP_LDS void *)(dst + 1024 * k), 16,
                                                     j < steps ? step_off(gw, nw, j) + 1024u * k + 16u * lane : OOB,
                                                     0, 0, 2 /* nt */);
    }
    __device__ __forceinline__ void first() {
#pragma unroll
        for (int d = 0; d < D; ++d) issue(d, d);
    }
    // consume every step (the first D already issued); returns the XOR of one
    // dword a lane read per step
    __device__ __forceinline__ u32 run() {
        u32 acc = 0;
        for (u32 j = 0; j < steps; j += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                wait_vm<NLD * (D - 1)>();
                acc ^= *reinterpret_cast<const u32 *>(ring + d * SPAN + 16 * lane + 1024 * ((j + d) % NLD));
                wait_lgkm0();
                issue(d, j + d + D);
            }
        }
        wait_vm<0>();
        return acc;
    }
};

template <int D>
__global__ __launch_bounds__(1024) void stream_lds_kernel(const uint8_t *src, u32 bytes, u32 *sink) {
    extern __shared__ char smem[];
    const int waves = blockDim.x >> 6;
    const u32 wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    LdsRing<D> r;
    r.ring = smem + wave * D * SPAN;
    r.rs = mk(src, bytes);
    r.nw = gridDim.x * waves;
    r.gw = blockIdx.x * waves + wave;
    r.steps = wave_steps(((uint64_t)bytes + SPAN - 1) / SPAN, r.gw, r.nw);
    r.lane = lane;
    r.first();
    sink[(blockIdx.x * waves + wave) * 64 + lane] = r.run();
}

__global__ void empty_kernel() {}

// ---- dependent phases.  Phase p reads its weights at src + p * stride after
// staging xbytes of activations in LDS.  COOP: all phases in one launch with a
// grid-wide barrier between them (arrival: work-group barrier, agent-scope
// release, one atomic add; wait: relaxed agent-scope loads of the count, then
// an agent-scope acquire), the count returned to 0 by the last arrival of the
// launch.  With prefetch the next phase's first ring loads are issued between
// arrival and wait.
// Activations of phase p: with COH (coherent mode) 16-byte loads at device
// scope (they read the coherence point, never a stale line in this XCD's L2),
// else plain loads after the acquire.
__device__ __forceinline__ f4 ld_x(const float *x, int i, bool coh) {
    if (!coh) return reinterpret_cast<const f4 *>(x)[i];
    const rsrc_t r = mk(x, 0x7ffffff0u);
    return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, 16u * i, 0, 16 /* sc1 */));
}

template <bool COOP>
__global__ __launch_bounds__(1024) void phased_kernel(const uint8_t *src, uint64_t stride, u32 pbytes, int p0,
                                                      int nphases, const float *x, int xbytes, int prefetch,
                                                      u32 *ctr, u32 *sink) {
    // prefetch bit 0: issue the next phase's first loads before the wait;
    // bit 1: coherent mode -- no cache maintenance at the barrier (the data
    // crossing it is written and read at device scope), only the count
    const bool coh = (prefetch & 2) != 0;
    extern __shared__ char smem[];
    const u32 wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    float *xs = reinterpret_cast<float *>(smem + PH_WAVES * PH_DEPTH * SPAN);
    LdsRing<PH_DEPTH> r;
    r.ring = smem + wave * PH_DEPTH * SPAN;
    r.nw = gridDim.x * PH_WAVES;
    r.gw = blockIdx.x * PH_WAVES + wave;
    r.lane = lane;
    const uint64_t nspans = ((uint64_t)pbytes + SPAN - 1) / SPAN;
    u32 acc = 0;
    float xacc = 0.f;
    bool issued = false;
    for (int p = p0; p < p0 + nphases; ++p) {
        if (!issued) {
            r.rs = mk(src + (uint64_t)p * stride, pbytes);
            r.steps = wave_steps(nspans, r.gw, r.nw);
            r.first();
        }
        issued = false;
        // stage the activations (register loads, then LDS, then a barrier)
        for (int i = threadIdx.x; i < xbytes / 16; i += blockDim.x) reinterpret_cast<f4 *>(xs)[i] = ld_x(x, i, coh);
        lds_barrier();
        if (xbytes >= 4) xacc += xs[(threadIdx.x * 4) % (xbytes / 4)];
        acc ^= r.run();
        if (COOP && p + 1 < p0 + nphases) {
            lds_barrier();
            if (threadIdx.x == 0) {
                if (coh)
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                else
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                __hip_atomic_fetch_add(&ctr[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            if (prefetch & 1) {
                r.rs = mk(src + (uint64_t)(p + 1) * stride, pbytes);
                r.steps = wave_steps(nspans, r.gw, r.nw);
                r.first();
                issued = true;
            }
            if (threadIdx.x == 0) {
                const u32 target = (u32)(p + 1 - p0) * gridDim.x;
                const int64_t t0 = (int64_t)__builtin_amdgcn_s_memrealtime();
                while (__hip_atomic_load(&ctr[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
                    if (__hip_atomic_load(&ctr[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) break;
                    if ((int64_t)__builtin_amdgcn_s_memrealtime() - t0 > SPIN_TICKS) {
                        __hip_atomic_store(&ctr[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                if (!coh) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            }
            lds_barrier();
        }
    }
    if (COOP) {
        lds_barrier();
        if (threadIdx.x == 0) {
            const u32 last = (u32)nphases * gridDim.x - 1;
            if (__hip_atomic_fetch_add(&ctr[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == last)
                __hip_atomic_store(&ctr[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    sink[(blockIdx.x * PH_WAVES + wave) * 64 + lane] = acc ^ __builtin_bit_cast(u32, xacc);
}

// ---- the 4x4x4 (16 blocks) f16 matrix instruction on one wave: D = A.B + C
// for 64 lanes' operands as given (each lane: 4 halves of A, 4 of B, 4 floats
// of C), so that the lane layout and the rounding of the instruction can be
// read off on the host.
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(64) void mfma4_kernel(const h4 *a, const h4 *b, const f4 *c, f4 *d) {
    const int l = threadIdx.x;
    d[l] = __builtin_amdgcn_mfma_f32_4x4x4f16(a[l], b[l], c[l], 0, 0, 0);
}

// ---- the 16x16x32 and 16x16x16 f16 matrix instructions on one wave: D =
// A.B + C for 64 lanes' operands as given (each lane: 8 or 4 halves of A and
// of B, 4 floats of C), so that their lane layouts can be read off on the host.
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
__global__ __launch_bounds__(64) void mfma16_kernel(const h8 *a, const h8 *b, const f4 *c, f4 *d, int k32) {
    const int l = threadIdx.x;
    if (k32) {
        d[l] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[l], b[l], c[l], 0, 0, 0);
    } else {
        const h8 av = a[l], bv = b[l];
        const h4 a4 = {av[0], av[1], av[2], av[3]}, b4 = {bv[0], bv[1], bv[2], bv[3]};
        d[l] = __builtin_amdgcn_mfma_f32_16x16x16f16(a4, b4, c[l], 0, 0, 0);
    }
}

// Issue rate of that instruction: `chains` independent accumulators per wave,
// `iters` instructions each, waves * nwg waves.
template <int CH>
__global__ __launch_bounds__(1024) void mfma4_rate_kernel(int iters, u32 *sink) {
    const int l = threadIdx.x & 63;
    h4 a = {(_Float16)(l & 3), (_Float16)1, (_Float16)0.5f, (_Float16)2};
    h4 b = {(_Float16)1, (_Float16)(l >> 4), (_Float16)0.25f, (_Float16)1};
    f4 acc[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) acc[i] = (f4){0.f, 0.f, 0.f, (float)i};
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int i = 0; i < CH; ++i) acc[i] = __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, acc[i], 0, 0, 0);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < CH; ++i) s += acc[i].x + acc[i].y + acc[i].z + acc[i].w;
    sink[blockIdx.x * blockDim.x + threadIdx.x] = __builtin_bit_cast(u32, s);
}

inline int cu_count() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return n;
}

template <typename K> bool allow(K k, size_t bytes) {
    return bytes <= 65536 ||
           hipFuncSetAttribute(reinterpret_cast<const void *>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes) == hipSuccess;
}

} // namespace kqp

using namespace kqp;

extern "C" {

int kqp_read_stream(const void *src, uint64_t bytes, int mode, int nwg, int waves, int depth, uint32_t *sink,
                    void *stream) {
    if (!src || !sink) return KQ_ERR_NULL;
    if (((uintptr_t)src | (uintptr_t)sink) & 15) return KQ_ERR_ALIGN;
    if (bytes == 0 || bytes % 16 || bytes > MAX_BYTES) return KQ_ERR_SHAPE;
    if ((mode != 0 && mode != 1) || nwg < 1 || nwg > 65535 || (waves != 4 && waves != 8 && waves != 16) || depth < 1 ||
        depth > 4)
        return KQ_ERR_ARG;
    const size_t lds = mode ? (size_t)waves * depth * SPAN : 0;
    if (lds > 160 * 1024) return KQ_ERR_ARG;
    hipStream_t st = (hipStream_t)stream;
    const dim3 g(nwg), b(64 * waves);
    const u32 n = (u32)bytes;
    const uint8_t *s = (const uint8_t *)src;
#define KQP_CASE(D)                                                                      \
    case D:                                                                              \
        if (mode == 0) {                                                                 \
            hipLaunchKernelGGL(stream_reg_kernel<D>, g, b, 0, st, s, n, sink);           \
        } else {                                                                         \
            if (!allow(stream_lds_kernel<D>, lds)) return KQ_ERR_LAUNCH;                 \
            hipLaunchKernelGGL(stream_lds_kernel<D>, g, b, lds, st, s, n, sink);         \
        }                                                                                \
        break;
    switch (depth) {
        KQP_CASE(1)
        KQP_CASE(2)
        KQP_CASE(3)
        KQP_CASE(4)
    }
#undef KQP_CASE
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_LAUNCH;
}

int kqp_empty(int nwg, int threads, void *stream) {
    if (nwg < 1 || nwg > 65535 || threads < 64 || threads > 1024 || threads % 64) return KQ_ERR_ARG;
    hipLaunchKernelGGL(empty_kernel, dim3(nwg), dim3(threads), 0, (hipStream_t)stream);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_LAUNCH;
}

int kqp_mfma4(const void *a, const void *b, const float *c, float *d, void *stream) {
    if (!a || !b || !c || !d) return KQ_ERR_NULL;
    if (((uintptr_t)a | (uintptr_t)b) & 7 || ((uintptr_t)c | (uintptr_t)d) & 15) return KQ_ERR_ALIGN;
    hipLaunchKernelGGL(mfma4_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, (const h4 *)a, (const h4 *)b,
                       (const f4 *)c, (f4 *)d);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_LAUNCH;
}

int kqp_mfma16(const void *a, const void *b, const float *c, float *d, int k32, void *stream) {
    if (!a || !b || !c || !d) return KQ_ERR_NULL;
    if (((uintptr_t)a | (uintptr_t)b | (uintptr_t)c | (uintptr_t)d) & 15) return KQ_ERR_ALIGN;
    hipLaunchKernelGGL(mfma16_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, (const h8 *)a, (const h8 *)b,
                       (const f4 *)c, (f4 *)d, k32);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_LAUNCH;
}

int kqp_mfma4_rate(int nwg, int waves, int chains, int iters, uint32_t *sink, void *stream) {
    if (!sink) return KQ_ERR_NULL;
    if (nwg < 1 || nwg > 65535 || waves < 1 || waves > 16 || iters < 1 || (chains != 1 && chains != 2 && chains != 4 &&
                                                                         chains != 8))
        return KQ_ERR_ARG;
    hipStream_t st = (hipStream_t)stream;
    const dim3 g(nwg), bl(64 * waves);
    switch (chains) {
    case 1: hipLaunchKernelGGL(mfma4_rate_kernel<1>, g, bl, 0, st, iters, sink); break;
    case 2: hipLaunchKernelGGL(mfma4_rate_kernel<2>, g, bl, 0, st, iters, sink); break;
    case 4: hipLaunchKernelGGL(mfma4_rate_kernel<4>, g, bl, 0, st, iters, sink); break;
    default: hipLaunchKernelGGL(mfma4_rate_kernel<8>, g, bl, 0, st, iters, sink); break;
    }
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_LAUNCH;
}

int kqp_phased_stream(const void *src, uint64_t phase_stride, uint64_t phase_bytes, int nphases, const float *x,
                      int xbytes, int persistent, int prefetch, uint32_t *ctr, uint32_t *sink, void *stream) {
    if (!src || !sink || (xbytes && !x) || (persistent && !ctr)) return KQ_ERR_NULL;
    if (((uintptr_t)src | (uintptr_t)sink | (uintptr_t)x) & 15 || ((uintptr_t)ctr & 3)) return KQ_ERR_ALIGN;
    if (phase_bytes == 0 || phase_bytes % 16 || phase_bytes > MAX_BYTES || nphases < 1 || xbytes < 0 ||
        xbytes % 16 || xbytes > PH_XMAX || phase_stride < phase_bytes)
        return KQ_ERR_SHAPE;
    const int nwg = cu_count();
    if (nwg <= 0) return KQ_ERR_DEVICE;
    hipStream_t st = (hipStream_t)stream;
    const size_t lds = (size_t)PH_WAVES * PH_DEPTH * SPAN + (size_t)xbytes;
    const u32 pb = (u32)phase_bytes;
    const uint8_t *s = (const uint8_t *)src;
    if (!persistent) {
        if (!allow(phased_kernel<false>, lds)) return KQ_ERR_LAUNCH;
        for (int p = 0; p < nphases; ++p) {
            hipLaunchKernelGGL(phased_kernel<false>, dim3(nwg), dim3(64 * PH_WAVES), lds, st, s, phase_stride, pb, p,
                               1, x, xbytes, 0, ctr, sink);
        }
        return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_LAUNCH;
    }
    if (!allow(phased_kernel<true>, lds)) return KQ_ERR_LAUNCH;
    int p0 = 0;
    void *args[] = {&s, &phase_stride, (void *)&pb, &p0, &nphases, &x, &xbytes, &prefetch, &ctr, &sink};
    const hipError_t e = hipLaunchCooperativeKernel(reinterpret_cast<const void *>(phased_kernel<true>), dim3(nwg),
                                                    dim3(64 * PH_WAVES), args, (unsigned)lds, st);
    return e == hipSuccess ? KQ_OK : KQ_ERR_LAUNCH;
}

} // extern "C"
