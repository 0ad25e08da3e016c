// kq_stamps.hip -- the batch-1 Q4_K pass with its weight ring in LDS (the
// library's qgemv1_dma_kernel: same templates, same launch shape) with
// timestamps at its phase boundaries, and the register-ring pass the same way
// for Q6_K, for kqp_stamped_qgemv1 (include/kqprobe.h).
// It shows where a launch's time goes: how late each work-group starts, its
// activation staging, the load of its activations into registers, the weight
// stream, and how far apart the work-groups and the XCDs finish.
//
// kq_impl.h is compiled here under a namespace of its own, so the copies of
// its templates in this library are distinct symbols from libkqgemv.so's.
#define kq kq_stamped
#include "kq_impl.h"
#undef kq

#include "kqprobe.h"

namespace kq_stamped {

__device__ __forceinline__ uint64_t now() { return __builtin_amdgcn_s_memrealtime(); }
__device__ __forceinline__ u32 xcc_id() {
    u32 id;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(id));
    return id & 0xFu;
}

// The body of qgemv1_dma_kernel<T_Q4_K, D, LB, MS, 64> with four stamps taken
// by wave 0 of each work-group: start, staging done (after its barrier),
// activations in registers, and the end (after a barrier that every wave
// reaches when its last row step is done).  stamps[8 g + i]: i = 0..3 the
// stamps (100 MHz constant clock), 4 the XCD, 5 the compute unit's hardware id.
template <int D, int LB, bool MS>
__global__ __launch_bounds__(LB) void stamped_q4k_kernel(const Segs sg, int64_t row_bytes, int K, int lpr, int ns,
                                                         const float *__restrict__ x, uint64_t *stamps) {
    constexpr int T = T_Q4_K;
    const uint64_t t0 = now();
    extern __shared__ float smem[];
    float (*part)[64] = reinterpret_cast<float (*)[64]>(smem);
    float *xs = smem + 16 * 64;
    const int XS = x_stride(K), SS = s_stride(K);
    float *ss = xs + XS;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    char *ring = reinterpret_cast<char *>(smem) + b1_ring_offset(K) + (size_t)wave * D * DmaGeom<T>::SLOT;
    const X1 xr = x1_load(x, K, (int)blockDim.x);
    __builtin_amdgcn_sched_barrier(0);
    B1Dma<T, D, MS, 1, 64> p(sg, row_bytes, K, lpr, ns, wave, lane, blockIdx.x, gridDim.x, ring);
    p.issue_first();
    __builtin_amdgcn_sched_barrier(0);
    x1_store<true>(xr, K, (int)blockDim.x, smem, xs, ss);
    const uint64_t t1 = now();
    XReg<T> xa;
    p.x_from_lds(xa, xs, ss, XS, SS);
    const uint64_t t2 = now();
    p.run(xa, part);
    wg_sync<true>();
    const uint64_t t3 = now();
    if (threadIdx.x == 0) {
        u32 hw;
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
        uint64_t *o = stamps + 8 * (size_t)blockIdx.x;
        o[0] = t0;
        o[1] = t1;
        o[2] = t2;
        o[3] = t3;
        o[4] = xcc_id();
        o[5] = hw;
    }
}

// The body of qgemv1_kernel<T, D, LB, MS, 64> (the register ring) with the
// same stamps; its activations go to registers inside the pass, so stamp 2
// equals stamp 1 and the register load counts to the weight stream.
template <int T, int D, int LB, bool MS>
__global__ __launch_bounds__(LB) void stamped_reg_kernel(const Segs sg, int64_t row_bytes, int K, int lpr, int ns,
                                                         const float *__restrict__ x, uint64_t *stamps) {
    const uint64_t t0 = now();
    extern __shared__ float smem[];
    float (*part)[64] = reinterpret_cast<float (*)[64]>(smem);
    float *xs = smem + 16 * 64;
    const int XS = x_stride(K), SS = s_stride(K);
    float *ss = xs + XS;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const X1 xr = x1_load(x, K, (int)blockDim.x);
    __builtin_amdgcn_sched_barrier(0);
    B1Pass<T, D, MS, 64> p(sg, row_bytes, K, lpr, ns, wave, lane, blockIdx.x, gridDim.x);
    p.issue_first();
    __builtin_amdgcn_sched_barrier(0);
    x1_store<false>(xr, K, (int)blockDim.x, smem, xs, ss);
    const uint64_t t1 = now();
    p.run(xs, ss, XS, SS, part);
    __syncthreads();
    const uint64_t t3 = now();
    if (threadIdx.x == 0) {
        u32 hw;
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
        uint64_t *o = stamps + 8 * (size_t)blockIdx.x;
        o[0] = t0;
        o[1] = t1;
        o[2] = t1;
        o[3] = t3;
        o[4] = xcc_id();
        o[5] = hw;
    }
}

} // namespace kq_stamped

using namespace kq_stamped;

extern "C" int kqp_stamped_qgemv1(int type, int count, const void *const *W, const int64_t *N, int64_t K,
                                  const float *x, float *const *y, uint64_t *stamps, int max_groups, int *groups,
                                  void *stream) {
    if (!W || !N || !y || !x || !stamps || !groups) return KQ_ERR_NULL;
    if ((type != KQ_TYPE_Q4_K && type != KQ_TYPE_Q6_K) || count < 1 || count > MAX_SEGS || max_groups < 1)
        return KQ_ERR_ARG;
    if (K < 256 || K % 256 || K > (1 << 20)) return KQ_ERR_SHAPE;
    const int64_t rb = (K / 256) * (type == KQ_TYPE_Q4_K ? 144 : 210);
    Segs sg = {};
    int64_t rows = 0;
    for (int i = 0; i < count; ++i) {
        if (!W[i] || !y[i]) return KQ_ERR_NULL;
        if (N[i] < 1 || rows + N[i] >= (1 << 30)) return KQ_ERR_SHAPE;
        if ((uintptr_t)W[i] % 16) return KQ_ERR_ALIGN;
        sg.W[i] = (const uint8_t *)W[i];
        sg.y[i] = y[i];
        sg.start[i] = (int)rows;
        sg.rows[i] = (int)N[i];
        rows += N[i];
    }
    sg.start[count] = (int)rows;
    sg.n = count;
    B1Cfg c;
    const bool q4 = type == KQ_TYPE_Q4_K;
    if (q4 ? (!batch1_cfg<T_Q4_K>((int)K, rows, &c) || c.lpr != 64 || !dma_ok<T_Q4_K>(c, sg, rb, (int)K))
           : (!batch1_cfg<T_Q6_K>((int)K, rows, &c) || c.lpr != 64))
        return KQ_ERR_SHAPE;    // not a shape the library serves with these kernels
    const int64_t need = (rows + c.rs - 1) / c.rs;
    const int64_t cap = cu_count();
    const int grid = (int)(need < cap ? need : cap);
    if (grid > max_groups) return KQ_ERR_ARG;
    *groups = grid;
    const size_t lds = q4 ? dma_lds<T_Q4_K>(c, (int)K) : c.lds;
    const int nt = 64 * c.ns * c.rs;
    hipStream_t st = (hipStream_t)stream;
    if (!q4) {
#define KQS_REG(WW, MSS)                                                                                     \
    do {                                                                                                     \
        auto kern = stamped_reg_kernel<T_Q6_K, PREFETCH<T_Q6_K, WW>(), WW ? 1024 : 512, MSS>;                \
        if (allow_lds(kern, lds) != hipSuccess) return KQ_ERR_LAUNCH;                                        \
        hipLaunchKernelGGL(kern, dim3(grid), dim3(nt), lds, st, sg, rb, (int)K, c.lpr, c.ns, x, stamps);     \
    } while (0)
        if (c.wide) {
            if (count > 1) KQS_REG(true, true);
            else KQS_REG(true, false);
        } else {
            if (count > 1) KQS_REG(false, true);
            else KQS_REG(false, false);
        }
#undef KQS_REG
        return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_LAUNCH;
    }
#define KQS_LAUNCH(DD, LBB, MSS)                                                                             \
    do {                                                                                                     \
        auto kern = stamped_q4k_kernel<DD, LBB, MSS>;                                                        \
        if (allow_lds(kern, lds) != hipSuccess) return KQ_ERR_LAUNCH;                                        \
        hipLaunchKernelGGL(kern, dim3(grid), dim3(nt), lds, st, sg, rb, (int)K, c.lpr, c.ns, x, stamps);     \
    } while (0)
    if (c.wide) {
        if (count > 1) KQS_LAUNCH(DMA_DEPTH<true>(), 1024, true);
        else KQS_LAUNCH(DMA_DEPTH<true>(), 1024, false);
    } else {
        if (count > 1) KQS_LAUNCH(DMA_DEPTH<false>(), 512, true);
        else KQS_LAUNCH(DMA_DEPTH<false>(), 512, false);
    }
#undef KQS_LAUNCH
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_LAUNCH;
}
