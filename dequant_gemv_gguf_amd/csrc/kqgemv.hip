// kqgemv.hip -- C ABI of the fused GGUF K-quant dequant-GEMV library for AMD
// MI355X (gfx950), declared in include/kqgemv.h: argument checks, format
// dispatch and grouping of the products into launches.  The kernels and their
// launchers are in kq_impl.h.
#include "kq_impl.h"

#include <cstring>

#define KQ_VERSION 10000

namespace kq {

// y[t][o] = sum_j route_w[t][j] * ys[t][j][o], ascending j.
__global__ __launch_bounds__(WG_THREADS) void moe_combine_kernel(const float *__restrict__ ys,
                                                                 const float *__restrict__ rw, int T, int k, int N,
                                                                 float *__restrict__ y) {
    const int64_t i = (int64_t)blockIdx.x * WG_THREADS + threadIdx.x;
    if (i >= (int64_t)T * N) return;
    const int t = (int)(i / N);
    const int64_t o = i - (int64_t)t * N;
    float acc = 0.f;
    for (int j = 0; j < k; ++j) acc = __builtin_fmaf(rw[t * k + j], ys[((int64_t)t * k + j) * N + o], acc);
    y[i] = acc;
}

int launch_group_t(int type, int M, const std::vector<int> &ids, const void *const *W, const int64_t *N, int K,
                   const float *x, float *const *y, hipStream_t st) {
    const int64_t rb = kq_row_bytes_(type, K);
    return with_type(type, [&](auto tag) { return launch_group<decltype(tag)::value>(M, ids, W, N, rb, K, x, y, st); });
}

int launch_mixed_t(int ta, int tb, const std::vector<int> &ia, size_t *pa, const std::vector<int> &ib, size_t *pb,
                   const void *const *W, const int64_t *N, int K, const float *x, float *const *y, hipStream_t st) {
#define KQ_PAIR(A, B) \
    if (ta == KQ_TYPE_##A && tb == KQ_TYPE_##B) return launch_mixed<T_##A, T_##B>(ia, pa, ib, pb, W, N, K, x, y, st);
    KQ_PAIR(Q2_K, Q3_K) KQ_PAIR(Q2_K, Q4_K) KQ_PAIR(Q2_K, Q5_K) KQ_PAIR(Q2_K, Q6_K)
    KQ_PAIR(Q3_K, Q4_K) KQ_PAIR(Q3_K, Q5_K) KQ_PAIR(Q3_K, Q6_K)
    KQ_PAIR(Q4_K, Q5_K) KQ_PAIR(Q4_K, Q6_K) KQ_PAIR(Q5_K, Q6_K)
#undef KQ_PAIR
    return KQ_ERR_ARG;
}

// Whether the current device is a gfx950 (the only target the kernels are
// built for), looked up once per device.
constexpr int CHECKED_DEVICES = 64;
static std::atomic<int> device_state[CHECKED_DEVICES];   // 0 unknown, 1 gfx950, 2 other
static int device_check() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= CHECKED_DEVICES) return KQ_ERR_DEVICE;
    int st = device_state[dev].load(std::memory_order_acquire);
    if (!st) {
        hipDeviceProp_t prop;
        st = (hipGetDeviceProperties(&prop, dev) == hipSuccess && strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        device_state[dev].store(st, std::memory_order_release);
    }
    return st == 1 ? KQ_OK : KQ_ERR_DEVICE;
}

// Scratch of kq_qmoe_gemv_noalloc: the per-slot results of a routing-weighted
// sum served by the slot-major kernel, in a static device array instead of
// caller memory.  The array's name is a host-side stand-in: host code uses
// only the address hipGetSymbolAddress returns for the current device (each
// device holds its own copy), looked up once per device on the first call.
static __device__ __align__(256) float scratch[KQ_NOALLOC_SCRATCH_BYTES / sizeof(float)];

constexpr int SCRATCH_DEVICES = 64;
inline std::mutex &scratch_mutex() {
    static std::mutex mu;
    return mu;
}
static std::atomic<float *> scratch_addr[SCRATCH_DEVICES];

// The scratch array's address on the current device (KQ_ERR_DEVICE when it
// cannot be resolved).
static int scratch_of_device(float **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= SCRATCH_DEVICES) return KQ_ERR_DEVICE;
    float *p = scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(scratch_mutex());
        p = scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            void *a = nullptr;
            if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return KQ_ERR_DEVICE;
            p = static_cast<float *>(a);
            scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return KQ_OK;
}

} // namespace kq

using namespace kq;

// ---------------------------------------------------------------------------
// C ABI

extern "C" {

int kq_version(void) { return KQ_VERSION; }

const char *kq_status_string(int status) {
    switch (status) {
    case KQ_OK: return "ok";
    case KQ_ERR_TYPE: return "unsupported quant type";
    case KQ_ERR_SHAPE: return "invalid shape";
    case KQ_ERR_M: return "row count M (or T) outside 1..8";
    case KQ_ERR_NULL: return "required pointer is NULL";
    case KQ_ERR_ALIGN: return "pointer misaligned";
    case KQ_ERR_ARG: return "invalid argument";
    case KQ_ERR_LAUNCH: return "kernel launch failed";
    case KQ_ERR_DEVICE: return "no usable device";
    case KQ_ERR_IO: return "file could not be opened or mapped";
    case KQ_ERR_FORMAT: return "malformed or unsupported file";
    default: return "unknown status";
    }
}

int kq_block_info(int type, int *block_elems, int *block_bytes) {
    int qk, nb, upb;
    if (fmt_of(type, &qk, &nb, &upb)) return KQ_ERR_TYPE;
    if (!block_elems || !block_bytes) return KQ_ERR_NULL;
    *block_elems = qk;
    *block_bytes = nb;
    return KQ_OK;
}

int64_t kq_row_bytes(int type, int64_t K) {
    int qk, nb, upb;
    if (fmt_of(type, &qk, &nb, &upb)) return KQ_ERR_TYPE;
    if (K <= 0 || K % qk) return KQ_ERR_SHAPE;
    return (K / qk) * nb;
}

int kq_dequant(int type, const void *src, int64_t n_elems, float *dst, void *stream) {
    int qk, nb, upb;
    if (fmt_of(type, &qk, &nb, &upb)) return KQ_ERR_TYPE;
    if (n_elems < 0 || n_elems % qk || n_elems > ((int64_t)1 << 40)) return KQ_ERR_SHAPE;
    if (n_elems == 0) return KQ_OK;
    if (!src || !dst) return KQ_ERR_NULL;
    if (!aligned(src, 16) || !aligned(dst, 16)) return KQ_ERR_ALIGN;
    if (device_check()) return KQ_ERR_DEVICE;
    hipStream_t st = (hipStream_t)stream;
    return with_type(type, [&](auto tag) { return launch_dequant_t<decltype(tag)::value>(src, n_elems, dst, st); });
}

static int check_gemv_shape(int type, int64_t N, int64_t K, int64_t *row_bytes) {
    int qk, nb, upb;
    if (fmt_of(type, &qk, &nb, &upb)) return KQ_ERR_TYPE;
    if (K <= 0 || K % qk || K > ((int64_t)1 << 20)) return KQ_ERR_SHAPE;
    if (N < 0 || N >= ((int64_t)1 << 31)) return KQ_ERR_SHAPE;
    *row_bytes = (K / qk) * nb;
    // one work-group tile (at most 64 rows) must stay below 2^31 bytes
    if (64 * *row_bytes >= ((int64_t)1 << 31)) return KQ_ERR_SHAPE;
    return KQ_OK;
}

int kq_qgemv(int type, const void *W, int64_t N, int64_t K, const float *x, int M, float *y, void *stream) {
    int64_t row_bytes;
    int r = check_gemv_shape(type, N, K, &row_bytes);
    if (r) return r;
    if (M < 1 || M > 8) return KQ_ERR_M;
    if (N == 0) return KQ_OK;
    if (!W || !x || !y) return KQ_ERR_NULL;
    if (!aligned(W, 16) || !aligned(x, 16) || !aligned(y, 16)) return KQ_ERR_ALIGN;
    if (device_check()) return KQ_ERR_DEVICE;
    hipStream_t st = (hipStream_t)stream;
    return with_type(type, [&](auto tag) {
        return launch_qgemv_m<decltype(tag)::value>(M, W, row_bytes, (int)N, (int)K, x, y, st);
    });
}

// Every argument check of kq_qgemv_multi, in its order (also used by the
// host-streamed calls, on the slot addresses, before they issue anything).
__attribute__((visibility("hidden"))) int kq_multi_check(int count, const int *types, const void *const *W,
                                                         const int64_t *N, int64_t K, const float *x, int M,
                                                         float *const *y) {
    if (count < 0) return KQ_ERR_ARG;
    if (count == 0) return KQ_OK;
    if (!types || !W || !N || !y) return KQ_ERR_NULL;
    for (int i = 0; i < count; ++i) {
        int64_t rb;
        const int r = check_gemv_shape(types[i], N[i], K, &rb);
        if (r) return r;
    }
    if (M < 1 || M > 8) return KQ_ERR_M;
    bool any = false;
    for (int i = 0; i < count; ++i) {
        if (N[i] == 0) continue;
        if (!W[i] || !y[i]) return KQ_ERR_NULL;
        if (!aligned(W[i], 16) || !aligned(y[i], 16)) return KQ_ERR_ALIGN;
        any = true;
    }
    if (any && !x) return KQ_ERR_NULL;
    if (any && !aligned(x, 16)) return KQ_ERR_ALIGN;
    return KQ_OK;
}

int kq_qgemv_multi(int count, const int *types, const void *const *W, const int64_t *N, int64_t K, const float *x,
                   int M, float *const *y, void *stream) {
    const int chk = kq_multi_check(count, types, W, N, K, x, M, y);
    if (chk || count == 0) return chk;
    // the matrices to compute, by format, in the caller's order
    constexpr int NT = 7, NKQ = 5;                    // formats; the first NKQ are K-quants
    const int tids[NT] = {KQ_TYPE_Q4_K, KQ_TYPE_Q6_K, KQ_TYPE_Q5_K, KQ_TYPE_Q3_K, KQ_TYPE_Q2_K, KQ_TYPE_Q8_0,
                          KQ_TYPE_Q4_0};
    std::vector<int> by[NT];
    for (int i = 0; i < count; ++i) {
        if (N[i] == 0) continue;
        for (int t = 0; t < NT; ++t)
            if (types[i] == tids[t]) by[t].push_back(i);
    }
    bool any = false;
    for (int t = 0; t < NT; ++t) any = any || !by[t].empty();
    if (!any) return KQ_OK;
    if (device_check()) return KQ_ERR_DEVICE;
    hipStream_t st = (hipStream_t)stream;
    size_t pos[NT] = {};
    if (M == 1) {
        // two K-quant formats: pair them up in mixed launches while both last
        int a = -1, b = -1;
        for (int t = 0; t < NKQ; ++t) {
            if (by[t].empty()) continue;
            if (a < 0) a = t; else if (b < 0) b = t;
        }
        if (a >= 0 && b >= 0) {
            const int lo = tids[a] < tids[b] ? a : b, hi = lo == a ? b : a;
            while (pos[lo] < by[lo].size() && pos[hi] < by[hi].size()) {
                const int r = launch_mixed_t(tids[lo], tids[hi], by[lo], &pos[lo], by[hi], &pos[hi], W, N, (int)K, x,
                                             y, st);
                if (r == KQ_ERR_ARG) break;              // shapes do not pair: separate launches
                if (r) return r;
            }
        }
    }
    for (int t = 0; t < NT; ++t) {
        if (pos[t] >= by[t].size()) continue;
        const std::vector<int> rest(by[t].begin() + (long)pos[t], by[t].end());
        const int r = launch_group_t(tids[t], M, rest, W, N, (int)K, x, y, st);
        if (r) return r;
    }
    return KQ_OK;
}

int kq_qgemv_mc_multi(int count, const int *types, const void *const *W, const int64_t *N, int64_t K,
                      const float *x, int M, float *const *y, void *stream) {
    const int chk = kq_multi_check(count, types, W, N, K, x, M, y);
    if (chk || count == 0) return chk;
    bool any = false;
    for (int i = 0; i < count; ++i) {
        if (types[i] != KQ_TYPE_Q4_K && types[i] != KQ_TYPE_Q6_K) return KQ_ERR_TYPE;
        any = any || N[i] > 0;
    }
    if (!any) return KQ_OK;
    if (device_check()) return KQ_ERR_DEVICE;
    return mc_run(count, types, W, N, (int)K, x, M, y, (hipStream_t)stream);
}

int kq_qgemv_mc(int type, const void *W, int64_t N, int64_t K, const float *x, int M, float *y, void *stream) {
    const int types[1] = {type};
    const void *const Ws[1] = {W};
    const int64_t Ns[1] = {N};
    float *const ys[1] = {y};
    return kq_qgemv_mc_multi(1, types, Ws, Ns, K, x, M, ys, stream);
}

size_t kq_qmoe_workspace_bytes(int T, int k, int64_t N) {
    if (T < 1 || T > 8 || k < 1 || k > 16 || N < 0 || N >= ((int64_t)1 << 31)) return 0;
    return (size_t)T * (size_t)k * (size_t)N * sizeof(float);
}

// Argument checks of kq_qmoe_gemv (need_ws: a workspace is required when
// route_w is given), in their order; KQ_OK with *row_bytes set, or N == 0
// reported through *empty.
static int qmoe_check(int type, const void *W_exps, int64_t E, int64_t N, int64_t K, const int32_t *ids,
                      const float *route_w, int T, int k, const float *x, int x_mode, const float *y,
                      const float *workspace, bool need_ws, const int32_t *err_flag, int64_t *row_bytes, bool *empty) {
    int r = check_gemv_shape(type, N, K, row_bytes);
    if (r) return r;
    if (T < 1 || T > 8) return KQ_ERR_M;
    if (E < 1 || E >= ((int64_t)1 << 31) || k < 1 || k > 16 || k > E || (x_mode != 0 && x_mode != 1))
        return KQ_ERR_ARG;
    *empty = N == 0;
    if (N == 0) return KQ_OK;
    if (!W_exps || !ids || !x || !y || (need_ws && route_w && !workspace)) return KQ_ERR_NULL;
    if (!aligned(W_exps, 16) || !aligned(x, 16) || !aligned(y, 16) || !aligned(ids, 4) ||
        (route_w && (!aligned(route_w, 4) || (need_ws && !aligned(workspace, 16)))) ||
        (err_flag && !aligned(err_flag, 4)))
        return KQ_ERR_ALIGN;
    return KQ_OK;
}

// The routed-expert product once its arguments are checked: token-major with
// the sum in the same launch when the activation rows fit, else slot-major
// through `workspace` and the separate sum.
static int qmoe_run(int type, const void *W_exps, int64_t E, int64_t N, int64_t K, int64_t row_bytes,
                    const int32_t *ids, const float *route_w, int T, int k, const float *x, int x_mode, float *y,
                    float *workspace, int32_t *err_flag, hipStream_t st) {
    if (device_check()) return KQ_ERR_DEVICE;
    int r;
    MoeSet set = {};
    set.W[0] = (const uint8_t *)W_exps;
    set.y[0] = y;
    set.n = 1;
    // token-major, with the routing-weighted sums in the same launch, when the
    // activation rows fit; otherwise slot-major, then the separate sum
    r = with_type(type, [&](auto tag) {
        return launch_qmoe_tok_t<decltype(tag)::value>(set, row_bytes, (int)E, (int)N, (int)K, ids, route_w, T, k,
                                                       x, x_mode, err_flag, st);
    });
    if (r != KQ_ERR_ARG) return r;
    set.y[0] = route_w ? workspace : y;
    // a batch never holds more slots than there are tokens unless a token
    // repeats an expert; MAXM = T covers the distinct-ids case in one pass
    const int maxm = T;
    r = with_type(type, [&](auto tag) {
        return launch_qmoe_m<decltype(tag)::value>(maxm, set, row_bytes, (int)E, (int)N, (int)K, ids, T, k, x,
                                                   x_mode, err_flag, st);
    });
    if (r || !route_w) return r;
    const int64_t total = (int64_t)T * N;
    hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)((total + WG_THREADS - 1) / WG_THREADS)), dim3(WG_THREADS),
                       0, st, workspace, route_w, T, k, (int)N, y);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_LAUNCH;
}

int kq_qmoe_gemv(int type, const void *W_exps, int64_t E, int64_t N, int64_t K, const int32_t *ids,
                 const float *route_w, int T, int k, const float *x, int x_mode, float *y, float *workspace,
                 int32_t *err_flag, void *stream) {
    int64_t row_bytes;
    bool empty = false;
    const int r = qmoe_check(type, W_exps, E, N, K, ids, route_w, T, k, x, x_mode, y, workspace, true, err_flag,
                             &row_bytes, &empty);
    if (r || empty) return r;
    return qmoe_run(type, W_exps, E, N, K, row_bytes, ids, route_w, T, k, x, x_mode, y, workspace, err_flag,
                    (hipStream_t)stream);
}

int kq_qmoe_gemv_noalloc(int type, const void *W_exps, int64_t E, int64_t N, int64_t K, const int32_t *ids,
                         const float *route_w, int T, int k, const float *x, int x_mode, float *y,
                         int32_t *err_flag, void *stream) {
    int64_t row_bytes;
    bool empty = false;
    int r = qmoe_check(type, W_exps, E, N, K, ids, route_w, T, k, x, x_mode, y, nullptr, false, err_flag, &row_bytes,
                       &empty);
    if (r || empty) return r;
    float *ws = nullptr;
    if (route_w) {
        if (kq_qmoe_workspace_bytes(T, k, N) > KQ_NOALLOC_SCRATCH_BYTES) return KQ_ERR_SHAPE;
        r = scratch_of_device(&ws);
        if (r) return r;
    }
    return qmoe_run(type, W_exps, E, N, K, row_bytes, ids, route_w, T, k, x, x_mode, y, ws, err_flag,
                    (hipStream_t)stream);
}

int kq_qmoe_gemv_multi(int count, int type, const void *const *W_exps, int64_t E, int64_t N, int64_t K,
                       const int32_t *ids, int T, int k, const float *x, int x_mode, float *const *y,
                       int32_t *err_flag, void *stream) {
    int64_t row_bytes;
    int r = check_gemv_shape(type, N, K, &row_bytes);
    if (r) return r;
    if (count < 1 || count > MOE_SETS) return KQ_ERR_ARG;
    if (T < 1 || T > 8) return KQ_ERR_M;
    if (E < 1 || E >= ((int64_t)1 << 31) || k < 1 || k > 16 || k > E || (x_mode != 0 && x_mode != 1))
        return KQ_ERR_ARG;
    if (!W_exps || !y) return KQ_ERR_NULL;
    if (N == 0) return KQ_OK;
    if (!ids || !x) return KQ_ERR_NULL;
    MoeSet set = {};
    for (int i = 0; i < count; ++i) {
        if (!W_exps[i] || !y[i]) return KQ_ERR_NULL;
        if (!aligned(W_exps[i], 16) || !aligned(y[i], 16)) return KQ_ERR_ALIGN;
        set.W[i] = (const uint8_t *)W_exps[i];
        set.y[i] = y[i];
    }
    set.n = count;
    if (!aligned(x, 16) || !aligned(ids, 4) || (err_flag && !aligned(err_flag, 4))) return KQ_ERR_ALIGN;
    if (device_check()) return KQ_ERR_DEVICE;
    return with_type(type, [&](auto tag) {
        constexpr int TT = decltype(tag)::value;
        const int rt = launch_qmoe_tok_t<TT>(set, row_bytes, (int)E, (int)N, (int)K, ids, nullptr, T, k, x, x_mode,
                                             err_flag, (hipStream_t)stream);
        if (rt != KQ_ERR_ARG) return rt;
        return launch_qmoe_m<TT>(T, set, row_bytes, (int)E, (int)N, (int)K, ids, T, k, x, x_mode, err_flag,
                                 (hipStream_t)stream);
    });
}

} // extern "C"
