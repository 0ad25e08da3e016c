// Host-only driver for the GGUF reader's memory-safety test: built with the
// address and undefined-behaviour sanitizers together with
// dequant_gemv_gguf_amd/csrc/kq_gguf.cpp, it opens every file named on the
// command line and reads everything the C ABI exposes.  A file must either be
// rejected (KQ_ERR_FORMAT) or open and be read without any invalid access;
// the sanitizers abort the process on the first one.  The GPU copy is not
// exercised: hipMemcpyAsync is a stub here, so no HIP runtime is loaded.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstring>

#include "kqgguf.h"

hipError_t hipMemcpyAsync(void *, const void *, size_t, hipMemcpyKind, hipStream_t) { return hipSuccess; }

static unsigned long long touch(const void *p, uint64_t n) {
    unsigned long long h = 0;
    const unsigned char *b = static_cast<const unsigned char *>(p);
    for (uint64_t i = 0; i < n; ++i) h = h * 131 + b[i];
    return h;
}

int main(int argc, char **argv) {
    int opened = 0, rejected = 0;
    unsigned long long h = 0;
    for (int a = 1; a < argc; ++a) {
        kq_gguf *g = nullptr;
        const int r = kq_gguf_open(argv[a], &g);
        if (r != KQ_OK) {
            if (r != KQ_ERR_FORMAT) {
                std::fprintf(stderr, "%s: unexpected status %d\n", argv[a], r);
                return 2;
            }
            ++rejected;
            continue;
        }
        ++opened;
        h += (unsigned long long)kq_gguf_version(g) + (unsigned long long)kq_gguf_alignment(g);
        const int64_t nt = kq_gguf_tensor_count(g);
        for (int64_t i = 0; i < nt; ++i) {
            kq_gguf_tensor t;
            if (kq_gguf_tensor_info(g, i, &t) != KQ_OK) return 3;
            h += touch(t.name, std::strlen(t.name)) + touch(t.data, t.nbytes);
            if (kq_gguf_find_tensor(g, t.name) < 0) return 4;
            char dummy[16];
            if (t.nbytes) (void)kq_gguf_upload(g, i, dummy, nullptr);
        }
        const int64_t nm = kq_gguf_meta_count(g);
        for (int64_t i = 0; i < nm; ++i) {
            const char *key;
            int vt;
            if (kq_gguf_meta_key(g, i, &key, &vt) != KQ_OK) return 5;
            int64_t iv;
            double fv;
            const char *sv;
            uint64_t len, cnt;
            int et;
            const void *data;
            if (kq_gguf_meta_int(g, key, &iv) == KQ_OK) h += (unsigned long long)iv;
            if (kq_gguf_meta_float(g, key, &fv) == KQ_OK) h += (unsigned long long)(fv != fv);
            if (kq_gguf_meta_string(g, key, &sv, &len) == KQ_OK) h += touch(sv, len);
            if (kq_gguf_meta_array(g, key, &et, &cnt, &data) == KQ_OK) {
                if (et == KQ_GGUF_STRING) {
                    for (uint64_t j = 0; j < cnt; ++j)
                        if (kq_gguf_meta_array_string(g, key, j, &sv, &len) == KQ_OK) h += touch(sv, len);
                } else if (data) {
                    const uint64_t es = et == KQ_GGUF_U8 || et == KQ_GGUF_I8 || et == KQ_GGUF_BOOL ? 1
                                        : et == KQ_GGUF_U16 || et == KQ_GGUF_I16                 ? 2
                                        : et == KQ_GGUF_U64 || et == KQ_GGUF_I64 || et == KQ_GGUF_F64 ? 8 : 4;
                    h += touch(data, cnt * es);
                }
            }
        }
        kq_gguf_close(g);
    }
    std::printf("opened %d rejected %d digest %llu\n", opened, rejected, h);
    return 0;
}
