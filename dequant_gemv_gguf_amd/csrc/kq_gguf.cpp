// kq_gguf.cpp -- GGUF reader of libkqgemv.so (C ABI in include/kqgguf.h).
//
// The file is mapped read-only and stays the only copy of the weights (the
// RunNburn post: weights stay file-backed through mmap, no conversion step);
// the header, metadata and tensor table are parsed once at open with every
// read checked against the file size.  Tensor data is handed to the GEMV calls
// byte for byte: a GGUF tensor of a K-quant type is already the row-major
// block matrix kq_qgemv reads.
#include <hip/hip_runtime_api.h>

#include <fcntl.h>
#include <string.h>
#include <sys/mman.h>
#include <sys/stat.h>
#include <unistd.h>

#include <new>
#include <string>
#include <vector>

#include "kqgguf.h"

namespace {

// Elements per block and bytes per block of the tensor types whose size is
// known here (the GGUF/ggml type numbering); {0, 0} for the others.
struct TypeSize {
    int blck, bytes;
};
TypeSize type_size(uint32_t t) {
    switch (t) {
    case 0: return {1, 4};       // F32
    case 1: return {1, 2};       // F16
    case 2: return {32, 18};     // Q4_0
    case 3: return {32, 20};     // Q4_1
    case 6: return {32, 22};     // Q5_0
    case 7: return {32, 24};     // Q5_1
    case 8: return {32, 34};     // Q8_0
    case 9: return {32, 36};     // Q8_1
    case 10: return {256, 84};   // Q2_K
    case 11: return {256, 110};  // Q3_K
    case 12: return {256, 144};  // Q4_K
    case 13: return {256, 176};  // Q5_K
    case 14: return {256, 210};  // Q6_K
    case 15: return {256, 292};  // Q8_K
    case 24: return {1, 1};      // I8
    case 25: return {1, 2};      // I16
    case 26: return {1, 4};      // I32
    case 27: return {1, 8};      // I64
    case 28: return {1, 8};      // F64
    case 30: return {1, 2};      // BF16
    default: return {0, 0};
    }
}

// Size in bytes of a fixed-size metadata value type; 0 for string and array.
uint64_t value_size(uint32_t vt) {
    switch (vt) {
    case KQ_GGUF_U8: case KQ_GGUF_I8: case KQ_GGUF_BOOL: return 1;
    case KQ_GGUF_U16: case KQ_GGUF_I16: return 2;
    case KQ_GGUF_U32: case KQ_GGUF_I32: case KQ_GGUF_F32: return 4;
    case KQ_GGUF_U64: case KQ_GGUF_I64: case KQ_GGUF_F64: return 8;
    default: return 0;
    }
}

struct Meta {
    std::string key;
    uint32_t type;        // value type
    uint64_t pos;         // file offset of the value (after the type field)
    uint32_t elem_type;   // arrays: element type
    uint64_t count;       // arrays: element count
    std::vector<uint64_t> str_pos;   // string arrays: offset of each element's length field
};

struct Tensor {
    std::string name;
    uint32_t type;
    int n_dims;
    int64_t dims[4];
    uint64_t rel;         // offset relative to the data section
    uint64_t offset;      // absolute offset
    uint64_t nbytes;
};

// Little-endian reads with bounds checks; any failure latches `bad`.
struct Cursor {
    const uint8_t *base;
    uint64_t size, pos;
    bool bad;
    bool need(uint64_t n) {
        if (bad || n > size || pos > size - n) bad = true;
        return !bad;
    }
    uint64_t uint(int nb) {
        if (!need((uint64_t)nb)) return 0;
        uint64_t v = 0;
        for (int i = 0; i < nb; ++i) v |= (uint64_t)base[pos + i] << (8 * i);
        pos += (uint64_t)nb;
        return v;
    }
    uint32_t u32() { return (uint32_t)uint(4); }
    uint64_t u64() { return uint(8); }
    // a string: u64 length then bytes; returns the offset of the bytes
    uint64_t str(uint64_t *len) {
        *len = u64();
        const uint64_t at = pos;
        if (need(*len)) pos += *len;
        return at;
    }
    void skip(uint64_t n) {
        if (need(n)) pos += n;
    }
};

uint64_t load_le(const uint8_t *p, int nb) {
    uint64_t v = 0;
    for (int i = 0; i < nb; ++i) v |= (uint64_t)p[i] << (8 * i);
    return v;
}

} // namespace

struct kq_gguf {
    int fd = -1;
    const uint8_t *map = nullptr;
    uint64_t size = 0;
    uint32_t version = 0;
    uint64_t alignment = 32;
    uint64_t data_start = 0;
    std::vector<Meta> meta;
    std::vector<Tensor> tensors;

    const Meta *find_meta(const char *key) const {
        for (const Meta &m : meta)
            if (m.key == key) return &m;
        return nullptr;
    }
};

namespace {

// Skip one value of type vt at the cursor (nested arrays allowed, depth-limited).
void skip_value(Cursor &c, uint32_t vt, int depth) {
    if (c.bad) return;
    if (vt == KQ_GGUF_STRING) {
        uint64_t len;
        c.str(&len);
    } else if (vt == KQ_GGUF_ARRAY) {
        const uint32_t et = c.u32();
        const uint64_t n = c.u64();
        if (c.bad || depth > 8) {
            c.bad = true;
            return;
        }
        const uint64_t es = value_size(et);
        if (es) {
            if (n > (c.size - c.pos) / es) c.bad = true;
            else c.skip(n * es);
        } else if (et == KQ_GGUF_STRING || et == KQ_GGUF_ARRAY) {
            // each element takes at least 8 bytes (its length or header)
            if (n > (c.size - c.pos) / 8) c.bad = true;
            for (uint64_t i = 0; i < n && !c.bad; ++i) skip_value(c, et, depth + 1);
        } else {
            c.bad = true;
        }
    } else {
        const uint64_t vs = value_size(vt);
        if (!vs) c.bad = true;
        else c.skip(vs);
    }
}

int parse(kq_gguf *g) {
    Cursor c{g->map, g->size, 0, false};
    const uint32_t magic = c.u32();
    if (c.bad || magic != 0x46554747u) return KQ_ERR_FORMAT;   // "GGUF"
    g->version = c.u32();
    if (g->version != 2 && g->version != 3) return KQ_ERR_FORMAT;
    const uint64_t n_tensors = c.u64(), n_kv = c.u64();
    if (c.bad) return KQ_ERR_FORMAT;
    // every entry takes at least 12 bytes of the file
    if (n_kv > g->size / 12 || n_tensors > g->size / 12) return KQ_ERR_FORMAT;
    for (uint64_t i = 0; i < n_kv; ++i) {
        Meta m;
        uint64_t klen;
        const uint64_t kat = c.str(&klen);
        m.type = c.u32();
        if (c.bad) return KQ_ERR_FORMAT;
        // keys and names are looked up as C strings: an embedded NUL is malformed
        if (memchr(g->map + kat, 0, (size_t)klen)) return KQ_ERR_FORMAT;
        m.key.assign((const char *)g->map + kat, (size_t)klen);
        m.pos = c.pos;
        m.elem_type = 0;
        m.count = 0;
        if (m.type == KQ_GGUF_ARRAY) {
            m.elem_type = c.u32();
            m.count = c.u64();
            if (c.bad) return KQ_ERR_FORMAT;
            if (m.elem_type == KQ_GGUF_STRING) {
                if (m.count > (c.size - c.pos) / 8) return KQ_ERR_FORMAT;
                for (uint64_t j = 0; j < m.count && !c.bad; ++j) {
                    m.str_pos.push_back(c.pos);
                    uint64_t l;
                    c.str(&l);
                }
            } else {
                c.pos = m.pos;
                skip_value(c, KQ_GGUF_ARRAY, 0);
            }
        } else {
            skip_value(c, m.type, 0);
        }
        if (c.bad) return KQ_ERR_FORMAT;
        g->meta.push_back(std::move(m));
    }
    if (const Meta *a = g->find_meta("general.alignment")) {
        if (a->type != KQ_GGUF_U32) return KQ_ERR_FORMAT;
        const uint64_t al = load_le(g->map + a->pos, 4);
        if (al == 0 || (al & (al - 1)) != 0) return KQ_ERR_FORMAT;
        g->alignment = al;
    }
    for (uint64_t i = 0; i < n_tensors; ++i) {
        Tensor t;
        uint64_t nlen;
        const uint64_t nat = c.str(&nlen);
        const uint32_t nd = c.u32();
        if (c.bad || nd < 1 || nd > 4) return KQ_ERR_FORMAT;
        if (memchr(g->map + nat, 0, (size_t)nlen)) return KQ_ERR_FORMAT;
        t.name.assign((const char *)g->map + nat, (size_t)nlen);
        t.n_dims = (int)nd;
        for (int d = 0; d < 4; ++d) t.dims[d] = 1;
        for (uint32_t d = 0; d < nd; ++d) {
            const uint64_t v = c.u64();
            if (v > ((uint64_t)1 << 40)) return KQ_ERR_FORMAT;
            t.dims[d] = (int64_t)v;
        }
        t.type = c.u32();
        t.rel = c.u64();
        if (c.bad) return KQ_ERR_FORMAT;
        if (t.rel % g->alignment) return KQ_ERR_FORMAT;
        const TypeSize ts = type_size(t.type);
        t.nbytes = 0;
        if (ts.blck) {
            if (t.dims[0] % ts.blck) return KQ_ERR_FORMAT;
            // rows * blocks per row * block bytes, each factor bounded above
            unsigned __int128 n = (unsigned __int128)(t.dims[0] / ts.blck) * (uint64_t)ts.bytes;
            for (int d = 1; d < 4; ++d) n *= (uint64_t)t.dims[d];
            if (n > (unsigned __int128)g->size) return KQ_ERR_FORMAT;
            t.nbytes = (uint64_t)n;
        }
        g->tensors.push_back(std::move(t));
    }
    // the data section starts at the next multiple of the alignment
    const uint64_t start = (c.pos + g->alignment - 1) / g->alignment * g->alignment;
    if (n_tensors && start > g->size) return KQ_ERR_FORMAT;
    g->data_start = start;
    for (Tensor &t : g->tensors) {
        if (t.rel > g->size - start) return KQ_ERR_FORMAT;
        t.offset = start + t.rel;
        if (t.nbytes > g->size - t.offset) return KQ_ERR_FORMAT;
    }
    return KQ_OK;
}

} // namespace

extern "C" {

int kq_gguf_open(const char *path, kq_gguf **out) {
    if (!out) return KQ_ERR_NULL;
    *out = nullptr;
    if (!path) return KQ_ERR_NULL;
    kq_gguf *g = new (std::nothrow) kq_gguf;
    if (!g) return KQ_ERR_IO;
    g->fd = open(path, O_RDONLY | O_CLOEXEC);
    struct stat st;
    if (g->fd < 0 || fstat(g->fd, &st) != 0 || !S_ISREG(st.st_mode)) {
        kq_gguf_close(g);
        return KQ_ERR_IO;
    }
    if (st.st_size < 24) {                       // shorter than the fixed header
        kq_gguf_close(g);
        return KQ_ERR_FORMAT;
    }
    g->size = (uint64_t)st.st_size;
    void *m = mmap(nullptr, (size_t)g->size, PROT_READ, MAP_PRIVATE, g->fd, 0);
    if (m == MAP_FAILED) {
        kq_gguf_close(g);
        return KQ_ERR_IO;
    }
    g->map = (const uint8_t *)m;
    int r;
    try {
        r = parse(g);
    } catch (const std::bad_alloc &) {
        r = KQ_ERR_FORMAT;
    }
    if (r != KQ_OK) {
        kq_gguf_close(g);
        return r;
    }
    *out = g;
    return KQ_OK;
}

void kq_gguf_close(kq_gguf *g) {
    if (!g) return;
    if (g->map) munmap(const_cast<uint8_t *>(g->map), (size_t)g->size);
    if (g->fd >= 0) close(g->fd);
    delete g;
}

int kq_gguf_version(const kq_gguf *g) { return g ? (int)g->version : KQ_ERR_NULL; }

int64_t kq_gguf_alignment(const kq_gguf *g) { return g ? (int64_t)g->alignment : KQ_ERR_NULL; }

int64_t kq_gguf_tensor_count(const kq_gguf *g) { return g ? (int64_t)g->tensors.size() : KQ_ERR_NULL; }

int64_t kq_gguf_find_tensor(const kq_gguf *g, const char *name) {
    if (!g || !name) return KQ_ERR_NULL;
    for (size_t i = 0; i < g->tensors.size(); ++i)
        if (g->tensors[i].name == name) return (int64_t)i;
    return KQ_ERR_ARG;
}

int kq_gguf_tensor_info(const kq_gguf *g, int64_t i, kq_gguf_tensor *out) {
    if (!g || !out) return KQ_ERR_NULL;
    if (i < 0 || (uint64_t)i >= g->tensors.size()) return KQ_ERR_ARG;
    const Tensor &t = g->tensors[(size_t)i];
    out->name = t.name.c_str();
    out->type = (int)t.type;
    out->n_dims = t.n_dims;
    for (int d = 0; d < 4; ++d) out->dims[d] = t.dims[d];
    out->offset = t.offset;
    out->nbytes = t.nbytes;
    out->data = g->map + t.offset;
    return KQ_OK;
}

int kq_gguf_upload(const kq_gguf *g, int64_t i, void *dst, void *stream) {
    if (!g || !dst) return KQ_ERR_NULL;
    if (i < 0 || (uint64_t)i >= g->tensors.size()) return KQ_ERR_ARG;
    const Tensor &t = g->tensors[(size_t)i];
    if (t.nbytes == 0 && type_size(t.type).blck == 0) return KQ_ERR_ARG;
    if (t.nbytes == 0) return KQ_OK;
    const hipError_t e = hipMemcpyAsync(dst, g->map + t.offset, (size_t)t.nbytes, hipMemcpyHostToDevice,
                                        (hipStream_t)stream);
    return e == hipSuccess ? KQ_OK : KQ_ERR_LAUNCH;
}

int64_t kq_gguf_meta_count(const kq_gguf *g) { return g ? (int64_t)g->meta.size() : KQ_ERR_NULL; }

int kq_gguf_meta_key(const kq_gguf *g, int64_t i, const char **key, int *value_type) {
    if (!g || !key || !value_type) return KQ_ERR_NULL;
    if (i < 0 || (uint64_t)i >= g->meta.size()) return KQ_ERR_ARG;
    *key = g->meta[(size_t)i].key.c_str();
    *value_type = (int)g->meta[(size_t)i].type;
    return KQ_OK;
}

int kq_gguf_meta_int(const kq_gguf *g, const char *key, int64_t *out) {
    if (!g || !key || !out) return KQ_ERR_NULL;
    const Meta *m = g->find_meta(key);
    if (!m) return KQ_ERR_ARG;
    const uint8_t *p = g->map + m->pos;
    switch (m->type) {
    case KQ_GGUF_U8: case KQ_GGUF_BOOL: *out = (int64_t)p[0]; return KQ_OK;
    case KQ_GGUF_I8: *out = (int64_t)(int8_t)p[0]; return KQ_OK;
    case KQ_GGUF_U16: *out = (int64_t)load_le(p, 2); return KQ_OK;
    case KQ_GGUF_I16: *out = (int64_t)(int16_t)load_le(p, 2); return KQ_OK;
    case KQ_GGUF_U32: *out = (int64_t)load_le(p, 4); return KQ_OK;
    case KQ_GGUF_I32: *out = (int64_t)(int32_t)load_le(p, 4); return KQ_OK;
    case KQ_GGUF_I64: *out = (int64_t)load_le(p, 8); return KQ_OK;
    case KQ_GGUF_U64: {
        const uint64_t v = load_le(p, 8);
        if (v > (uint64_t)INT64_MAX) return KQ_ERR_ARG;
        *out = (int64_t)v;
        return KQ_OK;
    }
    default: return KQ_ERR_ARG;
    }
}

int kq_gguf_meta_float(const kq_gguf *g, const char *key, double *out) {
    if (!g || !key || !out) return KQ_ERR_NULL;
    const Meta *m = g->find_meta(key);
    if (!m) return KQ_ERR_ARG;
    const uint8_t *p = g->map + m->pos;
    if (m->type == KQ_GGUF_F32) {
        const uint32_t b = (uint32_t)load_le(p, 4);
        float f;
        memcpy(&f, &b, 4);
        *out = f;
        return KQ_OK;
    }
    if (m->type == KQ_GGUF_F64) {
        const uint64_t b = load_le(p, 8);
        memcpy(out, &b, 8);
        return KQ_OK;
    }
    return KQ_ERR_ARG;
}

int kq_gguf_meta_string(const kq_gguf *g, const char *key, const char **out, uint64_t *len) {
    if (!g || !key || !out || !len) return KQ_ERR_NULL;
    const Meta *m = g->find_meta(key);
    if (!m || m->type != KQ_GGUF_STRING) return KQ_ERR_ARG;
    *len = load_le(g->map + m->pos, 8);
    *out = (const char *)g->map + m->pos + 8;
    return KQ_OK;
}

int kq_gguf_meta_array(const kq_gguf *g, const char *key, int *elem_type, uint64_t *count, const void **data) {
    if (!g || !key || !elem_type || !count || !data) return KQ_ERR_NULL;
    const Meta *m = g->find_meta(key);
    if (!m || m->type != KQ_GGUF_ARRAY) return KQ_ERR_ARG;
    *elem_type = (int)m->elem_type;
    *count = m->count;
    *data = value_size(m->elem_type) ? (const void *)(g->map + m->pos + 12) : nullptr;
    return KQ_OK;
}

int kq_gguf_meta_array_string(const kq_gguf *g, const char *key, uint64_t j, const char **out, uint64_t *len) {
    if (!g || !key || !out || !len) return KQ_ERR_NULL;
    const Meta *m = g->find_meta(key);
    if (!m || m->type != KQ_GGUF_ARRAY || m->elem_type != KQ_GGUF_STRING || j >= m->count) return KQ_ERR_ARG;
    const uint64_t at = m->str_pos[(size_t)j];
    *len = load_le(g->map + at, 8);
    *out = (const char *)g->map + at + 8;
    return KQ_OK;
}

} // extern "C"
