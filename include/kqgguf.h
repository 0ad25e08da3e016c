/*
 * kqgguf.h -- C ABI of the GGUF reader in libkqgemv.so: the tensor table and
 * metadata of a GGUF model file, and its tensor data handed to the GEMV calls
 * of kqgemv.h byte for byte, with no conversion.
 *
 * Why it is here.  The pages describe engines that parse GGUF files with
 * their own code (Kortex summary, section Key points; "Kortex: Streaming 70B
 * Models on Consumer GPUs", section on what makes it original) and keep the
 * weights file-backed through a memory map, using the file on disk as the only
 * copy of the weights -- no converted cache ("RunNburn - Run a 295B Moe from a
 * 98GB GGUF on a 64GB RAM Desktop").  The packed blocks a GGUF file stores are
 * exactly the blocks kq_qgemv / kq_qmoe_gemv / kq_dequant read, so a tensor is
 * uploaded as it is and used directly.
 *
 * File layout read (GGUF versions 2 and 3, little-endian; the pages name the
 * format but print no layout, so this is the published GGUF convention):
 *   "GGUF" magic, u32 version, u64 tensor count, u64 metadata count;
 *   metadata: key (u64 length + bytes), u32 value type, value, where a value is
 *     u8 i8 u16 i16 u32 i32 f32 bool(u8) string u64 i64 f64 (types 0..12 in
 *     the order u8=0, i8=1, u16=2, i16=3, u32=4, i32=5, f32=6, bool=7,
 *     string=8, array=9, u64=10, i64=11, f64=12) or an array (u32 element
 *     type, u64 count, elements);
 *   tensor table: name (string), u32 dimension count (1..4), u64 dims (dims[0]
 *     varies fastest: for a matrix, dims[0] = K columns and dims[1] = N rows),
 *     u32 tensor type, u64 offset relative to the data section;
 *   padding to `general.alignment` (u32 metadata, default 32), then the data
 *   section; every tensor offset is a multiple of the alignment.
 *
 * Conventions:
 *  - kq_gguf_open maps the file read-only and parses it completely; every read
 *    is bounds-checked against the file size, so a truncated or malformed file
 *    is rejected with KQ_ERR_FORMAT and never read past its end.
 *  - The handle owns its strings and tables; pointers it returns stay valid
 *    until kq_gguf_close.  A handle may be read from several threads at once;
 *    open and close are not concurrent with other calls on the same handle.
 *  - Errors are negative kq_status values (kqgemv.h), plus KQ_ERR_IO when the
 *    file cannot be opened or mapped.
 */
#ifndef KQGGUF_H
#define KQGGUF_H

#include <stddef.h>
#include <stdint.h>

#include "kqgemv.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kq_gguf kq_gguf;

/* One entry of the tensor table. */
typedef struct kq_gguf_tensor {
    const char *name;   /* NUL-terminated; owned by the handle                 */
    int type;           /* tensor type id (kq_type for the GEMV formats)       */
    int n_dims;         /* 1..4                                                */
    int64_t dims[4];    /* dims[0] fastest; entries past n_dims are 1          */
    uint64_t offset;    /* absolute byte offset of the data in the file        */
    uint64_t nbytes;    /* bytes of data; 0 when the type's size is not known  */
    const void *data;   /* host address of the data inside the mapping         */
} kq_gguf_tensor;

/* Metadata value types (the GGUF numbering). */
typedef enum kq_gguf_value_type {
    KQ_GGUF_U8 = 0, KQ_GGUF_I8 = 1, KQ_GGUF_U16 = 2, KQ_GGUF_I16 = 3, KQ_GGUF_U32 = 4,
    KQ_GGUF_I32 = 5, KQ_GGUF_F32 = 6, KQ_GGUF_BOOL = 7, KQ_GGUF_STRING = 8, KQ_GGUF_ARRAY = 9,
    KQ_GGUF_U64 = 10, KQ_GGUF_I64 = 11, KQ_GGUF_F64 = 12
} kq_gguf_value_type;

/* Open and parse `path`; *out receives the handle (NULL on failure).
 * Returns KQ_OK, KQ_ERR_NULL, KQ_ERR_IO (open/stat/mmap failed) or
 * KQ_ERR_FORMAT (bad magic, unsupported version, a value or table entry that
 * runs past the end of the file, an unknown value type, a bad alignment, a
 * misaligned offset, a dimension that is not a whole number of blocks, tensor
 * data past the end of the file, or a key or tensor name holding a NUL byte,
 * which could not be looked up as a C string). */
int kq_gguf_open(const char *path, kq_gguf **out);

/* Unmap and free.  NULL is a no-op. */
void kq_gguf_close(kq_gguf *g);

/* Format version (2 or 3) and data alignment of an open file. */
int kq_gguf_version(const kq_gguf *g);
int64_t kq_gguf_alignment(const kq_gguf *g);

/* Number of tensors; index of the tensor named `name`, or KQ_ERR_ARG if there
 * is none (KQ_ERR_NULL for NULL arguments). */
int64_t kq_gguf_tensor_count(const kq_gguf *g);
int64_t kq_gguf_find_tensor(const kq_gguf *g, const char *name);

/* Table entry i (0 <= i < count) into *out.  KQ_ERR_ARG for a bad index. */
int kq_gguf_tensor_info(const kq_gguf *g, int64_t i, kq_gguf_tensor *out);

/* Copy the data of tensor i (nbytes bytes) into device memory at `dst`, on
 * `stream` (a hipStream_t as void*, NULL = null stream).  The source is the
 * mapped file (pageable memory), so the call returns once the bytes have been
 * handed to the runtime; the copy is ordered on `stream` before later work.
 * KQ_ERR_ARG for a bad index or a tensor of unknown size, KQ_ERR_LAUNCH if the
 * copy fails. */
int kq_gguf_upload(const kq_gguf *g, int64_t i, void *dst, void *stream);

/* Metadata.  Keys are matched exactly.  KQ_ERR_ARG when the key is absent or
 * its value does not have a matching type. */
int64_t kq_gguf_meta_count(const kq_gguf *g);
int kq_gguf_meta_key(const kq_gguf *g, int64_t i, const char **key, int *value_type);
/* integer or bool values (u64 values above INT64_MAX are KQ_ERR_ARG) */
int kq_gguf_meta_int(const kq_gguf *g, const char *key, int64_t *out);
/* f32 or f64 values */
int kq_gguf_meta_float(const kq_gguf *g, const char *key, double *out);
/* string values: *out points into the mapping (not NUL-terminated) */
int kq_gguf_meta_string(const kq_gguf *g, const char *key, const char **out, uint64_t *len);
/* arrays: element type and count; for fixed-size element types *data points
 * at the packed little-endian elements inside the mapping, for strings and
 * nested arrays it is NULL (use kq_gguf_meta_array_string for strings). */
int kq_gguf_meta_array(const kq_gguf *g, const char *key, int *elem_type, uint64_t *count,
                       const void **data);
/* element j of a string array */
int kq_gguf_meta_array_string(const kq_gguf *g, const char *key, uint64_t j, const char **out,
                              uint64_t *len);

#ifdef __cplusplus
}
#endif

#endif /* KQGGUF_H */
