"""Fused GGUF K-quant dequant-GEMV for AMD MI355X (gfx950).

A thin ctypes binding of ``libkqgemv.so`` whose C ABI is declared in
``include/kqgemv.h``, ``include/kqgguf.h`` and ``include/kqstream.h``.  The functions keep the C names and only marshal
arguments (torch tensors -> device pointers, the current torch stream ->
hipStream_t); every step of the computation runs in the HIP kernels.  There is
no fallback: if the shared library is missing, loading it raises.
"""
from ._binding import (  # noqa: F401
    GGUFTensor,
    KQError,
    KQ_TYPE_Q2_K,
    KQ_TYPE_Q3_K,
    KQ_TYPE_Q4_0,
    KQ_TYPE_Q4_K,
    KQ_TYPE_Q5_K,
    KQ_TYPE_Q6_K,
    KQ_TYPE_Q8_0,
    STATUS,
    kq_block_info,
    kq_dequant,
    kq_gguf_alignment,
    kq_gguf_close,
    kq_gguf_find_tensor,
    kq_gguf_meta_array,
    kq_gguf_meta_array_string,
    kq_gguf_meta_count,
    kq_gguf_meta_float,
    kq_gguf_meta_int,
    kq_gguf_meta_key,
    kq_gguf_meta_string,
    kq_gguf_open,
    kq_gguf_tensor_count,
    kq_gguf_tensor_info,
    kq_gguf_upload,
    kq_gguf_version,
    kq_qgemv,
    kq_qgemv_multi,
    kq_qmoe_gemv,
    kq_qmoe_gemv_multi,
    kq_qmoe_gemv_noalloc,
    kq_qmoe_workspace_bytes,
    kq_row_bytes,
    kq_stream_qgemv,
    kq_stream_qgemv_multi,
    kq_streamer_create,
    kq_streamer_destroy,
    kq_streamer_sync,
    kq_status_string,
    kq_version,
    lib,
    lib_path,
)
