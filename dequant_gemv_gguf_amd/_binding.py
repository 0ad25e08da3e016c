"""ctypes marshalling for libkqgemv.so (see include/kqgemv.h for semantics)."""
import ctypes
import os

KQ_TYPE_Q4_0, KQ_TYPE_Q8_0, KQ_TYPE_Q2_K, KQ_TYPE_Q3_K = 2, 8, 10, 11
KQ_TYPE_Q4_K, KQ_TYPE_Q5_K, KQ_TYPE_Q6_K = 12, 13, 14

STATUS = {
    0: "KQ_OK", -1: "KQ_ERR_TYPE", -2: "KQ_ERR_SHAPE", -3: "KQ_ERR_M", -4: "KQ_ERR_NULL",
    -5: "KQ_ERR_ALIGN", -6: "KQ_ERR_ARG", -7: "KQ_ERR_LAUNCH", -8: "KQ_ERR_DEVICE",
    -9: "KQ_ERR_IO", -10: "KQ_ERR_FORMAT",
}

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libkqgemv.so")

_lib = None


class GGUFTensor(ctypes.Structure):
    """struct kq_gguf_tensor (include/kqgguf.h)."""
    _fields_ = [("name", ctypes.c_char_p), ("type", ctypes.c_int), ("n_dims", ctypes.c_int),
                ("dims", ctypes.c_int64 * 4), ("offset", ctypes.c_uint64), ("nbytes", ctypes.c_uint64),
                ("data", ctypes.c_void_p)]


class KQError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (fn, kq_status_string(status), status))


def lib():
    """Load the in-tree shared library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise ImportError("libkqgemv.so is not built; run __graft_entry__.build() or "
                              "python dequant_gemv_gguf_amd/build.py")
        L = ctypes.CDLL(lib_path)
        P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        L.kq_version.restype = I
        L.kq_status_string.argtypes = [I]
        L.kq_status_string.restype = ctypes.c_char_p
        L.kq_block_info.argtypes = [I, P, P]
        L.kq_row_bytes.argtypes = [I, I64]
        L.kq_row_bytes.restype = I64
        L.kq_dequant.argtypes = [I, P, I64, P, P]
        L.kq_qgemv.argtypes = [I, P, I64, I64, P, I, P, P]
        L.kq_qgemv_multi.argtypes = [I, P, P, P, I64, P, I, P, P]
        L.kq_qgemv_mc_multi.argtypes = [I, P, P, P, I64, P, I, P, P]
        L.kq_qgemv_mc.argtypes = [I, P, I64, I64, P, I, P, P]
        L.kq_qmoe_workspace_bytes.argtypes = [I, I, I64]
        L.kq_qmoe_workspace_bytes.restype = ctypes.c_size_t
        L.kq_qmoe_gemv.argtypes = [I, P, I64, I64, I64, P, P, I, I, P, I, P, P, P, P]
        L.kq_qmoe_gemv_multi.argtypes = [I, I, P, I64, I64, I64, P, I, I, P, I, P, P, P]
        L.kq_qmoe_gemv_noalloc.argtypes = [I, P, I64, I64, I64, P, P, I, I, P, I, P, P, P]
        U64, CP = ctypes.c_uint64, ctypes.c_char_p
        L.kq_gguf_open.argtypes = [CP, ctypes.POINTER(P)]
        L.kq_gguf_close.argtypes = [P]
        L.kq_gguf_close.restype = None
        L.kq_gguf_version.argtypes = [P]
        L.kq_gguf_alignment.argtypes = [P]
        L.kq_gguf_alignment.restype = I64
        L.kq_gguf_tensor_count.argtypes = [P]
        L.kq_gguf_tensor_count.restype = I64
        L.kq_gguf_find_tensor.argtypes = [P, CP]
        L.kq_gguf_find_tensor.restype = I64
        L.kq_gguf_tensor_info.argtypes = [P, I64, ctypes.POINTER(GGUFTensor)]
        L.kq_gguf_upload.argtypes = [P, I64, P, P]
        L.kq_gguf_meta_count.argtypes = [P]
        L.kq_gguf_meta_count.restype = I64
        L.kq_gguf_meta_key.argtypes = [P, I64, ctypes.POINTER(CP), ctypes.POINTER(I)]
        L.kq_gguf_meta_int.argtypes = [P, CP, ctypes.POINTER(I64)]
        L.kq_gguf_meta_float.argtypes = [P, CP, ctypes.POINTER(ctypes.c_double)]
        L.kq_gguf_meta_string.argtypes = [P, CP, ctypes.POINTER(P), ctypes.POINTER(U64)]
        L.kq_gguf_meta_array.argtypes = [P, CP, ctypes.POINTER(I), ctypes.POINTER(U64), ctypes.POINTER(P)]
        L.kq_gguf_meta_array_string.argtypes = [P, CP, U64, ctypes.POINTER(P), ctypes.POINTER(U64)]
        L.kq_streamer_create.argtypes = [P, ctypes.c_size_t, I, P, ctypes.POINTER(P)]
        L.kq_streamer_destroy.argtypes = [P]
        L.kq_streamer_destroy.restype = None
        L.kq_streamer_sync.argtypes = [P]
        L.kq_stream_qgemv_multi.argtypes = [P, I, P, P, P, I64, P, I, P]
        L.kq_stream_qgemv.argtypes = [P, I, P, I64, I64, P, I, P]
        _lib = L
    return _lib


def _ptr(t):
    """Device pointer of a torch tensor, an int address, or None (NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream, like):
    if stream is not None:
        return ctypes.c_void_p(stream if isinstance(stream, int) else stream.cuda_stream)
    if like is not None and not isinstance(like, int) and like.is_cuda:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream(like.device).cuda_stream)
    return None


def _check(fn, r):
    if r != 0:
        raise KQError(fn, r)


def kq_version():
    return lib().kq_version()


def kq_status_string(status):
    return lib().kq_status_string(int(status)).decode()


def kq_block_info(qtype):
    qk, nb = ctypes.c_int(), ctypes.c_int()
    _check("kq_block_info", lib().kq_block_info(int(qtype), ctypes.byref(qk), ctypes.byref(nb)))
    return qk.value, nb.value


def kq_row_bytes(qtype, K):
    r = lib().kq_row_bytes(int(qtype), int(K))
    if r < 0:
        raise KQError("kq_row_bytes", int(r))
    return int(r)


def kq_dequant(qtype, src, n_elems, dst, stream=None):
    _check("kq_dequant", lib().kq_dequant(int(qtype), _ptr(src), int(n_elems), _ptr(dst),
                                          _stream(stream, dst)))


def kq_qgemv(qtype, W, N, K, x, M, y, stream=None):
    _check("kq_qgemv", lib().kq_qgemv(int(qtype), _ptr(W), int(N), int(K), _ptr(x), int(M), _ptr(y),
                                      _stream(stream, y)))


def _addr(t):
    if t is None:
        return 0
    return t if isinstance(t, int) else t.data_ptr()


def kq_qgemv_multi(types, Ws, Ns, K, x, M, ys, stream=None):
    """types: one kq_type for every matrix, or a sequence of them; Ws, Ns, ys:
    equal-length sequences (tensors or int addresses, row counts, tensors or
    int addresses), marshalled into the host arrays the C call takes."""
    count = len(Ws)
    if isinstance(types, int):
        types = [types] * count
    if len(types) != count or len(Ns) != count or len(ys) != count:
        raise ValueError("kq_qgemv_multi: types, Ws, Ns and ys must have the same length")
    n = max(count, 1)
    Ta = (ctypes.c_int * n)(*[int(t) for t in types])
    Wa = (ctypes.c_void_p * n)(*[_addr(w) for w in Ws])
    Na = (ctypes.c_int64 * n)(*[int(v) for v in Ns])
    Ya = (ctypes.c_void_p * n)(*[_addr(y) for y in ys])
    like = next((y for y in ys if y is not None and not isinstance(y, int)), None)
    _check("kq_qgemv_multi", lib().kq_qgemv_multi(count, Ta, Wa, Na, int(K), _ptr(x), int(M), Ya,
                                                  _stream(stream, like)))


def kq_qgemv_mc(qtype, W, N, K, x, M, y, stream=None):
    _check("kq_qgemv_mc", lib().kq_qgemv_mc(int(qtype), _ptr(W), int(N), int(K), _ptr(x), int(M), _ptr(y),
                                            _stream(stream, y)))


def kq_qgemv_mc_multi(types, Ws, Ns, K, x, M, ys, stream=None):
    """As kq_qgemv_multi, on the matrix-core kernels."""
    count = len(Ws)
    if isinstance(types, int):
        types = [types] * count
    if len(types) != count or len(Ns) != count or len(ys) != count:
        raise ValueError("kq_qgemv_mc_multi: types, Ws, Ns and ys must have the same length")
    n = max(count, 1)
    Ta = (ctypes.c_int * n)(*[int(t) for t in types])
    Wa = (ctypes.c_void_p * n)(*[_addr(w) for w in Ws])
    Na = (ctypes.c_int64 * n)(*[int(v) for v in Ns])
    Ya = (ctypes.c_void_p * n)(*[_addr(y) for y in ys])
    like = next((y for y in ys if y is not None and not isinstance(y, int)), None)
    _check("kq_qgemv_mc_multi", lib().kq_qgemv_mc_multi(count, Ta, Wa, Na, int(K), _ptr(x), int(M), Ya,
                                                        _stream(stream, like)))


def kq_qmoe_workspace_bytes(T, k, N):
    return int(lib().kq_qmoe_workspace_bytes(int(T), int(k), int(N)))


def kq_qmoe_gemv(qtype, W_exps, E, N, K, ids, route_w, T, k, x, x_mode, y, workspace=None,
                 err_flag=None, stream=None):
    _check("kq_qmoe_gemv", lib().kq_qmoe_gemv(int(qtype), _ptr(W_exps), int(E), int(N), int(K), _ptr(ids),
                                              _ptr(route_w), int(T), int(k), _ptr(x), int(x_mode), _ptr(y),
                                              _ptr(workspace), _ptr(err_flag), _stream(stream, y)))


def kq_qmoe_gemv_noalloc(qtype, W_exps, E, N, K, ids, route_w, T, k, x, x_mode, y, err_flag=None, stream=None):
    _check("kq_qmoe_gemv_noalloc", lib().kq_qmoe_gemv_noalloc(int(qtype), _ptr(W_exps), int(E), int(N), int(K),
                                                              _ptr(ids), _ptr(route_w), int(T), int(k), _ptr(x),
                                                              int(x_mode), _ptr(y), _ptr(err_flag),
                                                              _stream(stream, y)))


def kq_qmoe_gemv_multi(qtype, W_exps, E, N, K, ids, T, k, x, x_mode, ys, err_flag=None, stream=None):
    """W_exps, ys: equal-length sequences (tensors or int addresses) marshalled
    into the host arrays the C call takes."""
    count = len(W_exps)
    if len(ys) != count:
        raise ValueError("kq_qmoe_gemv_multi: W_exps and ys must have the same length")
    n = max(count, 1)
    Wa = (ctypes.c_void_p * n)(*[_addr(w) for w in W_exps])
    Ya = (ctypes.c_void_p * n)(*[_addr(y) for y in ys])
    like = next((y for y in ys if y is not None and not isinstance(y, int)), None)
    _check("kq_qmoe_gemv_multi", lib().kq_qmoe_gemv_multi(count, int(qtype), Wa, int(E), int(N), int(K), _ptr(ids),
                                                          int(T), int(k), _ptr(x), int(x_mode), Ya,
                                                          _ptr(err_flag), _stream(stream, like)))


# ---- GGUF reader (include/kqgguf.h) ------------------------------------------
# A handle is the opaque kq_gguf* as an int.

def kq_gguf_open(path):
    h = ctypes.c_void_p()
    _check("kq_gguf_open", lib().kq_gguf_open(os.fsencode(path), ctypes.byref(h)))
    return h.value


def kq_gguf_close(h):
    lib().kq_gguf_close(h)


def kq_gguf_version(h):
    return int(lib().kq_gguf_version(h))


def kq_gguf_alignment(h):
    return int(lib().kq_gguf_alignment(h))


def kq_gguf_tensor_count(h):
    return int(lib().kq_gguf_tensor_count(h))


def kq_gguf_find_tensor(h, name):
    r = int(lib().kq_gguf_find_tensor(h, name.encode()))
    if r < 0:
        raise KQError("kq_gguf_find_tensor", r)
    return r


def kq_gguf_tensor_info(h, i):
    t = GGUFTensor()
    _check("kq_gguf_tensor_info", lib().kq_gguf_tensor_info(h, int(i), ctypes.byref(t)))
    return {"name": t.name.decode(), "type": t.type, "n_dims": t.n_dims, "dims": tuple(t.dims[:t.n_dims]),
            "offset": int(t.offset), "nbytes": int(t.nbytes), "data": t.data}


def kq_gguf_upload(h, i, dst, stream=None):
    _check("kq_gguf_upload", lib().kq_gguf_upload(h, int(i), _ptr(dst), _stream(stream, dst)))


def kq_gguf_meta_count(h):
    return int(lib().kq_gguf_meta_count(h))


def kq_gguf_meta_key(h, i):
    k, t = ctypes.c_char_p(), ctypes.c_int()
    _check("kq_gguf_meta_key", lib().kq_gguf_meta_key(h, int(i), ctypes.byref(k), ctypes.byref(t)))
    return k.value.decode(), t.value


def kq_gguf_meta_int(h, key):
    v = ctypes.c_int64()
    _check("kq_gguf_meta_int", lib().kq_gguf_meta_int(h, key.encode(), ctypes.byref(v)))
    return v.value


def kq_gguf_meta_float(h, key):
    v = ctypes.c_double()
    _check("kq_gguf_meta_float", lib().kq_gguf_meta_float(h, key.encode(), ctypes.byref(v)))
    return v.value


def kq_gguf_meta_string(h, key):
    p, n = ctypes.c_void_p(), ctypes.c_uint64()
    _check("kq_gguf_meta_string", lib().kq_gguf_meta_string(h, key.encode(), ctypes.byref(p), ctypes.byref(n)))
    return ctypes.string_at(p.value, n.value) if n.value else b""


def kq_gguf_meta_array(h, key):
    """(element type, count, host address of the packed elements or None)."""
    t, n, p = ctypes.c_int(), ctypes.c_uint64(), ctypes.c_void_p()
    _check("kq_gguf_meta_array", lib().kq_gguf_meta_array(h, key.encode(), ctypes.byref(t), ctypes.byref(n),
                                                          ctypes.byref(p)))
    return t.value, n.value, p.value


def kq_gguf_meta_array_string(h, key, j):
    p, n = ctypes.c_void_p(), ctypes.c_uint64()
    _check("kq_gguf_meta_array_string", lib().kq_gguf_meta_array_string(h, key.encode(), int(j), ctypes.byref(p),
                                                                        ctypes.byref(n)))
    return ctypes.string_at(p.value, n.value) if n.value else b""


# ---- host-streamed GEMV (include/kqstream.h) -----------------------------------
# A streamer is the opaque kq_streamer* as an int.  Weights are HOST tensors or
# addresses (page-locked for overlap); x and y are device tensors.

def kq_streamer_create(slots, slot_bytes, nslots, stream=None):
    h = ctypes.c_void_p()
    _check("kq_streamer_create", lib().kq_streamer_create(_ptr(slots), int(slot_bytes), int(nslots),
                                                          _stream(stream, slots), ctypes.byref(h)))
    return h.value


def kq_streamer_destroy(h):
    lib().kq_streamer_destroy(h)


def kq_streamer_sync(h):
    _check("kq_streamer_sync", lib().kq_streamer_sync(h))


def kq_stream_qgemv_multi(h, types, Ws, Ns, K, x, M, ys):
    count = len(Ws)
    if isinstance(types, int):
        types = [types] * count
    if len(types) != count or len(Ns) != count or len(ys) != count:
        raise ValueError("kq_stream_qgemv_multi: types, Ws, Ns and ys must have the same length")
    n = max(count, 1)
    Ta = (ctypes.c_int * n)(*[int(t) for t in types])
    Wa = (ctypes.c_void_p * n)(*[_addr(w) for w in Ws])
    Na = (ctypes.c_int64 * n)(*[int(v) for v in Ns])
    Ya = (ctypes.c_void_p * n)(*[_addr(y) for y in ys])
    _check("kq_stream_qgemv_multi", lib().kq_stream_qgemv_multi(h, count, Ta, Wa, Na, int(K), _ptr(x), int(M), Ya))


def kq_stream_qgemv(h, qtype, W, N, K, x, M, y):
    _check("kq_stream_qgemv", lib().kq_stream_qgemv(h, int(qtype), _ptr(W), int(N), int(K), _ptr(x), int(M),
                                                    _ptr(y)))
