"""CPU checks of the C ABI: the library loads, exports every function the
header declares, and every synchronous argument error is reported before any
HIP call (no GPU is touched here: each call below fails validation first)."""
import ctypes
import os
import re

import pytest

import dequant_gemv_gguf_amd as kq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

Q4, Q6, Q2, Q8 = kq.KQ_TYPE_Q4_K, kq.KQ_TYPE_Q6_K, kq.KQ_TYPE_Q2_K, kq.KQ_TYPE_Q8_0
FAKE = 0x10000          # a 16-B aligned non-NULL address that is never dereferenced
ODD = 0x10002           # 2-B aligned only


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(kq_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    assert names == sorted(["kq_version", "kq_status_string", "kq_block_info", "kq_row_bytes",
                            "kq_dequant", "kq_qgemv", "kq_qgemv_multi", "kq_qmoe_workspace_bytes",
                            "kq_qgemv_mc", "kq_qgemv_mc_multi",
                            "kq_qmoe_gemv", "kq_qmoe_gemv_multi", "kq_qmoe_gemv_noalloc",
                            "kq_gguf_open", "kq_gguf_close", "kq_gguf_version", "kq_gguf_alignment",
                            "kq_gguf_tensor_count", "kq_gguf_find_tensor", "kq_gguf_tensor_info",
                            "kq_gguf_upload", "kq_gguf_meta_count", "kq_gguf_meta_key", "kq_gguf_meta_int",
                            "kq_gguf_meta_float", "kq_gguf_meta_string", "kq_gguf_meta_array",
                            "kq_gguf_meta_array_string",
                            "kq_streamer_create", "kq_streamer_destroy", "kq_streamer_sync",
                            "kq_stream_qgemv_multi", "kq_stream_qgemv"])


def test_probe_library_exports_its_header():
    probe = os.path.join(os.path.dirname(kq.lib_path), "libkqprobe.so")
    L = ctypes.CDLL(probe)
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "kqprobe.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(kqp_[a-z_0-9]+)\s*\(", text)))
    assert "kqp_stamped_qgemv1" in names and "kqp_read_stream" in names
    for name in names:
        assert hasattr(L, name), name


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(kq.lib_path)
    for name in declared_functions():
        assert hasattr(L, name), name
        assert hasattr(kq, name), name          # binding keeps the C names


def test_version_and_status_strings():
    assert kq.kq_version() >= 10000
    for code in kq.STATUS:
        s = kq.kq_status_string(code)
        assert isinstance(s, str) and s
    assert kq.kq_status_string(12345) == "unknown status"


@pytest.mark.parametrize("qtype,qk,nb", [(Q4, 256, 144), (Q6, 256, 210), (Q2, 256, 84), (Q8, 32, 34),
                                         (2, 32, 18), (13, 256, 176), (11, 256, 110)])
def test_block_info_and_row_bytes(qtype, qk, nb):
    assert kq.kq_block_info(qtype) == (qk, nb)
    assert kq.kq_row_bytes(qtype, 8 * qk) == 8 * nb
    with pytest.raises(kq.KQError):
        kq.kq_row_bytes(qtype, qk + 1)
    with pytest.raises(kq.KQError):
        kq.kq_row_bytes(qtype, 0)


def test_unknown_type():
    with pytest.raises(kq.KQError) as e:
        kq.kq_block_info(3)
    assert e.value.status == -1
    for t in (0, 1, 6, 7, 9, 15, 16, -1):
        with pytest.raises(kq.KQError):
            kq.kq_block_info(t)


def _status(fn, *args):
    try:
        fn(*args)
    except kq.KQError as e:
        return e.status
    return 0


def test_qgemv_argument_errors():
    g = kq.kq_qgemv
    assert _status(g, 99, FAKE, 4, 256, FAKE, 1, FAKE) == -1            # type
    assert _status(g, Q4, FAKE, 4, 100, FAKE, 1, FAKE) == -2            # K not a multiple
    assert _status(g, Q4, FAKE, 4, 0, FAKE, 1, FAKE) == -2
    assert _status(g, Q4, FAKE, -1, 256, FAKE, 1, FAKE) == -2           # N < 0
    assert _status(g, Q4, FAKE, 4, 1 << 21, FAKE, 1, FAKE) == -2        # K too large
    assert _status(g, Q4, FAKE, 4, 256, FAKE, 0, FAKE) == -3            # M
    assert _status(g, Q4, FAKE, 4, 256, FAKE, 9, FAKE) == -3
    assert _status(g, Q4, None, 4, 256, FAKE, 1, FAKE) == -4            # NULL
    assert _status(g, Q4, FAKE, 4, 256, None, 1, FAKE) == -4
    assert _status(g, Q4, FAKE, 4, 256, FAKE, 1, None) == -4
    assert _status(g, Q4, ODD, 4, 256, FAKE, 1, FAKE) == -5             # alignment
    assert _status(g, Q4, FAKE, 4, 256, ODD, 1, FAKE) == -5
    assert _status(g, Q4, FAKE, 4, 256, FAKE, 1, ODD) == -5
    assert _status(g, Q4, None, 0, 256, None, 1, None) == 0             # N == 0: nothing to do


def test_qgemv_multi_argument_errors():
    def g(types=Q4, Ws=(FAKE, FAKE), Ns=(4, 8), K=256, x=FAKE, M=1, ys=(FAKE, FAKE)):
        return _status(kq.kq_qgemv_multi, types, list(Ws), list(Ns), K, x, M, list(ys))
    assert g(types=99) == -1 and g(types=[Q4, 99]) == -1
    assert g(K=100) == -2 and g(Ns=(4, -1)) == -2 and g(K=1 << 21) == -2
    assert g(types=[Q4, Q8], K=32) == -2                               # K must suit every type
    assert g(M=0) == -3 and g(M=9) == -3
    assert g(Ws=(FAKE, None)) == -4 and g(ys=(None, FAKE)) == -4 and g(x=None) == -4
    assert g(Ws=(FAKE, ODD)) == -5 and g(ys=(ODD, FAKE)) == -5 and g(x=ODD) == -5
    assert g(Ws=(), Ns=(), ys=()) == 0                                  # count == 0
    assert g(Ws=(None, None), Ns=(0, 0), ys=(None, None), x=None) == 0   # every matrix empty
    assert g(Ws=(None, FAKE), Ns=(0, 8), ys=(None, ODD)) == -5          # empty ones are skipped
    L = kq.lib()
    assert L.kq_qgemv_multi(-1, None, None, None, 256, None, 1, None, None) == -6
    assert L.kq_qgemv_multi(2, None, None, None, 256, None, 1, None, None) == -4


def test_dequant_argument_errors():
    d = kq.kq_dequant
    assert _status(d, 99, FAKE, 256, FAKE) == -1
    assert _status(d, Q4, FAKE, 100, FAKE) == -2
    assert _status(d, Q8, FAKE, -32, FAKE) == -2
    assert _status(d, Q4, None, 256, FAKE) == -4
    assert _status(d, Q4, FAKE, 256, None) == -4
    assert _status(d, Q4, ODD, 256, FAKE) == -5
    assert _status(d, Q6, FAKE, 256, ODD) == -5
    assert _status(d, Q6, None, 0, None) == 0


def test_qmoe_argument_errors():
    def m(qtype=Q4, W=FAKE, E=8, N=16, K=256, ids=FAKE, rw=None, T=1, k=2, x=FAKE, xm=0, y=FAKE, ws=None, flag=None):
        return _status(kq.kq_qmoe_gemv, qtype, W, E, N, K, ids, rw, T, k, x, xm, y, ws, flag)
    assert m(qtype=5) == -1
    assert m(K=300) == -2
    assert m(N=-3) == -2
    assert m(T=0) == -3 and m(T=9) == -3
    assert m(k=0) == -6 and m(k=17) == -6 and m(E=1, k=2) == -6 and m(E=0) == -6
    assert m(xm=2) == -6
    assert m(W=None) == -4 and m(ids=None) == -4 and m(x=None) == -4 and m(y=None) == -4
    assert m(rw=FAKE, ws=None) == -4                                     # combine needs a workspace
    assert m(W=ODD) == -5 and m(ids=FAKE + 2) == -5 and m(y=ODD) == -5
    assert m(rw=FAKE, ws=ODD) == -5 and m(flag=FAKE + 1) == -5
    assert m(N=0, W=None, ids=None, x=None, y=None) == 0


def test_workspace_bytes():
    assert kq.kq_qmoe_workspace_bytes(8, 8, 2048) == 8 * 8 * 2048 * 4
    assert kq.kq_qmoe_workspace_bytes(0, 8, 2048) == 0
    assert kq.kq_qmoe_workspace_bytes(8, 17, 2048) == 0


def test_streamer_argument_errors():
    L = kq.lib()
    h = ctypes.c_void_p(77)
    assert L.kq_streamer_create(None, 1 << 20, 2, None, ctypes.byref(h)) == -4 and h.value is None
    assert L.kq_streamer_create(ctypes.c_void_p(FAKE), 1 << 20, 2, None, None) == -4
    assert L.kq_streamer_create(ctypes.c_void_p(FAKE + 16), 1 << 20, 2, None, ctypes.byref(h)) == -5
    for nslots, nbytes in [(0, 1 << 20), (65, 1 << 20), (2, 0), (2, 1000)]:
        assert L.kq_streamer_create(ctypes.c_void_p(FAKE), nbytes, nslots, None, ctypes.byref(h)) == -6
    one = (ctypes.c_int * 1)(Q4)
    P1 = (ctypes.c_void_p * 1)(FAKE)
    N1 = (ctypes.c_int64 * 1)(4)
    assert L.kq_stream_qgemv_multi(None, 1, one, P1, N1, 256, ctypes.c_void_p(FAKE), 1, P1) == -4
    assert L.kq_stream_qgemv(None, Q4, ctypes.c_void_p(FAKE), 4, 256, ctypes.c_void_p(FAKE), 1,
                             ctypes.c_void_p(FAKE)) == -4
    assert L.kq_streamer_sync(None) == -4
    L.kq_streamer_destroy(None)


def test_qmoe_multi_argument_errors():
    L = kq.lib()
    P2 = (ctypes.c_void_p * 2)(FAKE, FAKE)
    ids, x = ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE)
    call = lambda count, qtype=Q4, W=P2, E=16, N=64, K=256, T=1, k=2, xm=0, Y=P2, ids=ids, x=x: \
        L.kq_qmoe_gemv_multi(count, qtype, W, E, N, K, ids, T, k, x, xm, Y, None, None)
    assert call(0) == -6 and call(5) == -6                      # count outside 1..4
    assert call(2, qtype=3) == -1                               # type
    assert call(2, K=100) == -2                                 # K not a whole number of blocks
    assert call(2, T=0) == -3 and call(2, T=9) == -3
    assert call(2, k=17) == -6 and call(2, E=1) == -6 and call(2, xm=2) == -6
    assert call(2, W=None) == -4 and call(2, Y=None) == -4 and call(2, ids=None) == -4
    assert call(2, W=(ctypes.c_void_p * 2)(FAKE, None)) == -4
    assert call(2, W=(ctypes.c_void_p * 2)(FAKE, ODD)) == -5
    assert call(2, x=ctypes.c_void_p(ODD)) == -5
    assert call(2, N=0) == 0                                     # nothing to do: no launch


def test_qmoe_noalloc_argument_errors():
    # the same checks as kq_qmoe_gemv without the workspace, and the scratch
    # limit (T * k * N * 4 bytes with routing weights) refused before any HIP
    # call
    def m(qtype=Q4, W=FAKE, E=8, N=16, K=256, ids=FAKE, rw=None, T=1, k=2, x=FAKE, xm=0, y=FAKE, flag=None):
        return _status(kq.kq_qmoe_gemv_noalloc, qtype, W, E, N, K, ids, rw, T, k, x, xm, y, flag)
    assert m(qtype=5) == -1
    assert m(K=300) == -2
    assert m(T=0) == -3 and m(T=9) == -3
    assert m(k=17) == -6 and m(xm=2) == -6
    assert m(W=None) == -4 and m(ids=None) == -4 and m(x=None) == -4 and m(y=None) == -4
    assert m(W=ODD) == -5 and m(rw=FAKE + 2) == -5 and m(flag=FAKE + 1) == -5
    assert m(N=0, W=None, ids=None, x=None, y=None) == 0
    limit = 4 << 20
    N = limit // (8 * 16 * 4)
    assert N * 8 * 16 * 4 == limit
    assert m(E=16, N=N + 1, T=8, k=16, rw=FAKE) == -2           # one row past the scratch
