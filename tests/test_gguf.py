"""CPU tests of the GGUF reader (include/kqgguf.h): files written by an
independent writer (tests/gguf_writer.py) are parsed by the library; the tensor
table, the data bytes and the metadata must come back exactly, and malformed
files must be rejected (KQ_ERR_FORMAT) without reading past their end.  No GPU
is touched: kq_gguf_upload is exercised by the GPU tests."""
import ctypes
import os
import random
import struct

import numpy as np
import pytest

import dequant_gemv_gguf_amd as kq
import kqsynth
from gguf_writer import (ARRAY, BOOL, F32, F64, I8, I16, I32, I64, STRING, U8, U16, U32, U64, build,
                         write)

ERR_ARG, ERR_NULL, ERR_IO, ERR_FORMAT = -6, -4, -9, -10


def sample_tensors(seed=0):
    rng = kqsynth.rng_for(seed, 77)
    out = []
    for name, qt, N, K in [("blk.0.ffn_up.weight", kqsynth.Q4_K, 3, 512),
                           ("blk.0.ffn_down.weight", kqsynth.Q6_K, 5, 256),
                           ("blk.0.attn_v.weight", kqsynth.Q8_0, 2, 96),
                           ("blk.0.attn_k.weight", kqsynth.Q5_K, 2, 256),
                           ("blk.0.attn_q.weight", kqsynth.Q3_K, 1, 256),
                           ("blk.0.attn_o.weight", kqsynth.Q4_0, 4, 64),
                           ("blk.0.ffn_gate.weight", kqsynth.Q2_K, 2, 256)]:
        out.append((name, qt, [K, N], kqsynth.matrix(qt, N, K, rng).tobytes()))
    norm = rng.standard_normal(7).astype(np.float32)
    out.append(("output_norm.weight", 0, [7], norm.tobytes()))
    return out


META = [
    ("general.architecture", STRING, "llama"),
    ("general.alignment", U32, 64),
    ("llama.block_count", U32, 1),
    ("test.u8", U8, 250), ("test.i8", I8, -7), ("test.u16", U16, 65000), ("test.i16", I16, -30000),
    ("test.i32", I32, -2000000000), ("test.u64", U64, 2 ** 40 + 3), ("test.i64", I64, -(2 ** 50)),
    ("test.f32", F32, 0.15625), ("test.f64", F64, -1.0e-300), ("test.bool", BOOL, 1),
    ("test.u32s", ARRAY, (U32, [1, 2, 3, 4000000000])),
    ("tokenizer.ggml.tokens", ARRAY, (STRING, ["<s>", "", "héllo", "x" * 300])),
    ("test.nested", ARRAY, (ARRAY, [(I16, [1, -2]), (STRING, ["a", "bc"])])),
    ("test.empty", STRING, ""),
]


@pytest.fixture()
def gguf_file(tmp_path):
    tensors = sample_tensors()
    path = str(tmp_path / "model.gguf")
    offs = write(path, META, tensors, alignment=64)
    return path, tensors, offs


def status_of(fn, *args):
    try:
        fn(*args)
    except kq.KQError as e:
        return e.status
    return 0


def open_status(path):
    h = ctypes.c_void_p(1234)
    r = kq.lib().kq_gguf_open(os.fsencode(path), ctypes.byref(h))
    if r == 0:
        kq.kq_gguf_close(h.value)
    else:
        assert h.value is None          # *out is NULL on failure
    return r


def test_tensor_table_and_data_round_trip(gguf_file):
    path, tensors, offs = gguf_file
    h = kq.kq_gguf_open(path)
    try:
        assert kq.kq_gguf_version(h) == 3
        assert kq.kq_gguf_alignment(h) == 64
        assert kq.kq_gguf_tensor_count(h) == len(tensors)
        for i, ((name, t, dims, data), off) in enumerate(zip(tensors, offs)):
            info = kq.kq_gguf_tensor_info(h, i)
            assert info["name"] == name and info["type"] == t
            assert info["n_dims"] == len(dims) and list(info["dims"]) == dims
            assert info["offset"] == off and off % 64 == 0
            assert info["nbytes"] == len(data)
            assert ctypes.string_at(info["data"], info["nbytes"]) == data
            assert kq.kq_gguf_find_tensor(h, name) == i
            if t != 0:
                # a quantized tensor is the block matrix the GEMV reads: K = dims[0], N = dims[1]
                assert info["nbytes"] == dims[1] * kq.kq_row_bytes(t, dims[0])
        assert status_of(kq.kq_gguf_find_tensor, h, "missing.weight") == ERR_ARG
        assert status_of(kq.kq_gguf_tensor_info, h, len(tensors)) == ERR_ARG
        assert status_of(kq.kq_gguf_tensor_info, h, -1) == ERR_ARG
    finally:
        kq.kq_gguf_close(h)


def test_metadata_values(gguf_file):
    path, _, _ = gguf_file
    h = kq.kq_gguf_open(path)
    try:
        assert kq.kq_gguf_meta_count(h) == len(META)
        for i, (key, vt, _) in enumerate(META):
            assert kq.kq_gguf_meta_key(h, i) == (key, vt)
        assert kq.kq_gguf_meta_string(h, "general.architecture") == b"llama"
        assert kq.kq_gguf_meta_string(h, "test.empty") == b""
        ints = {"llama.block_count": 1, "test.u8": 250, "test.i8": -7, "test.u16": 65000, "test.i16": -30000,
                "test.i32": -2000000000, "test.u64": 2 ** 40 + 3, "test.i64": -(2 ** 50), "test.bool": 1,
                "general.alignment": 64}
        for k, v in ints.items():
            assert kq.kq_gguf_meta_int(h, k) == v, k
        assert kq.kq_gguf_meta_float(h, "test.f32") == 0.15625
        assert kq.kq_gguf_meta_float(h, "test.f64") == -1.0e-300
        et, n, p = kq.kq_gguf_meta_array(h, "test.u32s")
        assert (et, n) == (U32, 4)
        assert list(struct.unpack("<4I", ctypes.string_at(p, 16))) == [1, 2, 3, 4000000000]
        et, n, p = kq.kq_gguf_meta_array(h, "tokenizer.ggml.tokens")
        assert (et, n, p) == (STRING, 4, None)
        toks = [kq.kq_gguf_meta_array_string(h, "tokenizer.ggml.tokens", j) for j in range(4)]
        assert toks == [b"<s>", b"", "héllo".encode(), b"x" * 300]
        assert kq.kq_gguf_meta_array(h, "test.nested")[:2] == (ARRAY, 2)
        # wrong-type and missing keys
        assert status_of(kq.kq_gguf_meta_int, h, "general.architecture") == ERR_ARG
        assert status_of(kq.kq_gguf_meta_float, h, "test.u8") == ERR_ARG
        assert status_of(kq.kq_gguf_meta_string, h, "test.u32s") == ERR_ARG
        assert status_of(kq.kq_gguf_meta_int, h, "no.such.key") == ERR_ARG
        assert status_of(kq.kq_gguf_meta_array_string, h, "tokenizer.ggml.tokens", 4) == ERR_ARG
        assert status_of(kq.kq_gguf_meta_array_string, h, "test.u32s", 0) == ERR_ARG
    finally:
        kq.kq_gguf_close(h)


def test_default_alignment_and_version_2(tmp_path):
    tensors = sample_tensors(1)[:3]
    path = str(tmp_path / "v2.gguf")
    offs = write(path, [("general.architecture", STRING, "llama")], tensors, alignment=32, version=2)
    h = kq.kq_gguf_open(path)
    try:
        assert kq.kq_gguf_version(h) == 2 and kq.kq_gguf_alignment(h) == 32
        for i, off in enumerate(offs):
            assert kq.kq_gguf_tensor_info(h, i)["offset"] == off
    finally:
        kq.kq_gguf_close(h)


def test_no_tensors_and_unknown_tensor_type(tmp_path):
    path = str(tmp_path / "empty.gguf")
    write(path, [], [])
    h = kq.kq_gguf_open(path)
    assert kq.kq_gguf_tensor_count(h) == 0 and kq.kq_gguf_meta_count(h) == 0
    kq.kq_gguf_close(h)
    # a type whose size the reader does not know: listed with nbytes 0, not uploadable
    path = str(tmp_path / "unknown.gguf")
    write(path, [], [("w", 99, [64, 2], bytes(40))])
    h = kq.kq_gguf_open(path)
    try:
        info = kq.kq_gguf_tensor_info(h, 0)
        assert info["type"] == 99 and info["nbytes"] == 0
        assert kq.lib().kq_gguf_upload(h, 0, ctypes.c_void_p(0x10000), None) == ERR_ARG
    finally:
        kq.kq_gguf_close(h)


def test_null_and_io_errors(tmp_path):
    L = kq.lib()
    h = ctypes.c_void_p()
    assert L.kq_gguf_open(None, ctypes.byref(h)) == ERR_NULL
    assert L.kq_gguf_open(b"x", None) == ERR_NULL
    assert open_status(str(tmp_path / "does_not_exist.gguf")) == ERR_IO
    assert open_status(str(tmp_path)) == ERR_IO                     # a directory
    assert L.kq_gguf_tensor_count(None) == ERR_NULL
    assert L.kq_gguf_find_tensor(None, b"x") == ERR_NULL
    L.kq_gguf_close(None)


def _raw(meta, tensors, **kw):
    return build(meta, tensors, **kw)[0]


def _check_format_error(tmp_path, data, name):
    p = tmp_path / name
    p.write_bytes(data)
    assert open_status(str(p)) == ERR_FORMAT, name


def test_malformed_headers(tmp_path):
    good = sample_tensors(2)[:2]
    _check_format_error(tmp_path, _raw([], good, magic=b"GGUX"), "magic")
    _check_format_error(tmp_path, _raw([], good, version=1), "v1")
    _check_format_error(tmp_path, _raw([], good, version=4), "v4")
    _check_format_error(tmp_path, b"", "empty")
    _check_format_error(tmp_path, b"GGUF\x03\x00\x00\x00", "short")
    # alignment: not a power of two, zero, wrong value type
    _check_format_error(tmp_path, _raw([("general.alignment", U32, 48)], good, alignment=48), "align48")
    _check_format_error(tmp_path, _raw([("general.alignment", U32, 0)], []), "align0")
    _check_format_error(tmp_path, _raw([("general.alignment", U64, 32)], good), "align_u64")
    # unknown metadata value type
    bad = bytearray(_raw([("k", U32, 5)], []))
    at = bad.index(b"k") + 1
    bad[at:at + 4] = struct.pack("<I", 13)
    _check_format_error(tmp_path, bytes(bad), "value_type")
    # counts far beyond the file
    bad = bytearray(_raw([], good))
    bad[8:16] = struct.pack("<Q", 2 ** 62)
    _check_format_error(tmp_path, bytes(bad), "tensor_count")
    bad = bytearray(_raw([("k", STRING, "v")], []))
    at = bad.index(b"k") + 5
    bad[at:at + 8] = struct.pack("<Q", 2 ** 63)
    _check_format_error(tmp_path, bytes(bad), "string_len")


def test_malformed_tensor_entries(tmp_path):
    K, N = 256, 2
    data = kqsynth.matrix(kqsynth.Q4_K, N, K, kqsynth.rng_for(3)).tobytes()
    # a row that is not a whole number of blocks
    _check_format_error(tmp_path, _raw([], [("w", kqsynth.Q4_K, [K + 32, N], data)]), "ragged")
    # 0 and 5 dimensions
    _check_format_error(tmp_path, _raw([], [("w", kqsynth.Q4_K, [], data)]), "dims0")
    _check_format_error(tmp_path, _raw([], [("w", kqsynth.Q4_K, [K, N, 1, 1, 1], data)]), "dims5")
    # a name or key holding a NUL byte cannot be looked up as a C string
    _check_format_error(tmp_path, _raw([], [("w\x00x", kqsynth.Q4_K, [K, N], data)]), "nul_name")
    _check_format_error(tmp_path, _raw([("a\x00b", U32, 1)], []), "nul_key")
    # data past the end of the file: claim more rows than were written
    _check_format_error(tmp_path, _raw([], [("w", kqsynth.Q4_K, [K, N + 1], data)]), "past_end")
    # a misaligned offset
    raw = bytearray(_raw([], [("a", 0, [4], bytes(16)), ("b", 0, [4], bytes(16))]))
    at = raw.index(b"b") + 1 + 4 + 8 + 4
    off = struct.unpack("<Q", raw[at:at + 8])[0]
    raw[at:at + 8] = struct.pack("<Q", off + 4)
    _check_format_error(tmp_path, bytes(raw), "misaligned")


def test_every_truncation_is_rejected(tmp_path):
    tensors = [("w", kqsynth.Q8_0, [64, 2], kqsynth.matrix(kqsynth.Q8_0, 2, 64, kqsynth.rng_for(4)).tobytes())]
    meta = [("general.architecture", STRING, "llama"), ("a", ARRAY, (STRING, ["x", "yz"]))]
    full = _raw(meta, tensors)
    p = tmp_path / "t.gguf"
    p.write_bytes(full)
    assert open_status(str(p)) == 0
    for n in range(len(full)):
        p.write_bytes(full[:n])
        assert open_status(str(p)) == ERR_FORMAT, n


def test_random_corruption_never_crashes(tmp_path):
    full = _raw(META[:6] + META[13:], sample_tensors(5)[:3], alignment=64)
    p = tmp_path / "c.gguf"
    rnd = random.Random(1234)
    outcomes = set()
    for _ in range(400):
        b = bytearray(full)
        for _ in range(rnd.randint(1, 4)):
            i = rnd.randrange(0, min(len(b), 900))
            b[i] = rnd.randrange(256)
        p.write_bytes(bytes(b))
        r = open_status(str(p))
        assert r in (0, ERR_FORMAT)
        outcomes.add(r)
    assert ERR_FORMAT in outcomes


def _build_sanitized_driver(tmp_path):
    import shutil
    import subprocess
    gxx = shutil.which("g++")
    if not gxx:
        pytest.skip("no g++")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    exe = str(tmp_path / "gguf_fuzz")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(root, "include"),
           os.path.join(root, "tests", "gguf_fuzz_main.cpp"),
           os.path.join(root, "dequant_gemv_gguf_amd", "csrc", "kq_gguf.cpp"), "-o", exe]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode:
        pytest.skip("sanitized build unavailable: " + r.stdout[-300:])
    return exe


def test_reader_is_memory_safe_under_sanitizers(tmp_path):
    # the reader compiled with ASan + UBSan opens valid, truncated, corrupted
    # and crafted files; each must be read cleanly or rejected
    import subprocess
    exe = _build_sanitized_driver(tmp_path)
    full = _raw(META, sample_tensors(9), alignment=64)
    files = []

    def add(name, data):
        p = tmp_path / name
        p.write_bytes(data)
        files.append(str(p))

    add("valid.gguf", full)
    for n in range(0, len(full), 97):
        add("trunc%d.gguf" % n, full[:n])
    rnd = random.Random(99)
    for i in range(300):
        b = bytearray(full)
        for _ in range(rnd.randint(1, 8)):
            at = rnd.randrange(0, len(b)) if rnd.random() < 0.3 else rnd.randrange(0, min(len(b), 1200))
            b[at] = rnd.randrange(256)
        add("mut%d.gguf" % i, bytes(b))
    # crafted: huge lengths and counts in every length field of a small file
    small = _raw([("k", STRING, "v"), ("a", ARRAY, (STRING, ["x"]))], [("w", 0, [4], bytes(16))])
    for off in range(8, len(small) - 8):
        for v in (2 ** 63, 2 ** 40, len(small)):
            b = bytearray(small)
            b[off:off + 8] = struct.pack("<Q", v)
            add("craft%d_%d.gguf" % (off, v.bit_length()), bytes(b))
    for i in range(0, len(files), 200):
        r = subprocess.run([exe] + files[i:i + 200], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                           timeout=120)
        assert r.returncode == 0, r.stdout[-2000:]
        assert "opened" in r.stdout
