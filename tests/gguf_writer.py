"""A GGUF file writer for the reader's tests (test infrastructure).

Written from the published GGUF layout (version 3, little-endian): magic,
version, tensor count, metadata count, metadata entries, tensor table, padding
to the alignment, tensor data.  It shares nothing with the library's C++
reader.  Metadata values are given as (value type, value); an array value is
(element type, [elements]).
"""
import struct

U8, I8, U16, I16, U32, I32, F32, BOOL, STRING, ARRAY, U64, I64, F64 = range(13)
_PACK = {U8: "<B", I8: "<b", U16: "<H", I16: "<h", U32: "<I", I32: "<i", F32: "<f", BOOL: "<B",
         U64: "<Q", I64: "<q", F64: "<d"}


def gguf_string(s):
    b = s.encode() if isinstance(s, str) else bytes(s)
    return struct.pack("<Q", len(b)) + b


def value_bytes(vt, v):
    if vt == STRING:
        return gguf_string(v)
    if vt == ARRAY:
        et, items = v
        return struct.pack("<IQ", et, len(items)) + b"".join(value_bytes(et, x) for x in items)
    return struct.pack(_PACK[vt], v)


def build(meta, tensors, alignment=32, version=3, magic=b"GGUF"):
    """meta: [(key, value type, value)]; tensors: [(name, type id, dims, data bytes)].
    Returns (file bytes, [absolute data offset of each tensor]).  Each tensor's
    data starts at the next multiple of `alignment` after the previous one."""
    head = bytearray(magic + struct.pack("<IQQ", version, len(tensors), len(meta)))
    for key, vt, v in meta:
        head += gguf_string(key) + struct.pack("<I", vt) + value_bytes(vt, v)
    rel, at = [], 0
    for (_, _, _, data) in tensors:
        at = (at + alignment - 1) // alignment * alignment
        rel.append(at)
        at += len(data)
    for (name, t, dims, _), r in zip(tensors, rel):
        head += gguf_string(name) + struct.pack("<I", len(dims))
        head += b"".join(struct.pack("<Q", d) for d in dims)
        head += struct.pack("<IQ", t, r)
    start = (len(head) + alignment - 1) // alignment * alignment
    out = bytearray(head) + bytes(start - len(head))
    for (_, _, _, data), r in zip(tensors, rel):
        out += bytes(start + r - len(out)) + bytes(data)
    return bytes(out), [start + r for r in rel]


def write(path, meta, tensors, **kw):
    data, offs = build(meta, tensors, **kw)
    with open(path, "wb") as f:
        f.write(data)
    return offs
