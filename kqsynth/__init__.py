"""Seeded synthetic inputs for the K-quant dequant-GEMV (shared by both sides).

This module only draws random numbers and places them in the packed block
formats; it holds none of the method's arithmetic (no dequantization, no dot,
no combine).  The tests, the benchmark and the smoke check use it to feed the
same bytes to the GPU library and to the CPU oracle.

Recipe (every draw seeded; numpy ``default_rng(SeedSequence([seed, *path]))``):
  * Block scale fields d (and dmin) are fp16(|N(0,1)| * 1e-3), rounded to
    nearest-even by numpy; fp16 subnormals are kept.
  * Every other bit of a K-quant block is uniform random.  Because the 6-bit,
    4-bit and 2-bit fields are bijective bit packings, uniform bytes give
    exactly the uniform field distributions of the workloads: Q4_K scales and
    mins uniform 0..63 and quants 0..15; Q6_K quants 0..63 and int8 scales
    -128..127; Q2_K scale and min nibbles 0..15 and quants 0..3.
  * Q8_0 quants are int8 uniform in -127..127.
  * Q4_0 quants uniform 0..15; Q5_K quants 0..31 with Q4_K's scale fields;
    Q3_K quants -4..3 and stored 6-bit scales 0..63 (uniform bytes give all
    of these exactly).
  * Activations are fp32 N(0,1).
  * MoE routing: per token, k distinct expert ids uniform without replacement;
    routing weights are the softmax (fp64, then fp32) of k N(0,1) logits.
Draw order per tensor: d, dmin, then the remaining block bytes.

Block byte sizes and the offsets of the fp16 fields follow the GGUF K-quant
convention (a reading; the pages name the formats but print no layout).
"""
import numpy as np

Q4_0, Q8_0, Q2_K, Q3_K, Q4_K, Q5_K, Q6_K = 2, 8, 10, 11, 12, 13, 14
TYPE_NAMES = {Q4_0: "Q4_0", Q8_0: "Q8_0", Q2_K: "Q2_K", Q3_K: "Q3_K", Q4_K: "Q4_K", Q5_K: "Q5_K", Q6_K: "Q6_K"}

# weights per block, bytes per block, byte offsets of the fp16 d / dmin fields
BLOCK = {
    Q4_K: (256, 144, 0, 2),
    Q6_K: (256, 210, 208, None),
    Q2_K: (256, 84, 80, 82),
    Q8_0: (32, 34, 0, None),
    Q4_0: (32, 18, 0, None),
    Q5_K: (256, 176, 0, 2),
    Q3_K: (256, 110, 108, None),
}


def row_bytes(qtype, K):
    qk, nb = BLOCK[qtype][:2]
    assert K % qk == 0
    return (K // qk) * nb


def rng_for(seed, *path):
    return np.random.default_rng(np.random.SeedSequence([int(seed)] + [int(p) for p in path]))


def _scale_f16(rng, n):
    return (np.abs(rng.standard_normal(n)) * 1e-3).astype(np.float16)


def blocks(qtype, n_blocks, rng):
    """Return n_blocks packed blocks as a uint8 array [n_blocks, block_bytes]."""
    qk, nb, d_off, dmin_off = BLOCK[qtype]
    d = _scale_f16(rng, n_blocks)
    dmin = _scale_f16(rng, n_blocks) if dmin_off is not None else None
    out = rng.integers(0, 256, size=(n_blocks, nb), dtype=np.uint8)
    if qtype == Q8_0:
        out[:, 2:34] = rng.integers(-127, 128, size=(n_blocks, 32), dtype=np.int8).view(np.uint8)
    out[:, d_off:d_off + 2] = d.view(np.uint8).reshape(n_blocks, 2)
    if dmin is not None:
        out[:, dmin_off:dmin_off + 2] = dmin.view(np.uint8).reshape(n_blocks, 2)
    return out


def matrix(qtype, N, K, rng):
    """N x K weight matrix as uint8 [N, row_bytes]."""
    qk = BLOCK[qtype][0]
    return blocks(qtype, N * (K // qk), rng).reshape(N, -1)


def activations(M, K, rng):
    return rng.standard_normal((M, K)).astype(np.float32)


def routing(T, k, E, rng):
    """Expert ids [T][k] (distinct per token) and softmax weights [T][k]."""
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    logits = rng.standard_normal((T, k))
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    return ids, (z / z.sum(axis=1, keepdims=True)).astype(np.float32)


# ---- device-side generation (large sweeps) --------------------------------
# The same recipe drawn with torch's seeded generator directly in device
# memory, so that tens of GB of distinct layers never pass through the host.
# Parity at these sizes copies sampled rows back and gives them to the oracle.

def device_matrix(qtype, N, K, seed, device):
    import torch
    qk, nb, d_off, dmin_off = BLOCK[qtype]
    nblk = N * (K // qk)
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    out = torch.randint(0, 256, (nblk, nb), dtype=torch.uint8, device=device, generator=g)
    if qtype == Q8_0:
        q = torch.randint(-127, 128, (nblk, 32), dtype=torch.int16, device=device, generator=g)
        out[:, 2:34] = q.to(torch.int8).view(torch.uint8)
    for off in (d_off, dmin_off):
        if off is None:
            continue
        v = (torch.randn(nblk, device=device, generator=g).abs() * 1e-3).to(torch.float16)
        out[:, off:off + 2] = v.view(torch.uint8).view(nblk, 2)
    return out.view(N, -1)


# ---- workload shapes --------------------------------------------------------
# (name, quant type, N = output rows, K = input columns)

def dense_layer(hidden, ffn, kv):
    """Q4_K_M-style decode layer: attention wq/wk/wo and FFN w1/w3 in Q4_K,
    wv and w2 in Q6_K."""
    return [
        ("wq", Q4_K, hidden, hidden),
        ("wk", Q4_K, kv, hidden),
        ("wv", Q6_K, kv, hidden),
        ("wo", Q4_K, hidden, hidden),
        ("w1", Q4_K, ffn, hidden),
        ("w3", Q4_K, ffn, hidden),
        ("w2", Q6_K, hidden, ffn),
    ]


LLAMA3_8B = dict(hidden=4096, ffn=14336, kv=1024, layers=32)
LLAMA3_70B = dict(hidden=8192, ffn=28672, kv=1024, layers=80)
QWEN3_30B_A3B_MOE = dict(hidden=2048, experts=128, ffn=768, top_k=8, layers=48)


def reencode(layer, qtype):
    """The same shapes with every tensor in one quant type (verify sweep)."""
    return [(n, qtype, N, K) for (n, _, N, K) in layer]


def layer_bytes(layer):
    return sum(N * row_bytes(t, K) for (_, t, N, K) in layer)


def moe_layer(hidden, experts, ffn):
    """Per-layer expert tensors [E][N][K]: gate/up in Q4_K, down in Q6_K."""
    return [
        ("gate", Q4_K, experts, ffn, hidden),
        ("up", Q4_K, experts, ffn, hidden),
        ("down", Q6_K, experts, hidden, ffn),
    ]
