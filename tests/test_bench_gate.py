"""The benchmark's parity gate, on the CPU: sampled outputs that the oracle
itself produced pass it, and one output moved past the tolerance, one flipped
bit of a dequantized weight or one wrong slot of a routed-expert output make
it fail.  (The gate runs before anything is timed; a failing gate ends the
run with no value.)  Tensors stay on the CPU: the gate only indexes them and
copies them to numpy."""
import numpy as np
import pytest

import bench
import kqsynth
import oracle

torch = pytest.importorskip("torch")


def gemv_check(qtype, N, K, M, seed):
    W = kqsynth.matrix(qtype, N, K, kqsynth.rng_for(seed, 1))
    x = kqsynth.activations(M, K, kqsynth.rng_for(seed, 2))
    y, _ = oracle.gemv(qtype, W, N, K, x)
    return {"kind": "gemv", "qtype": qtype, "N": N, "K": K, "W": torch.from_numpy(W),
            "x": torch.from_numpy(x), "y": torch.from_numpy(y.astype(np.float32))}


@pytest.mark.parametrize("qtype", [kqsynth.Q4_K, kqsynth.Q6_K, kqsynth.Q2_K, kqsynth.Q8_0])
def test_gate_passes_oracle_outputs_and_catches_a_moved_one(qtype):
    c = gemv_check(qtype, 300, 1024, 2, 5)
    worst, n = bench.parity_gate(torch, [c])
    assert worst <= 1.0 and n > 0
    rows = bench.sample_rows(c["N"], c["N"] + c["K"])
    r = int(rows[len(rows) // 2])
    _, S = oracle.gemv(qtype, c["W"].numpy()[r:r + 1], 1, c["K"], c["x"].numpy())
    c["y"][1, r] += float(3 * (bench.TOL_REL * S[1, 0] + bench.TOL_ABS))
    worst, _ = bench.parity_gate(torch, [c])
    assert worst > 1.0


def test_gate_dequant_needs_every_bit():
    qtype, n = kqsynth.Q4_K, 256 * 64
    Wb = kqsynth.blocks(qtype, n // 256, kqsynth.rng_for(6, 1))
    out = oracle.dequant(qtype, Wb, n)
    c = {"kind": "dequant", "qtype": qtype, "W": torch.from_numpy(Wb.reshape(-1)), "out": torch.from_numpy(out),
         "n": n, "block": kqsynth.BLOCK[qtype][:2]}
    worst, _ = bench.parity_gate(torch, [c])
    assert worst == 0.0
    picked = bench.sample_rows(n // 256, n // 256, 30)
    i = int(picked[0]) * 256 + 17
    bad = out.copy()
    bad.view(np.uint32)[i] ^= 1                       # one ulp of one weight
    c["out"] = torch.from_numpy(bad)
    worst, _ = bench.parity_gate(torch, [c])
    assert worst == float("inf")


def test_gate_routed_experts():
    qtype, E, N, K, T, k = kqsynth.Q4_K, 10, 64, 512, 3, 4
    W = kqsynth.blocks(qtype, E * N * (K // 256), kqsynth.rng_for(7, 1)).reshape(E * N, -1)
    ids, p = kqsynth.routing(T, k, E, kqsynth.rng_for(7, 2))
    x = kqsynth.activations(T, K, kqsynth.rng_for(7, 3))
    y, _, _ = oracle.moe(qtype, W, E, N, K, ids, None, x, 0)
    c = {"kind": "moe", "qtype": qtype, "E": E, "N": N, "K": K, "W": torch.from_numpy(W),
         "ids": torch.from_numpy(ids), "p": None, "x": torch.from_numpy(x), "x_mode": 0,
         "y": torch.from_numpy(y.astype(np.float32))}
    worst, _ = bench.parity_gate(torch, [c])
    assert worst <= 1.0
    rows = bench.sample_rows(N, N + K, 10)
    c["y"][2, 1, int(rows[0])] = -c["y"][2, 1, int(rows[0])] + 1.0   # one slot's row wrong
    worst, _ = bench.parity_gate(torch, [c])
    assert worst > 1.0
