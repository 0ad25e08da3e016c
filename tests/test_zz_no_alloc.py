"""kq_qmoe_gemv_noalloc against kq_qmoe_gemv (the same call with a caller
workspace), through the C ABI: routing-weighted sums whose activation rows are
too large for the token-major kernel (16 rows of K = 4096 per token), so the
slot-major kernel writes its per-slot results to the library's static scratch
and the sum reads them back.  Two calls in a row, the second smaller, each
bit-identical to the workspace call and within the oracle's tolerance; a call
without routing weights (no scratch) too."""
import numpy as np
import pytest

import kqsynth
import oracle

torch = pytest.importorskip("torch")
import dequant_gemv_gguf_amd as kq  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def test_noalloc_matches_the_workspace_call_on_two_calls_in_a_row():
    qtype, E, K, k = kqsynth.Q4_K, 20, 4096, 16
    for step, (T, N) in enumerate([(2, 256), (1, 64)]):
        print("noalloc call", step, "T", T, "N", N, flush=True)
        rng = kqsynth.rng_for(70, step)
        W = kqsynth.blocks(qtype, E * N * (K // 256), rng)
        ids, p = kqsynth.routing(T, k, E, kqsynth.rng_for(71, step))
        x = kqsynth.activations(T * k, K, kqsynth.rng_for(72, step))
        Wd, idd, pd, xd = dev(W.reshape(-1)), dev(ids), dev(p), dev(x)
        ws = torch.empty(kq.kq_qmoe_workspace_bytes(T, k, N) // 4, device="cuda")
        y_ref = torch.full((T, N), float("nan"), device="cuda")
        y = torch.full((T, N), float("nan"), device="cuda")
        kq.kq_qmoe_gemv(qtype, Wd, E, N, K, idd, pd, T, k, xd, 1, y_ref, ws)
        kq.kq_qmoe_gemv_noalloc(qtype, Wd, E, N, K, idd, pd, T, k, xd, 1, y)
        torch.cuda.synchronize()
        a, b = y.cpu().numpy(), y_ref.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), step
        yo, S, _ = oracle.moe(qtype, W, E, N, K, ids, p, x, 1)
        assert np.all(np.abs(a.astype(np.float64) - yo) <= 1e-4 * S + 1e-6), step
    # without routing weights no scratch is used: per-slot outputs
    ys = torch.empty((T, k, N), device="cuda")
    ys_ref = torch.empty((T, k, N), device="cuda")
    kq.kq_qmoe_gemv(qtype, Wd, E, N, K, idd, None, T, k, xd, 1, ys_ref)
    kq.kq_qmoe_gemv_noalloc(qtype, Wd, E, N, K, idd, None, T, k, xd, 1, ys)
    torch.cuda.synchronize()
    assert np.array_equal(ys.cpu().numpy().view(np.uint32), ys_ref.cpu().numpy().view(np.uint32))
