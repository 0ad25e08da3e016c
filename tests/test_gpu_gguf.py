"""GPU: tensors read from a GGUF file go straight into the GEMV with no
conversion.  A file written by the independent test writer is opened by the
library's reader, each tensor is uploaded with kq_gguf_upload and multiplied
with kq_qgemv using the type and dims of its table entry; the result must equal
the same call on the bytes uploaded directly, bit for bit, and the oracle within
|dy| <= 1e-4 * sum|w*x| + 1e-6."""
import numpy as np
import pytest

import kqsynth
import oracle
from gguf_writer import STRING, U32, write

torch = pytest.importorskip("torch")
import dequant_gemv_gguf_amd as kq  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


SHAPES = [("blk.0.attn_q.weight", kqsynth.Q4_K, 37, 4096), ("blk.0.attn_v.weight", kqsynth.Q6_K, 9, 768),
          ("blk.0.ffn_up.weight", kqsynth.Q5_K, 20, 2048), ("blk.0.ffn_down.weight", kqsynth.Q3_K, 11, 1280),
          ("blk.0.attn_k.weight", kqsynth.Q8_0, 17, 1184), ("blk.0.attn_output.weight", kqsynth.Q4_0, 5, 96),
          ("blk.0.ffn_gate.weight", kqsynth.Q2_K, 33, 512)]


@pytest.mark.parametrize("M", [1, 3])
def test_gguf_tensors_feed_qgemv(tmp_path, M):
    mats = [(name, qt, N, K, kqsynth.matrix(qt, N, K, kqsynth.rng_for(90 + i, qt, N, K)))
            for i, (name, qt, N, K) in enumerate(SHAPES)]
    path = str(tmp_path / "m.gguf")
    write(path, [("general.architecture", STRING, "llama"), ("general.alignment", U32, 64)],
          [(name, qt, [K, N], W.tobytes()) for (name, qt, N, K, W) in mats], alignment=64)
    h = kq.kq_gguf_open(path)
    try:
        for (name, qt, N, K, W) in mats:
            i = kq.kq_gguf_find_tensor(h, name)
            info = kq.kq_gguf_tensor_info(h, i)
            assert info["type"] == qt and info["dims"] == (K, N)
            dev = torch.empty(info["nbytes"], dtype=torch.uint8, device="cuda")
            kq.kq_gguf_upload(h, i, dev)
            x = kqsynth.activations(M, K, kqsynth.rng_for(91, M, K))
            xd = torch.from_numpy(x).cuda()
            y = torch.empty((M, N), device="cuda")
            kq.kq_qgemv(info["type"], dev, info["dims"][1], info["dims"][0], xd, M, y)
            y2 = torch.empty((M, N), device="cuda")
            kq.kq_qgemv(qt, torch.from_numpy(W.reshape(-1)).cuda(), N, K, xd, M, y2)
            torch.cuda.synchronize()
            assert np.array_equal(dev.cpu().numpy(), W.reshape(-1)), name
            assert torch.equal(y.view(torch.int32), y2.view(torch.int32)), name
            yo, S = oracle.gemv(qt, W, N, K, x)
            err = np.abs(y.cpu().numpy().astype(np.float64) - yo)
            assert np.all(err <= 1e-4 * S + 1e-6), name
    finally:
        kq.kq_gguf_close(h)
