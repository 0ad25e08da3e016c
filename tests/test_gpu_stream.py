"""GPU: the host-streamed GEMV (include/kqstream.h).  Weights held in host
memory (page-locked, or pageable) are copied through a ring of device slots;
every result must be bit-identical to kq_qgemv_multi on device-resident copies
of the same bytes, whatever the ring depth, and argument errors must be
reported before anything is issued."""
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


def groups(seed):
    # a few "layers": groups of matrices sharing K and x, two formats mixed
    out = []
    for g, (K, mats) in enumerate([(1024, [(kqsynth.Q4_K, 37), (kqsynth.Q6_K, 9), (kqsynth.Q4_K, 5)]),
                                   (2048, [(kqsynth.Q4_K, 70), (kqsynth.Q4_K, 70)]),
                                   (1280, [(kqsynth.Q6_K, 33)]),
                                   (1024, [(kqsynth.Q5_K, 20), (kqsynth.Q8_0, 11)]),
                                   (2048, [(kqsynth.Q2_K, 64), (kqsynth.Q3_K, 0), (kqsynth.Q4_0, 7)])]):
        Ws = [kqsynth.matrix(t, max(n, 1), K, kqsynth.rng_for(seed, g, i, t))[:n] for i, (t, n) in enumerate(mats)]
        out.append((K, mats, Ws))
    return out


def run_streamed(gs, M, nslots, pinned, slot_bytes=1 << 20):
    slots = torch.empty(nslots * slot_bytes, dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream()
    h = kq.kq_streamer_create(slots, slot_bytes, nslots, st)
    hosts, outs = [], []
    try:
        for r in range(2):                       # twice: every slot is reused
            for (K, mats, Ws) in gs:
                Wh = [torch.from_numpy(np.ascontiguousarray(w).reshape(-1)) for w in Ws]
                if pinned:
                    Wh = [w.pin_memory() for w in Wh]
                hosts.append(Wh)                 # kept alive until the copies ran
                x = torch.from_numpy(kqsynth.activations(M, K, kqsynth.rng_for(5, K, M, r))).cuda()
                ys = [torch.full((M, n), float("nan"), device="cuda") for _, n in mats]
                kq.kq_stream_qgemv_multi(h, [t for t, _ in mats], [w.data_ptr() if w.numel() else 0 for w in Wh],
                                         [n for _, n in mats], K, x, M, ys)
                outs.append((K, mats, Ws, x, ys))
        kq.kq_streamer_sync(h)
        torch.cuda.synchronize()
    finally:
        kq.kq_streamer_destroy(h)
    return outs


@pytest.mark.parametrize("nslots,pinned,M", [(2, True, 1), (3, True, 3), (1, True, 1), (2, False, 1)])
def test_streamed_equals_resident(nslots, pinned, M):
    gs = groups(60 + nslots)
    for (K, mats, Ws, x, ys) in run_streamed(gs, M, nslots, pinned):
        Wd = [torch.from_numpy(np.ascontiguousarray(w).reshape(-1)).cuda() if w.size else None for w in Ws]
        ref = [torch.empty((M, n), device="cuda") for _, n in mats]
        kq.kq_qgemv_multi([t for t, _ in mats], Wd, [n for _, n in mats], K, x, M, ref)
        torch.cuda.synchronize()
        for i, (t, n) in enumerate(mats):
            if n == 0:
                continue
            assert torch.equal(ys[i].view(torch.int32), ref[i].view(torch.int32)), (K, i)
            yo, S = oracle.gemv(t, Ws[i], n, K, x.cpu().numpy())
            err = np.abs(ys[i].cpu().numpy().astype(np.float64) - yo)
            assert np.all(err <= 1e-4 * S + 1e-6)


def test_streamer_errors_issue_nothing():
    slot_bytes = 1 << 16
    slots = torch.empty(2 * slot_bytes, dtype=torch.uint8, device="cuda")
    h = kq.kq_streamer_create(slots, slot_bytes, 2)
    try:
        K = 1024
        big = kqsynth.matrix(kqsynth.Q4_K, 200, K, kqsynth.rng_for(7))      # 115200 B > one slot
        x = torch.from_numpy(kqsynth.activations(1, K, kqsynth.rng_for(8))).cuda()
        y = torch.empty((1, 200), device="cuda")
        Wh = torch.from_numpy(big.reshape(-1)).pin_memory()
        for args, status in [((kqsynth.Q4_K, Wh, 200, K, x, 1, y), -2),      # does not fit a slot
                             ((3, Wh, 10, K, x, 1, y), -1),                  # unknown type
                             ((kqsynth.Q4_K, Wh, 10, K, x, 9, y), -3),        # M
                             ((kqsynth.Q4_K, Wh, 10, K + 1, x, 1, y), -2)]:   # K
            with pytest.raises(kq.KQError) as e:
                kq.kq_stream_qgemv(h, *args)
            assert e.value.status == status
        # the ring is untouched: a valid call still lands in order
        small = torch.from_numpy(np.ascontiguousarray(big[:50]).reshape(-1)).pin_memory()
        kq.kq_stream_qgemv(h, kqsynth.Q4_K, small, 50, K, x, 1, y)
        kq.kq_streamer_sync(h)
        torch.cuda.synchronize()
        ref = torch.empty((1, 50), device="cuda")
        kq.kq_qgemv(kqsynth.Q4_K, small.cuda(), 50, K, x, 1, ref)
        torch.cuda.synchronize()
        assert torch.equal(y[:, :50].view(torch.int32), ref.view(torch.int32))
    finally:
        kq.kq_streamer_destroy(h)
