"""The selection path captured in a HIP graph (through torch.cuda.CUDAGraph) and replayed.

Serving loops replay a captured step instead of launching its kernels one by one.
The library enqueues kernels only (no allocation, copy, memset or synchronization on
the launch path), so the whole pass (pool, score + top-k, expand) can be captured:
with a caller workspace through kpool_score_topk, with flags 0 (every launch on the
caller's stream) and with the chunk overlap (chunks alternate with a helper stream,
whose fork and join events become dependencies of the graph), and through the
allocation-free kpool_score_topk_noalloc.  Each
graph is replayed several times, with the outputs refilled by eager torch fills and
other eager library work between the replays; every replay must equal the eager run of
the same pass bit for bit (pooled keys, pool ids, scores, token ids).
"""
import numpy as np
import pytest
import torch

from gpu_helpers import device_tensors
from pool_score_top_amd import kpool as K
from pool_score_top_amd import synth

pytestmark = pytest.mark.gpu


def _setup(T, cu, kpool, budget, seed, overlap=False):
    wl = synth.workload("sq4096", T=T, kpool=kpool, budget=budget)
    r = synth.host_inputs(wl, seed)
    q, k, w = device_tensors(r)
    cu = np.asarray(cu, dtype=np.int32)
    cu_pools, max_pools, P = K.count_pools(cu, kpool)
    dev = {
        "q": q, "k": k, "w": w,
        "cu_dev": torch.from_numpy(cu).cuda(), "cu_pools_dev": torch.from_numpy(cu_pools).cuda(),
        "kp": torch.empty((P, wl.D), dtype=torch.int16, device="cuda"),
        "ids": torch.empty((T, budget), dtype=torch.int32, device="cuda"),
        "scores": torch.empty((T, max_pools), dtype=torch.float32, device="cuda"),
        "tok": torch.empty((T, budget * kpool), dtype=torch.int32, device="cuda"),
        # several chunks: the captured pass runs the chunk loop more than once (with the
        # overlap, two buffers of about T/8 rows on two streams)
        "ws": torch.empty(K.workspace_bytes(0, (T + 3) // 4 if overlap else (T + 1) // 2, max_pools,
                                            2 if overlap else 1), dtype=torch.uint8, device="cuda"),
    }
    return cu, dev


def _pass(cu, d, kpool, budget, noalloc, overlap=False):
    T = int(cu[-1])
    K.pool_keys(d["k"], cu, d["cu_dev"], d["cu_pools_dev"], kpool, out=d["kp"])
    if noalloc:
        K.score_topk_noalloc(d["q"], d["kp"], d["w"], cu, d["cu_dev"], kpool, budget, 0, T, d["ids"],
                             scores_out=d["scores"])
    else:
        K.score_topk(d["q"], d["kp"], d["w"], cu, d["cu_dev"], kpool, budget, 0, T,
                     workspace=d["ws"], pool_ids=d["ids"], scores_out=d["scores"], overlap=overlap)
    K.expand(d["ids"], cu, d["cu_dev"], kpool, budget, 0, T, out=d["tok"])


def _snapshot(d):
    return {n: d[n].cpu().numpy().copy() for n in ("kp", "ids", "scores", "tok")}


def _refill(d):
    d["kp"].fill_(0x7F7F)
    d["ids"].fill_(-7)
    d["scores"].fill_(3.5)
    d["tok"].fill_(-9)


@pytest.mark.parametrize("noalloc,overlap", [(False, False), (False, True), (True, False)])
def test_captured_pass_replays_equal_eager(noalloc, overlap):
    T, kpool, budget = 3000, 4, 64
    cu, d = _setup(T, [0, 1100, 1100, 3000], kpool, budget, 91, overlap)
    if overlap:
        assert K.chunk_rows(d["scores"].shape[1], d["ws"].numel(), True) == (375, 2)
    # eager reference (also warms the library's per-device state before the capture;
    # torch captures on a side stream of its own, whose helper stream the library
    # creates during the capture when the overlap is on)
    _pass(cu, d, kpool, budget, noalloc, overlap)
    torch.cuda.synchronize()
    ref = _snapshot(d)
    assert (ref["ids"] >= -1).all() and (ref["ids"][:, 0] >= 0).all()
    # other eager work between replays: a different batch through the same library
    cu2, d2 = _setup(1500, [0, 700, 1500], 3, 16, 92)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _pass(cu, d, kpool, budget, noalloc, overlap)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _pass(cu, d, kpool, budget, noalloc, overlap)
    torch.cuda.synchronize()
    for rep in range(4):
        _refill(d)
        _pass(cu2, d2, 3, 16, noalloc)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(d)
        for n in ref:
            assert np.array_equal(got[n].view(np.uint8), ref[n].view(np.uint8)), \
                f"replay {rep}: {n} differs from the eager pass (noalloc={noalloc}, overlap={overlap})"
    print(f"[graph] noalloc={noalloc} overlap={overlap}: 4 replays equal the eager pass bit for bit",
          flush=True)
