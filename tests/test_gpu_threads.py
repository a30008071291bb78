"""Concurrent callers: host threads inside the library at once, each on its own stream.

ctypes releases the GIL around every library call, so the threads below really run the
library's host code at the same time: argument checks, the chunk plan, the per-device
score-slot cache, the map of helper streams behind the chunk overlap, the thread-local
error text, and the launches.  Each worker thread runs whole passes (pool the keys,
score + select with a small workspace, so that the chunk loop runs many chunks, expand)
on its own inputs and stream, some with the chunk overlap and some without.  Two more
threads meanwhile provoke different argument errors and check that the error text they
read names their own call.  Every worker's results must equal, bit for bit, the same pass
run alone beforehand.  (The allocation-free entry point is left out: by its contract,
overlapping calls on one GPU share its scratch.)
"""
import threading

import numpy as np
import pytest
import torch

from gpu_helpers import device_tensors
from pool_score_top_amd import kpool as K
from pool_score_top_amd import synth

pytestmark = pytest.mark.gpu

# (cu_seqlens, kpool, budget, chunk overlap, workspace rows, input seed)
CASES = [
    ([0, 1100, 1100, 3000], 4, 64, True, 97, 401),
    ([0, 2500], 3, 513, False, 41, 402),
    ([0, 700, 2600, 4000], 1, 1025, True, 150, 403),
    ([0, 900, 1800], 5, 7, False, 33, 404),
]
PASSES = 3


def _setup(case):
    cu, kpool, budget, overlap, ws_rows, seed = case
    cu = np.asarray(cu, dtype=np.int32)
    T = int(cu[-1])
    wl = synth.workload("sq4096", T=T, kpool=kpool, budget=budget)
    r = synth.host_inputs(wl, seed)
    q, k, w = device_tensors(r)
    cu_pools, max_pools, P = K.count_pools(cu, kpool)
    nb = K.workspace_bytes(0, ws_rows, max_pools, 2 if overlap else 1)
    return {
        "cu": cu, "kpool": kpool, "budget": budget, "overlap": overlap, "T": T,
        "q": q, "k": k, "w": w,
        "cu_dev": torch.from_numpy(cu).cuda(), "cu_pools_dev": torch.from_numpy(cu_pools).cuda(),
        "kp": torch.empty((P, wl.D), dtype=torch.int16, device="cuda"),
        "ids": torch.empty((T, budget), dtype=torch.int32, device="cuda"),
        "tok": torch.empty((T, budget * kpool), dtype=torch.int32, device="cuda"),
        "ws": torch.empty(nb, dtype=torch.uint8, device="cuda"),
        "stream": torch.cuda.Stream(),
    }


def _pass(d):
    s = d["stream"]
    with torch.cuda.stream(s):
        d["kp"].fill_(0x7F7F)
        d["ids"].fill_(-7)
        d["tok"].fill_(-9)
    K.pool_keys(d["k"], d["cu"], d["cu_dev"], d["cu_pools_dev"], d["kpool"], out=d["kp"], stream=s)
    K.score_topk(d["q"], d["kp"], d["w"], d["cu"], d["cu_dev"], d["kpool"], d["budget"], 0, d["T"],
                 workspace=d["ws"], pool_ids=d["ids"], overlap=d["overlap"], stream=s)
    K.expand(d["ids"], d["cu"], d["cu_dev"], d["kpool"], d["budget"], 0, d["T"], out=d["tok"], stream=s)


def _snapshot(d):
    d["stream"].synchronize()
    return {n: d[n].cpu().numpy().copy() for n in ("kp", "ids", "tok")}


def test_concurrent_threads_match_serial_passes():
    runs = [_setup(c) for c in CASES]
    for d in runs:  # (also warms the library's per-device state)
        assert K.chunk_rows(K.count_pools(d["cu"], d["kpool"])[1], d["ws"].numel(), d["overlap"])[0] < d["T"]
    refs = []
    for d in runs:
        _pass(d)
        refs.append(_snapshot(d))
    torch.cuda.synchronize()

    start = threading.Barrier(len(runs) + 2)
    failures = []

    def worker(i):
        try:
            start.wait()
            for p in range(PASSES):
                _pass(runs[i])
                got = _snapshot(runs[i])
                for n, ref in refs[i].items():
                    if not np.array_equal(got[n].view(np.uint8), ref.view(np.uint8)):
                        failures.append(f"worker {i} pass {p}: {n} differs from the serial pass")
        except Exception as e:  # reported by the main thread
            failures.append(f"worker {i}: {type(e).__name__}: {e}")

    def provoker(bad_budget):
        # argument errors from this thread; the message read back must be this call's
        d = runs[0]
        try:
            start.wait()
            for _ in range(200):
                try:
                    if bad_budget:
                        K.score_topk(d["q"], d["kp"], d["w"], d["cu"], d["cu_dev"], d["kpool"], 0, 0, d["T"],
                                     workspace=d["ws"], pool_ids=d["ids"])
                    else:
                        K.expand(d["ids"], d["cu"], d["cu_dev"], 0, d["budget"], 0, d["T"], out=d["tok"])
                    failures.append("provoker: an invalid call succeeded")
                    return
                except RuntimeError as e:
                    want = "budget must be in" if bad_budget else "kpool must be >= 1"
                    if want not in str(e):
                        failures.append(f"provoker: error text of another call: {e}")
                        return
        except Exception as e:
            failures.append(f"provoker: {type(e).__name__}: {e}")

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(runs))]
    threads += [threading.Thread(target=provoker, args=(b,)) for b in (True, False)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    torch.cuda.synchronize()
    assert not failures, "\n".join(failures[:10])
    print(f"[threads] {len(runs)} workers x {PASSES} passes equal their serial passes bit for bit; "
          f"2 threads' argument errors kept their own text", flush=True)
