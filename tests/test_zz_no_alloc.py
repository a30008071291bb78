"""kpool_score_topk_noalloc (the entry point for callers that cannot allocate device
memory) against kpool_score_topk, through the C ABI.

Both run the same kernels; the allocation-free call takes its workspace from the
library's 64 MiB static scratch, so its chunks are shorter.  Scores do not depend
on the chunking, so pool ids and fp32 scores must match bit for bit.  Two calls in
a row, the second on a smaller input, show that the shared scratch keeps no state
that matters between calls.  Sizes beyond the scratch are rejected before any GPU
work (checked without a GPU).
"""
import ctypes

import numpy as np
import pytest
import torch

from gpu_helpers import device_tensors
from pool_score_top_amd import kpool as K
from pool_score_top_amd import synth


def _both(r, cu, kpool, budget, q_lo, q_hi):
    q, k, w = device_tensors(r)
    cu = np.asarray(cu, dtype=np.int32)
    cu_dev = torch.from_numpy(cu).cuda()
    cu_pools, max_pools, _ = K.count_pools(cu, kpool)
    kp = K.pool_keys(k, cu, cu_dev, torch.from_numpy(cu_pools).cuda(), kpool)
    rows = q_hi - q_lo
    ref_ids, ref_sc = K.score_topk(q, kp, w, cu, cu_dev, kpool, budget, q_lo, q_hi, want_scores=True)
    ids = torch.full((rows, budget), -7, dtype=torch.int32, device="cuda")
    sc = torch.full((rows, max_pools), 3.0, dtype=torch.float32, device="cuda")
    K.score_topk_noalloc(q, kp, w, cu, cu_dev, kpool, budget, q_lo, q_hi, ids, sc)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), sc.cpu().numpy(), ref_ids.cpu().numpy(), ref_sc.cpu().numpy()


@pytest.mark.gpu
def test_noalloc_matches_score_topk_on_two_calls():
    # 1: one sequence of 40000 tokens at the indexer shape: a score row is 42704 bytes, so
    #    the 64 MiB scratch holds 1571-row chunks (26 chunks), against one chunk for the
    #    allocating call
    wl = synth.workload("sq4096", T=40000)
    r = synth.host_inputs(wl, 21)
    ids, sc, ref_ids, ref_sc = _both(r, [0, 40000], 4, 512, 0, 40000)
    np.testing.assert_array_equal(ids, ref_ids)
    np.testing.assert_array_equal(sc, ref_sc)
    # 2: a smaller, packed input with another pool size and budget, over a row range
    wl2 = synth.workload("sq4096", T=3000)
    r2 = synth.host_inputs(wl2, 22)
    cu2 = [0, 5, 700, 700, 2100, 3000]
    ids2, sc2, ref_ids2, ref_sc2 = _both(r2, cu2, 2, 9, 3, 2900)
    np.testing.assert_array_equal(ids2, ref_ids2)
    np.testing.assert_array_equal(sc2, ref_sc2)


def test_noalloc_rejects_rows_beyond_the_scratch():
    """One sequence of 16M pools (kpool 1, H=4, D=16): a score row plus its group maxima is
    68,000,000 bytes, beyond the 64 MiB scratch, and the call says so (no GPU needed: the
    check comes before any GPU work)."""
    L = K.lib()
    vp = ctypes.c_void_p
    cu = np.array([0, 16_000_000], dtype=np.int32)
    rc = L.kpool_score_topk_noalloc(vp(16), vp(16), vp(16), cu.ctypes.data_as(vp), vp(16), 1, 4, 16,
                                    1, ctypes.c_float(0.25), 0, 16_000_000, 4, 0, vp(16), None, None)
    assert rc == K.KPOOL_EWORKSPACE
    msg = K.lib().kpool_last_error().decode()
    assert "static scratch" in msg and "68000000" in msg
    # the other argument checks are those of kpool_score_topk
    cu = np.array([0, 64], dtype=np.int32)
    assert L.kpool_score_topk_noalloc(vp(16), vp(16), vp(16), cu.ctypes.data_as(vp), vp(16), 1, 4, 16,
                                      4, ctypes.c_float(0.25), 5, 4, 4, 0, vp(16), None, None) == K.KPOOL_EINVAL
    assert L.kpool_score_topk_noalloc(vp(16), vp(16), vp(16), cu.ctypes.data_as(vp), vp(16), 1, 4, 16,
                                      4, ctypes.c_float(0.25), 0, 64, 4, 4, vp(16), None, None) == K.KPOOL_EINVAL
    assert L.kpool_score_topk_noalloc(None, None, None, cu.ctypes.data_as(vp), None, 1, 4, 16, 4,
                                      ctypes.c_float(0.25), 9, 9, 4, 0, None, None, None) == K.KPOOL_OK
