"""GPU parity of tail mode (KPOOL_FLAG_TAIL) through the C ABI, against the oracle.

Tail mode is a reading of the pages' "tail append" (Megatron-LM PR #8299,
"Change": pool expansion, tail append and mask filtering): a sequence's pools
are its full pools only, and its remaining L mod kpool tokens are appended to
every row's expanded token ids, filtered causally like them.  Parity against
the pages' own operator is unpinned; the oracle's reading is pinned on the CPU
(test_oracle_tail.py).  Here the HIP path must give: bit-exact pooled keys of
the full pools (mean and gated), scores within rel 1e-3 / abs 1e-4 and -inf
past each row's visible full pools, pool ids equal to the top of its own
scores and to the oracle's selection up to ties within tolerance at the
cutoff, and token ids (tail slots included) equal to the oracle's expansion of
the GPU's ids.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (check_gated_keys, check_scores, check_selection_vs_oracle, check_topk_self,
                         device_tensors, report)
from pool_score_top_amd import kpool as K
from pool_score_top_amd import synth

pytestmark = pytest.mark.gpu


def _run(r, cu, kpool, budget, tail=True, q_lo=0, q_hi=None, workspace_cap=None, overlap=True,
         gated=False):
    q, k, w = device_tensors(r)
    sel = K.Selector(cu, kpool, budget, r["q"].shape[1], r["q"].shape[2], q_lo=q_lo, q_hi=q_hi,
                     workspace_cap=workspace_cap, overlap=overlap, tail=tail)
    scores = torch.empty((sel.q_hi - sel.q_lo, max(sel.max_pools, 1)), dtype=torch.float32,
                         device="cuda")
    g = ape = None
    if gated:
        g = torch.from_numpy(r["g"].view(np.int16)).cuda()
        ape = torch.from_numpy(r["ape"]).cuda()
    out = sel.run(q, k, w, scores_out=scores if sel.max_pools else None, g=g, ape=ape)
    torch.cuda.synchronize()
    return {"kp": out["kp"].cpu().numpy().view(np.uint16), "pool_ids": out["pool_ids"].cpu().numpy(),
            "token_ids": out["token_ids"].cpu().numpy(), "scores": scores.cpu().numpy(),
            "max_pools": sel.max_pools}


def _check_all(r, cu, kpool, budget, res, where, gated=False):
    T = int(cu[-1])
    if gated:
        kp_o, vals = oracle.pool_keys_gated(r["k"], r["g"], r["ape"], cu, kpool, return_values=True,
                                            tail=True)
        check_gated_keys(res["kp"], vals, r["k"], r["g"], r["ape"], cu, kpool, where=where, tail=True)
        np.testing.assert_array_equal(res["kp"], kp_o)
    else:
        kp_o = oracle.pool_keys(r["k"], cu, kpool, tail=True)
        np.testing.assert_array_equal(res["kp"], kp_o)
    ref = oracle.select(r["q"], r["k"], r["w"], cu, kpool, budget, kp_bits=kp_o, tail=True)
    cu_pools, _ = oracle.count_pools(cu, kpool, tail=True)
    seq, t = oracle.row_positions(np.arange(T), cu)
    nvis = oracle.visible_pools(t, kpool, cu_pools[seq + 1] - cu_pools[seq])
    st_sel = {}
    if res["max_pools"]:
        st_s = check_scores(res["scores"][:, :ref["max_pools"]], ref["scores"], nvis, where)
        check_topk_self(res["scores"], res["pool_ids"], nvis, budget, where)
        st_sel = check_selection_vs_oracle(res["pool_ids"], ref["scores"], nvis, budget, where)
    else:
        st_s = {}
        assert np.all(res["pool_ids"] == -1)
    # token ids: the oracle's expansion (tail slots included) of the GPU's own ids
    for i in range(T):
        L = int(cu[seq[i] + 1] - cu[seq[i]])
        want = oracle.expand_row(res["pool_ids"][i], int(t[i]), kpool, (L // kpool * kpool, L))
        assert np.array_equal(res["token_ids"][i], want), f"{where} row {i}: token ids"
    same = (res["pool_ids"] == ref["pool_ids"]).all(axis=1)
    np.testing.assert_array_equal(res["token_ids"][same], ref["token_ids"][same])
    report(where, scores=st_s, selection=st_sel)


@pytest.mark.parametrize("kpool,budget", [(4, 4), (3, 5), (5, 2), (2, 9)])
def test_tail_mode_tiny_packed(kpool, budget):
    """Ragged sequences: lengths not a multiple of kpool, one shorter than kpool (no pool,
    only a tail), an empty one."""
    cu = np.array([0, 3, 3, 40, 41, 77, 120], dtype=np.int32)
    wl = synth.workload("tiny", T=120)
    r = synth.host_inputs(wl, 40 + kpool)
    res = _run(r, cu, kpool, budget)
    _check_all(r, cu, kpool, budget, res, f"tail tiny kpool {kpool}")


@pytest.mark.parametrize("kpool,budget", [(4, 64), (3, 100)])
def test_tail_mode_indexer_shape(kpool, budget):
    cu = np.array([0, 5, 703, 703, 2102, 3001], dtype=np.int32)
    wl = synth.workload("sq4096", T=3001)
    r = synth.host_inputs(wl, 50 + kpool)
    res = _run(r, cu, kpool, budget)
    _check_all(r, cu, kpool, budget, res, f"tail 3001 kpool {kpool}")


@pytest.mark.parametrize("overlap", [False, True])
def test_tail_mode_one_row_chunks_over_sequences_without_pools(overlap):
    """One-row chunks (a one-row workspace) in tail mode, over a batch in which sequences
    shorter than kpool (no full pool, so no visible pool for any of their rows) sit
    between sequences with pools: a chunk that holds only such a row has nothing to
    score, and its rows must still come out as -1 ids and tail tokens."""
    cu = np.array([0, 1, 12, 14, 25, 26, 40, 43, 60], dtype=np.int32)
    kpool, budget = 4, 8
    wl = synth.workload("tiny", T=60)
    r = synth.host_inputs(wl, 70)
    _, max_pools, _ = K.count_pools(cu, kpool, tail=True)
    cap = K.workspace_bytes(0, 1, max_pools, 1)
    res = _run(r, cu, kpool, budget, workspace_cap=cap, overlap=overlap)
    _check_all(r, cu, kpool, budget, res, f"tail one-row chunks overlap={overlap}")


def test_tail_mode_gated_pooling():
    cu = np.array([0, 7, 7, 50, 99, 100], dtype=np.int32)
    wl = synth.workload("tiny_gated", T=100)
    r = synth.host_inputs(wl, 60)
    res = _run(r, cu, 4, 4, gated=True)
    _check_all(r, cu, 4, 4, res, "tail gated", gated=True)


def test_tail_mode_equals_default_on_whole_pools():
    """Every sequence a multiple of kpool: same pools, scores and ids as the default
    mode; the tail slots are all -1."""
    cu = np.array([0, 400, 400, 1200, 2000], dtype=np.int32)
    wl = synth.workload("sq4096", T=2000)
    r = synth.host_inputs(wl, 61)
    a = _run(r, cu, 4, 64, tail=False)
    b = _run(r, cu, 4, 64, tail=True)
    for key in ("kp", "pool_ids", "scores"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
    np.testing.assert_array_equal(b["token_ids"][:, :256], a["token_ids"])
    assert np.all(b["token_ids"][:, 256:] == -1)


def test_tail_mode_row_slices_reassemble_and_noalloc_agrees():
    """Row slices with small workspaces (chunk edges inside sequences) and the
    allocation-free entry point give the full run's bits in tail mode too."""
    cu = np.array([0, 5, 703, 703, 2102, 3001], dtype=np.int32)
    wl = synth.workload("sq4096", T=3001)
    r = synth.host_inputs(wl, 62)
    full = _run(r, cu, 4, 32)
    ld = (full["max_pools"] + 63) // 64 * 64
    row_bytes = (ld + ld // 16) * 4
    for bounds, cap, ov in [((0, 700, 701, 3001), 5 * row_bytes, True),
                            ((0, 1500, 3001), row_bytes, False)]:
        parts = [_run(r, cu, 4, 32, q_lo=a, q_hi=b, workspace_cap=cap, overlap=ov)
                 for a, b in zip(bounds[:-1], bounds[1:])]
        for key in ("pool_ids", "token_ids", "scores"):
            np.testing.assert_array_equal(np.concatenate([p[key] for p in parts]), full[key],
                                          err_msg=f"{key} {bounds}")
    q, k, w = device_tensors(r)
    cu_dev = torch.from_numpy(cu).cuda()
    cu_pools, max_pools, _ = K.count_pools(cu, 4, tail=True)
    kp = K.pool_keys(k, cu, cu_dev, torch.from_numpy(cu_pools).cuda(), 4, tail=True)
    ids = torch.empty((3001, 32), dtype=torch.int32, device="cuda")
    sc = torch.empty((3001, max_pools), dtype=torch.float32, device="cuda")
    K.score_topk_noalloc(q, kp, w, cu, cu_dev, 4, 32, 0, 3001, ids, sc, tail=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy(), full["pool_ids"])
    np.testing.assert_array_equal(sc.cpu().numpy(), full["scores"])


def test_tail_mode_without_any_pool():
    """Every sequence shorter than kpool: no pool exists, every id is -1 and each row's
    token ids are its sequence's tail up to the row."""
    cu = np.array([0, 2, 3, 3, 6], dtype=np.int32)
    wl = synth.workload("tiny", T=6)
    r = synth.host_inputs(wl, 63)
    res = _run(r, cu, 4, 4)
    assert res["max_pools"] == 0 and np.all(res["pool_ids"] == -1)
    ref = oracle.select(r["q"], r["k"], r["w"], cu, 4, 4, tail=True)
    np.testing.assert_array_equal(res["token_ids"], ref["token_ids"])
    assert res["token_ids"][1, 16:].tolist() == [0, 1, -1] and res["token_ids"][5, 16:].tolist() == [0, 1, 2]
