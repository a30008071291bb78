"""GPU parity over seeded random configurations of the whole path, against the oracle.

(A one-off sweep of 324 such cases found one-row chunks in tail mode that held only rows
of sequences shorter than kpool, whose score launch had an empty grid; the chunk loop
now skips it.  64 cases run here.)

Each case draws, from its own seed: a packed batch of 1..12 sequences (some empty, the
rest of random lengths, up to 4000 tokens in all), kpool 1..6, a budget that lands in
either selection instance (1 .. 2048), mean or gated pooling, the default or the tail
mode, a query-row range [q_lo, q_hi) (often the whole batch), and a workspace of 1, 5 or
33 score rows or the default, with or without the chunk overlap.  The HIP path runs
through the C ABI; the comparison rules are those of the other parity tests (pooled keys
bit-exact, scores within rel 1e-3 / abs 1e-4 and the fp32 error bound, -inf past each
row's visible pools, ids equal to the top of the GPU's own scores and to the oracle's
selection up to ties at the cutoff, token ids equal to the oracle's expansion of the
GPU's ids).  Megatron-LM PR #8299, "Test plan" (packed varlen bounds, row ranges that
match the unsharded call) and "Change" (the chunk loop over a row range).
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
NCASES = 64


def _config(case):
    rng = np.random.default_rng(7000 + case)
    kpool = int(rng.choice([1, 2, 3, 4, 5, 6]))
    T = int(rng.integers(1, (2000 if kpool == 1 else 4000) + 1))
    nseq = int(rng.integers(1, 13))
    cuts = np.sort(rng.integers(0, T + 1, size=nseq - 1))
    cu = np.concatenate([[0], cuts, [T]]).astype(np.int32)
    budget = int(rng.choice([1, 2, 7, 64, 300, 512, 513, 1000, 2048]))
    tail = bool(rng.integers(0, 2))
    gated = bool(rng.integers(0, 4) == 0)
    q_lo, q_hi = 0, T
    if rng.integers(0, 2):
        q_lo = int(rng.integers(0, T))
        q_hi = int(rng.integers(q_lo + 1, T + 1))
    ws_rows = [None, 1, 5, 33][int(rng.integers(0, 4))]
    overlap = bool(rng.integers(0, 2))
    return dict(kpool=kpool, T=T, cu=cu, budget=budget, tail=tail, gated=gated, q_lo=q_lo,
                q_hi=q_hi, ws_rows=ws_rows, overlap=overlap)


@pytest.mark.parametrize("case", range(NCASES))
def test_random_configuration(case):
    c = _config(case)
    kpool, T, cu, budget, tail = c["kpool"], c["T"], c["cu"], c["budget"], c["tail"]
    where = (f"random case {case}: T={T} nseq={len(cu) - 1} kpool={kpool} budget={budget} "
             f"tail={tail} gated={c['gated']} rows=[{c['q_lo']},{c['q_hi']}) ws_rows={c['ws_rows']} "
             f"overlap={c['overlap']}")
    print(f"[case] {where}", flush=True)
    wl = synth.workload("sq4096_gated" if c["gated"] else "sq4096", T=T, kpool=kpool, budget=budget)
    r = synth.host_inputs(wl, 300 + case)
    _, max_pools, _ = K.count_pools(cu, kpool, tail=tail)
    cap = None
    if c["ws_rows"] is not None and max_pools > 0:
        cap = K.workspace_bytes(0, c["ws_rows"], max_pools, 1)

    # GPU
    q, k, w = device_tensors(r)
    sel = K.Selector(cu, kpool, budget, wl.H, wl.D, q_lo=c["q_lo"], q_hi=c["q_hi"], workspace_cap=cap,
                     overlap=c["overlap"], tail=tail)
    n = sel.q_hi - sel.q_lo
    scores = torch.empty((n, max(sel.max_pools, 1)), dtype=torch.float32, device="cuda")
    g = ape = None
    if c["gated"]:
        g = torch.from_numpy(r["g"].view(np.int16)).cuda()
        ape = torch.from_numpy(r["ape"]).cuda()
    out = sel.run(q, k, w, scores_out=scores if sel.max_pools else None, g=g, ape=ape)
    torch.cuda.synchronize()
    g_kp = out["kp"].cpu().numpy().view(np.uint16)
    g_ids = out["pool_ids"].cpu().numpy()
    g_tok = out["token_ids"].cpu().numpy()
    g_scores = scores.cpu().numpy()

    # oracle
    if c["gated"]:
        kp_o, vals = oracle.pool_keys_gated(r["k"], r["g"], r["ape"], cu, kpool, return_values=True,
                                            tail=tail)
        check_gated_keys(g_kp, vals, r["k"], r["g"], r["ape"], cu, kpool, where=where, tail=tail)
    else:
        kp_o = oracle.pool_keys(r["k"], cu, kpool, tail=tail)
    np.testing.assert_array_equal(g_kp, kp_o, err_msg=where)
    ref = oracle.select(r["q"], r["k"], r["w"], cu, kpool, budget, q_lo=c["q_lo"], q_hi=c["q_hi"],
                        kp_bits=kp_o, tail=tail)
    assert ref["max_pools"] == sel.max_pools
    rows = np.arange(c["q_lo"], c["q_hi"])
    cu_pools, _ = oracle.count_pools(cu, kpool, tail=tail)
    seq, t = oracle.row_positions(rows, cu)
    nvis = oracle.visible_pools(t, kpool, cu_pools[seq + 1] - cu_pools[seq])
    st_s = st_sel = {}
    if sel.max_pools:
        st_s = check_scores(g_scores[:, :ref["max_pools"]], ref["scores"], nvis, where)
        check_topk_self(g_scores, g_ids, nvis, budget, where)
        st_sel = check_selection_vs_oracle(g_ids, ref["scores"], nvis, budget, where)
    else:
        assert np.all(g_ids == -1), where
    for i in range(n):
        tl = None
        if tail:
            L = int(cu[seq[i] + 1] - cu[seq[i]])
            tl = (L // kpool * kpool, L)
        want = oracle.expand_row(g_ids[i], int(t[i]), kpool, tl)
        assert np.array_equal(g_tok[i], want), f"{where} row {rows[i]}: token ids"
    same = (g_ids == ref["pool_ids"]).all(axis=1)
    np.testing.assert_array_equal(g_tok[same], ref["token_ids"][same], err_msg=where)
    report(where, scores=st_s, selection=st_sel)
