"""GPU parity over a second, wider family of seeded random configurations.

Beyond test_gpu_random.py's cases, these reach: long sequences (16k-70k tokens, so the
selection reads group maxima and prunes), checked on a window of up to 200 rows that
the oracle scores on its own; kpool 1..16; any budget 1..2048 (every selection
instance); batches of up to 70 sequences (the score launch splits its segment list);
workspaces of 1, 2, 7 or 100 rows or the default, with or without the chunk overlap;
the allocation-free entry point; a score scale from 0.01 to 10 (the ABI takes any scale
> 0); and inputs with signed head weights, exact score ties (keys from {-1, 0, 1}),
all-zero weights or constant keys (every score tied: the selection's exact path).  The
family runs on both compiled score shapes: H=32, D=128 (24 cases, windows of up to 200
rows) and H=4, D=16 (32 cases, windows of up to 600 rows).  The rules are those of the
other parity tests.  Megatron-LM PR #8299, "Test plan" and "Change".
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (check_gated_keys, check_scores, check_selection_vs_oracle, check_topk_self,
                         device_tensors)
from pool_score_top_amd import kpool as K
from pool_score_top_amd import synth

pytestmark = pytest.mark.gpu
# shape: (workload, gated workload, case seed base, input seed base, window rows, cases)
SHAPES = {
    "h32d128": ("sq4096", "sq4096_gated", 90000, 5000, 200, 24),
    "h4d16": ("tiny", "tiny_gated", 120000, 8000, 600, 32),
}
CASES = [(shape, case) for shape, v in SHAPES.items() for case in range(v[5])]


def _config(case, seed_base, window):
    rng = np.random.default_rng(seed_base + case)
    kpool = int(rng.integers(1, 17))
    big = rng.integers(0, 3) == 0
    T = int(rng.integers(16384, 70001)) if big else int(rng.integers(1, 6001))
    nseq = int(rng.choice([1, 2, 5, 12, 40, 70])) if not big else int(rng.choice([1, 2, 3]))
    cuts = np.sort(rng.integers(0, T + 1, size=nseq - 1))
    cu = np.concatenate([[0], cuts, [T]]).astype(np.int32)
    budget = (int(rng.integers(1, 2049)) if rng.integers(0, 2)
              else int(rng.choice([1, 512, 513, 1024, 1025, 2048])))
    tail = bool(rng.integers(0, 3) == 0)
    gated = bool(rng.integers(0, 5) == 0)
    if big:
        q_lo = int(rng.integers(0, T))
        q_hi = min(T, q_lo + int(rng.integers(1, window)))
    else:
        q_lo, q_hi = 0, T
        if rng.integers(0, 2):
            q_lo = int(rng.integers(0, T))
            q_hi = int(rng.integers(q_lo + 1, T + 1))
    ws_rows = [None, 1, 2, 7, 100][int(rng.integers(0, 5))]
    overlap = bool(rng.integers(0, 2))
    noalloc = bool(rng.integers(0, 4) == 0)
    scale = float(np.float32(10.0 ** rng.uniform(-2, 1)))
    variant = str(rng.choice(["", "", "w_neg", "k_ternary", "w_zero", "k_const"]))
    return dict(kpool=kpool, T=T, cu=cu, budget=budget, tail=tail, gated=gated, q_lo=q_lo, q_hi=q_hi,
                ws_rows=ws_rows, overlap=overlap, noalloc=noalloc, scale=scale, variant=variant)


@pytest.mark.parametrize("shape,case", CASES)
def test_wide_random_configuration(shape, case):
    wl_name, wl_gated, seed_base, input_seed, window, _ = SHAPES[shape]
    c = _config(case, seed_base, window)
    kpool, T, cu, budget, tail = c["kpool"], c["T"], c["cu"], c["budget"], c["tail"]
    where = (f"wide case {shape}/{case}: " + str({k: v for k, v in c.items() if k != 'cu'}) +
             f" nseq={len(cu) - 1}")
    print(f"[case] {where}", flush=True)
    wl = synth.workload(wl_gated if c["gated"] else wl_name, T=T, kpool=kpool, budget=budget,
                        variant=c["variant"])
    r = synth.host_inputs(wl, input_seed + case)
    cu_pools_h, max_pools, P = K.count_pools(cu, kpool, tail=tail)
    q, k, w = device_tensors(r)
    n = c["q_hi"] - c["q_lo"]
    cu_dev = torch.from_numpy(cu).cuda()
    cup_dev = torch.from_numpy(cu_pools_h).cuda()
    kp = torch.empty((max(P, 1), wl.D), dtype=torch.int16, device="cuda")
    if c["gated"]:
        K.pool_keys_gated(k, torch.from_numpy(r["g"].view(np.int16)).cuda(), torch.from_numpy(r["ape"]).cuda(),
                          cu, cu_dev, cup_dev, kpool, out=kp, tail=tail)
    else:
        K.pool_keys(k, cu, cu_dev, cup_dev, kpool, out=kp, tail=tail)
    ids = torch.empty((n, budget), dtype=torch.int32, device="cuda")
    scores = torch.empty((n, max(max_pools, 1)), dtype=torch.float32, device="cuda")
    so = scores if max_pools else None
    if c["noalloc"]:
        K.score_topk_noalloc(q, kp, w, cu, cu_dev, kpool, budget, c["q_lo"], c["q_hi"], ids, scores_out=so,
                             scale=c["scale"], tail=tail)
    else:
        ws = None
        if max_pools:
            nb = K.workspace_bytes(c["q_lo"], c["q_hi"], max_pools, 2 if c["overlap"] else 1)
            if c["ws_rows"] is not None:
                nb = min(nb, K.workspace_bytes(0, c["ws_rows"], max_pools, 1))
            ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
        K.score_topk(q, kp, w, cu, cu_dev, kpool, budget, c["q_lo"], c["q_hi"], scale=c["scale"], workspace=ws,
                     pool_ids=ids, scores_out=so, overlap=c["overlap"], tail=tail)
    tok = K.expand(ids, cu, cu_dev, kpool, budget, c["q_lo"], c["q_hi"], tail=tail)
    torch.cuda.synchronize()
    g_kp = kp.cpu().numpy().view(np.uint16)[:P]
    g_ids, g_tok, g_scores = ids.cpu().numpy(), tok.cpu().numpy(), scores.cpu().numpy()
    if c["gated"]:
        kp_o, vals = oracle.pool_keys_gated(r["k"], r["g"], r["ape"], cu, kpool, return_values=True, tail=tail)
        check_gated_keys(g_kp, vals, r["k"], r["g"], r["ape"], cu, kpool, where=where, tail=tail)
    else:
        kp_o = oracle.pool_keys(r["k"], cu, kpool, tail=tail)
    assert np.array_equal(g_kp, kp_o), where + ": kp"
    ref = oracle.select(r["q"], r["k"], r["w"], cu, kpool, budget, q_lo=c["q_lo"], q_hi=c["q_hi"],
                        scale=c["scale"], kp_bits=kp_o, tail=tail)
    rows = np.arange(c["q_lo"], c["q_hi"])
    cu_pools, _ = oracle.count_pools(cu, kpool, tail=tail)
    seq, t = oracle.row_positions(rows, cu)
    nvis = oracle.visible_pools(t, kpool, cu_pools[seq + 1] - cu_pools[seq])
    if max_pools:
        check_scores(g_scores[:, :ref["max_pools"]], ref["scores"], nvis, where)
        check_topk_self(g_scores, g_ids, nvis, budget, where)
        check_selection_vs_oracle(g_ids, ref["scores"], nvis, budget, where)
    else:
        assert np.all(g_ids == -1), where
    for i in range(n):
        tl = None
        if tail:
            L = int(cu[seq[i] + 1] - cu[seq[i]])
            tl = (L // kpool * kpool, L)
        assert np.array_equal(g_tok[i], oracle.expand_row(g_ids[i], int(t[i]), kpool, tl)), where + f" row {rows[i]} tokens"

