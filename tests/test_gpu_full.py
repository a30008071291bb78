"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

The whole selection runs over 262144 and 524288 tokens (and the heaviest 1/8
query slice of 524288), with the workspace bench.py uses (one 2 GiB chunk
buffer, chunks one after the other on one stream).  Then, for at least 16
windows of 64 consecutive rows per workload (the first rows, both sides of
several chunk edges, the last rows, and seeded random windows):

  * the chunk that holds a window is run again on its own, exactly as the full
    run launched it (same chunk bounds, so the same row tiles and pool segments
    of the score kernel and the same top-k launch), with scores_out; its pool
    ids must equal the full run's bit for bit, and its fp32 scores are the
    production kernels' scores of those rows;
  * those scores are compared element by element with the fp64 oracle on every
    visible (row, pool) of the window, within rel 1e-3 / abs 1e-4 and within the
    fp32 error bound of the arithmetic (on the first windows);
  * the pool ids are exactly the top of the GPU's own scores, and agree with the
    oracle's selection up to pools within tolerance of the cutoff;
  * the token ids follow the expansion rule;
  * the pooled keys of the whole sequence are bit-exact.
The error figures are printed per workload.  The heaviest slice is checked
against the oracle with its own windows, and also equals the same rows of the
full run bit for bit (Megatron-LM PR #8299, "Test plan": every row of a sharded
run matches the unsharded computation).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (check_scores, check_selection_vs_oracle, check_tokens, check_topk_self,
                         fp32_error_bound, report)
from pool_score_top_amd import kpool as K
from pool_score_top_amd import synth

pytestmark = pytest.mark.gpu

WIN = 64
_CACHE = {}


def _inputs(wl, seed=0):
    key = (wl.T, wl.H, wl.D, wl.variant, seed)
    if key not in _CACHE:
        _CACHE.clear()  # one full-size input set at a time
        torch.cuda.empty_cache()
        _CACHE[key] = synth.device_inputs(wl, seed)
    return _CACHE[key]


def _windows(lo, hi, chunk, rng, n_random=8):
    """Window starts: first rows, both sides of chunk edges, last rows, random."""
    starts = {lo, hi - WIN}
    for e in (lo + chunk, lo + 2 * chunk, lo + (hi - lo) // 2 // chunk * chunk, hi - chunk):
        if lo + WIN // 2 <= e <= hi - WIN // 2:
            starts.add(e - WIN // 2)            # straddles the edge
            starts.add(max(lo, e - WIN))        # ends at the edge
            starts.add(min(hi - WIN, e))        # starts at the edge
    while len(starts) < 16 + n_random // 2:
        starts.add(int(rng.integers(lo, hi - WIN + 1)))
    return sorted(starts)


def _check_workload(name, seed=0, bound_windows=4):
    wl = synth.workload(name)
    inp = _inputs(wl, seed)
    cu = inp["cu_seqlens"]
    lo, hi = wl.rows
    print(f"[parity] {name}: full run of rows [{lo}, {hi})", flush=True)
    sel = K.Selector(cu, wl.kpool, wl.budget, wl.H, wl.D, q_lo=lo, q_hi=hi)
    out = sel.run(inp["q"], inp["k"], inp["w"])
    torch.cuda.synchronize()
    chunk = sel.chunk_rows()

    k_host = inp["k"].cpu().numpy().view(np.uint16)
    kp_o = oracle.pool_keys(k_host, cu, wl.kpool)
    np.testing.assert_array_equal(out["kp"].cpu().numpy().view(np.uint16), kp_o)

    starts = _windows(lo, hi, chunk, np.random.default_rng(seed + 17))
    assert len(starts) >= 16
    # chunks of the full run holding window rows, each re-run on its own with scores_out
    chunk_of = lambda r: lo + (r - lo) // chunk * chunk  # noqa: E731
    needed = sorted({chunk_of(s) for s in starts} | {chunk_of(s + WIN - 1) for s in starts})
    cu_pools, max_pools = oracle.count_pools(cu, wl.kpool)
    g_scores, g_ids = {}, {}
    scores_buf = torch.empty((min(chunk, hi - lo), sel.max_pools), dtype=torch.float32,
                             device="cuda")
    ids_buf = torch.empty((min(chunk, hi - lo), wl.budget), dtype=torch.int32, device="cuda")
    rows_all = np.concatenate([np.arange(s, s + WIN) for s in starts])
    for c0 in needed:
        c1 = min(hi, c0 + chunk)
        n = c1 - c0
        K.score_topk(inp["q"], out["kp"], inp["w"], cu, sel.cu_dev, wl.kpool, wl.budget, c0, c1,
                     workspace=sel.workspace, pool_ids=ids_buf[:n], scores_out=scores_buf[:n],
                     overlap=False)
        # the re-run chunk is the full run's chunk: every id of it equal
        assert torch.equal(ids_buf[:n], out["pool_ids"][c0 - lo:c1 - lo]), f"{name} chunk {c0}"
        mine = rows_all[(rows_all >= c0) & (rows_all < c1)]
        idx = torch.from_numpy(mine - c0).cuda()
        sc = scores_buf[:n].index_select(0, idx).cpu().numpy()
        ids = ids_buf[:n].index_select(0, idx).cpu().numpy()
        for j, r in enumerate(mine):
            g_scores[int(r)] = sc[j]
            g_ids[int(r)] = ids[j]
    torch.cuda.synchronize()

    tok_idx = torch.from_numpy(rows_all - lo).cuda()
    tok_all = out["token_ids"].index_select(0, tok_idx).cpu().numpy()
    stats_s, stats_sel = [], []
    for wi, s in enumerate(starts):
        rows = np.arange(s, s + WIN)
        qs = inp["q"][s:s + WIN].cpu().numpy().view(np.uint16)
        ws = inp["w"][s:s + WIN].cpu().numpy()
        seq, t = oracle.row_positions(rows, cu)
        o = oracle.row_scores(qs, ws, kp_o, cu_pools, seq, t, wl.kpool, width=max_pools)
        gs = np.stack([g_scores[int(r)] for r in rows])
        gi = np.stack([g_ids[int(r)] for r in rows])
        nvis = t // wl.kpool + 1
        bound = None
        if wi < bound_windows or s in (starts[0], starts[-1]):
            bound = fp32_error_bound(qs, ws, kp_o, cu_pools, seq, t, wl.kpool, wl.D, wl.H, max_pools)
        where = f"{name} window [{s}, {s + WIN})"
        stats_s.append(check_scores(gs, o, nvis, where, bound=bound))
        check_topk_self(gs, gi, nvis, wl.budget, where)
        stats_sel.append(check_selection_vs_oracle(gi, o, nvis, wl.budget, where))
        check_tokens(tok_all[wi * WIN:(wi + 1) * WIN], gi, t, wl.kpool, where=where)
    agg_s = {"windows": len(starts), "pairs": sum(x["pairs"] for x in stats_s)}
    for k in ("max_abs", "max_rel", "max_err_over_tol", "max_err_over_bound"):
        agg_s[k] = max(x[k] for x in stats_s)
    agg_sel = {k: sum(x[k] for x in stats_sel) for k in ("rows", "rows_differing", "pools_differing",
                                                         "pools_between_tau_and_2tau")}
    agg_sel["worst_cutoff_dist_over_tau"] = max(x["worst_cutoff_dist_over_tau"] for x in stats_sel)
    report(f"{name} (chunk {chunk} rows, {len(needed)} chunks re-run)", scores=agg_s,
           selection=agg_sel)
    return wl, inp, out


def test_sq262144_windows():
    _check_workload("sq262144")


def test_sq262144_per_token_windows():
    _check_workload("sq262144_k1")


def test_sq524288_windows():
    _check_workload("sq524288")


def test_sq524288_last_eighth_slice_windows_and_equality():
    wl, inp, out = _check_workload("sq524288_slice")
    lo, hi = wl.rows
    full = K.Selector(inp["cu_seqlens"], wl.kpool, wl.budget, wl.H, wl.D)
    fo = full.run(inp["q"], inp["k"], inp["w"])
    torch.cuda.synchronize()
    assert torch.equal(out["pool_ids"], fo["pool_ids"][lo:hi])
    assert torch.equal(out["token_ids"], fo["token_ids"][lo:hi])
