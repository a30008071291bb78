"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

The whole selection runs over 262144 and 524288 tokens (4096- and 8192-row
chunks of a 2 GiB score buffer).  The oracle then checks sampled rows (first
and last rows, both sides of chunk boundaries, random rows):
  * pooled keys of the whole sequence: bit-exact;
  * scores of the sampled rows (from single-row runs with scores_out, which
    must give the same pool ids as the full run): within rel 1e-3 / abs 1e-4;
  * pool ids: exactly the top of the GPU's own scores, and equal to the
    oracle's selection up to pools within tolerance of the cutoff;
  * token ids: the expansion rule.
The heaviest 1/8 row slice [7*sq/8, sq) of the 524288-token run must equal the
same rows of the full run bit for bit (the pages' per-rank query slice).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import check_scores, check_selection_vs_oracle, check_tokens, check_topk_self
from pool_score_top_amd import kpool as K
from pool_score_top_amd import synth

pytestmark = pytest.mark.gpu


def _sample_rows(T, chunk, rng, n_random=12):
    rows = {0, 1, 2, 3, 4, 5, 2047, 2048, T - 2, T - 1}
    for c in (chunk, 2 * chunk, T // 2, T - chunk):
        rows.update({c - 1, c})
    rows.update(rng.integers(0, T, size=n_random).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < T))


def _check_sampled(name, seed=0, n_random=12, check_slice=False):
    wl = synth.workload(name)
    inp = synth.device_inputs(wl, seed)
    cu = inp["cu_seqlens"]
    sel = K.Selector(cu, wl.kpool, wl.budget, wl.H, wl.D)
    out = sel.run(inp["q"], inp["k"], inp["w"])
    torch.cuda.synchronize()
    kp_gpu = out["kp"].cpu().numpy().view(np.uint16)
    ids_full = out["pool_ids"].cpu().numpy()
    tok_full = out["token_ids"].cpu().numpy()
    pitch = ((sel.max_pools + 63) // 64) * 64
    chunk = min(wl.T, (1 << 31) // (pitch * 4))

    k_host = inp["k"].cpu().numpy().view(np.uint16)
    kp_o = oracle.pool_keys(k_host, cu, wl.kpool)
    np.testing.assert_array_equal(kp_gpu, kp_o)

    rows = _sample_rows(wl.T, chunk, np.random.default_rng(seed + 17), n_random)
    # GPU scores of the sampled rows: single-row runs of the same kernels
    g_scores = np.empty((len(rows), sel.max_pools), dtype=np.float32)
    g_ids = np.empty((len(rows), wl.budget), dtype=np.int32)
    for i, r in enumerate(rows):
        ids, sc = K.score_topk(inp["q"], out["kp"], inp["w"], cu, sel.cu_dev, wl.kpool, wl.budget,
                               int(r), int(r) + 1, want_scores=True)
        g_scores[i] = sc.cpu().numpy()[0]
        g_ids[i] = ids.cpu().numpy()[0]
    np.testing.assert_array_equal(g_ids, ids_full[rows])

    idx = torch.from_numpy(rows).cuda()
    qs = inp["q"].index_select(0, idx).cpu().numpy().view(np.uint16)
    ws = inp["w"].index_select(0, idx).cpu().numpy()
    cu_pools, max_pools = oracle.count_pools(cu, wl.kpool)
    seq, t = oracle.row_positions(rows, cu)
    o_scores = np.full((len(rows), max_pools), -np.inf)
    for i in range(len(rows)):
        o_scores[i] = oracle.row_scores(qs[i:i + 1], ws[i:i + 1], kp_o, cu_pools, seq[i:i + 1],
                                        t[i:i + 1], wl.kpool, width=max_pools)[0]
    nvis = t // wl.kpool + 1
    check_scores(g_scores, o_scores, nvis, name)
    check_topk_self(g_scores, g_ids, nvis, wl.budget, name)
    check_selection_vs_oracle(g_ids, o_scores, nvis, wl.budget, name)
    check_tokens(tok_full[rows], ids_full[rows], t, wl.kpool, where=name)

    if check_slice:
        lo, hi = 7 * wl.T // 8, wl.T
        sl = K.Selector(cu, wl.kpool, wl.budget, wl.H, wl.D, q_lo=lo, q_hi=hi)
        so = sl.run(inp["q"], inp["k"], inp["w"])
        torch.cuda.synchronize()
        np.testing.assert_array_equal(so["pool_ids"].cpu().numpy(), ids_full[lo:hi])
        np.testing.assert_array_equal(so["token_ids"].cpu().numpy(), tok_full[lo:hi])


def test_sq262144_sampled_rows():
    _check_sampled("sq262144", seed=0, n_random=8)


def test_sq262144_per_token_sampled_rows():
    _check_sampled("sq262144_k1", seed=0, n_random=6)


def test_sq524288_sampled_rows_and_last_eighth_slice():
    _check_sampled("sq524288", seed=0, n_random=8, check_slice=True)
