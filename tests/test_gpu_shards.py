"""The pages' query-shard test matrix on one GPU, through the C ABI.

Megatron-LM PR #8299, "Change": with a shard group of size G, rank r scores
the rows [r*ceil(sq/G), min(sq, (r+1)*ceil(sq/G))) through the chunked path,
and the shards are concatenated.  "Test plan": every simulated rank's result
is compared bitwise with the unsharded call, for a causal mask with shard
sizes 2/3/8 and sq in {5, 24, 37} (a ragged last shard, and empty shards when
sq < G), batch 1 and 2, with and without a small score-chunk cap so that shard
edges fall inside the chunk loop; for packed THD batches with shard sizes 2/4;
each rank scores only its own rows, and the bounds cover every row once.

Here each rank is one kpool_score_topk / kpool_expand call over its row range.
Every call writes into its rows of buffers pre-filled with a sentinel, and
the rows outside its range must still hold the sentinel afterwards (the call
scored only its rows).  The concatenation must equal the unsharded call bit
for bit: pool ids, token ids and the fp32 scores.  The unsharded call itself
is checked against the oracle.  "Batch 2" is two sequences of sq tokens packed
one after the other; a rank's shard is its row range in each of them.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import device_tensors
from pool_score_top_amd import kpool as K
from pool_score_top_amd import synth

pytestmark = pytest.mark.gpu

SENT_ID = -7
SENT_SCORE = 12345.5


def shard_bounds(sq, G):
    per = -(-sq // G)
    return [(min(sq, r * per), min(sq, (r + 1) * per)) for r in range(G)]


def _run_sharded(r, cu, kpool, budget, ranges_per_rank, ws_rows, H, D):
    """Run every rank's row ranges into sentinel-filled buffers; return the buffers."""
    q, k, w = device_tensors(r)
    T = int(cu[-1])
    cu_dev = torch.from_numpy(cu).cuda()
    cu_pools, max_pools, _ = K.count_pools(cu, kpool)
    kp = K.pool_keys(k, cu, cu_dev, torch.from_numpy(cu_pools).cuda(), kpool)
    ld = (max_pools + 63) // 64 * 64
    ws = None if ws_rows is None else torch.empty(ws_rows * (ld + ld // 16) * 4, dtype=torch.uint8,
                                                  device="cuda")
    ids = torch.full((T, budget), SENT_ID, dtype=torch.int32, device="cuda")
    sc = torch.full((T, max_pools), SENT_SCORE, dtype=torch.float32, device="cuda")
    tok = torch.full((T, budget * kpool), SENT_ID, dtype=torch.int32, device="cuda")
    covered = np.zeros(T, dtype=np.int64)
    for rank_ranges in ranges_per_rank:
        before = (ids.clone(), sc.clone(), tok.clone())
        mine = np.zeros(T, dtype=bool)
        for lo, hi in rank_ranges:
            assert 0 <= lo <= hi <= T
            K.score_topk(q, kp, w, cu, cu_dev, kpool, budget, lo, hi, workspace=ws,
                         pool_ids=ids[lo:hi], scores_out=sc[lo:hi] if hi > lo else None,
                         overlap=ws_rows is None or ws_rows >= 2)
            K.expand(ids[lo:hi], cu, cu_dev, kpool, budget, lo, hi, out=tok[lo:hi])
            mine[lo:hi] = True
            covered[lo:hi] += 1
        torch.cuda.synchronize()
        other = torch.from_numpy(~mine).cuda()
        for a, b in zip((ids, sc, tok), before):
            assert torch.equal(a[other], b[other]), "a rank wrote rows outside its shard"
    assert np.all(covered == 1), "shard bounds must cover every row exactly once"
    return {"pool_ids": ids.cpu().numpy(), "scores": sc.cpu().numpy(),
            "token_ids": tok.cpu().numpy(), "max_pools": max_pools}


def _unsharded(r, cu, kpool, budget, H, D):
    full = _run_sharded(r, cu, kpool, budget, [[(0, int(cu[-1]))]], None, H, D)
    ref = oracle.select(r["q"], r["k"], r["w"], cu, kpool, budget)
    np.testing.assert_array_equal(full["pool_ids"], ref["pool_ids"])
    np.testing.assert_array_equal(full["token_ids"], ref["token_ids"])
    return full


def _assert_same(a, b, where):
    for key in ("pool_ids", "token_ids", "scores"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=f"{where}: {key}")


@pytest.mark.parametrize("sq", [5, 24, 37])
@pytest.mark.parametrize("batch", [1, 2])
def test_causal_shards_equal_unsharded(sq, batch):
    wl = synth.workload("tiny", T=batch * sq)
    r = synth.host_inputs(wl, 100 + sq)
    cu = np.array([b * sq for b in range(batch + 1)], dtype=np.int32)
    full = _unsharded(r, cu, wl.kpool, wl.budget, wl.H, wl.D)
    for G in (2, 3, 8):
        ranks = [[(b * sq + lo, b * sq + hi) for b in range(batch)] for lo, hi in shard_bounds(sq, G)]
        if sq < G:
            assert any(lo == hi for lo, hi in shard_bounds(sq, G))   # empty shards occur
        for ws_rows in (None, 1, 3):   # default workspace; a chunk cap of 1 and 3 rows
            got = _run_sharded(r, cu, wl.kpool, wl.budget, ranks, ws_rows, wl.H, wl.D)
            _assert_same(got, full, f"sq={sq} batch={batch} G={G} ws_rows={ws_rows}")


@pytest.mark.parametrize("G", [2, 4])
def test_thd_shards_equal_unsharded(G):
    """Packed ragged sequences (an empty one and a one-token one among them), shards over
    the packed rows, so shard edges fall inside sequences and inside pools."""
    cu = np.array([0, 7, 7, 30, 31, 52, 61], dtype=np.int32)
    T = int(cu[-1])
    wl = synth.workload("tiny", T=T)
    r = synth.host_inputs(wl, 200 + G)
    r["cu_seqlens"] = cu
    full = _unsharded(r, cu, wl.kpool, wl.budget, wl.H, wl.D)
    ranks = [[b] for b in shard_bounds(T, G)]
    for ws_rows in (None, 1, 3):
        got = _run_sharded(r, cu, wl.kpool, wl.budget, ranks, ws_rows, wl.H, wl.D)
        _assert_same(got, full, f"THD G={G} ws_rows={ws_rows}")


def test_shards_at_the_indexer_shape():
    """The same property at H=32, D=128, kpool 4 (budget 64), sq = 4099 with G = 8: a
    ragged last shard, shard edges inside 32-row score tiles, 64-pool stages and chunks."""
    sq = 4099
    wl = synth.workload("sq4096", T=sq, budget=64)
    r = synth.host_inputs(wl, 9)
    cu = np.array([0, sq], dtype=np.int32)
    full = _run_sharded(r, cu, 4, 64, [[(0, sq)]], None, wl.H, wl.D)
    ranks = [[b] for b in shard_bounds(sq, 8)]
    for ws_rows in (None, 100):
        got = _run_sharded(r, cu, 4, 64, ranks, ws_rows, wl.H, wl.D)
        _assert_same(got, full, f"sq={sq} G=8 ws_rows={ws_rows}")
