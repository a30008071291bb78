"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Sizes here are ones the oracle finishes in seconds but that still span many
score tiles (32 rows), LDS stages (64 pools), pool segments and top-k
candidate sorts, with ragged tails everywhere.  Full-size workloads are
checked on sampled rows in test_gpu_full.py.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (check_scores, check_selection_vs_oracle, check_tokens, check_topk_self,
                         device_tensors, oracle_rows, run_gpu)
from pool_score_top_amd import kpool as K
from pool_score_top_amd import synth

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _inputs(name, seed=0, **over):
    wl = synth.workload(name, **over)
    r = synth.host_inputs(wl, seed)
    return wl, r


def _full_check(wl, r, res, rows=None, where=""):
    """Every comparison rule on the given rows (default: all rows)."""
    cu = r["cu_seqlens"]
    if rows is None:
        rows = np.arange(wl.T)
    kp, o_scores, t = oracle_rows(r, wl.kpool, rows, width=res["max_pools"])
    np.testing.assert_array_equal(res["kp"], kp)
    nvis = t // wl.kpool + 1
    g_scores = res["scores"][rows - 0]
    check_scores(g_scores, o_scores, nvis, where)
    check_topk_self(g_scores, res["pool_ids"][rows], nvis, wl.budget, where)
    check_selection_vs_oracle(res["pool_ids"][rows], o_scores, nvis, wl.budget, where)
    o_ids = np.stack([oracle.select_row(o_scores[i, :nvis[i]], wl.budget) for i in range(len(rows))])
    o_tok = np.stack([oracle.expand_row(o_ids[i], int(t[i]), wl.kpool) for i in range(len(rows))])
    check_tokens(res["token_ids"][rows], res["pool_ids"][rows], t, wl.kpool, o_ids, o_tok, where)
    return o_ids


# ---------------------------------------------------------------------------
# Pooling: bit-exact
# ---------------------------------------------------------------------------

def test_pool_keys_hand_values():
    with open(os.path.join(GOLDEN, "pool_pins.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        k1 = np.array([int(x, 16) for x in c["keys"]], dtype=np.uint16)
        k = np.repeat(k1[:, None], 8, axis=1)          # D = 8, every column the same case
        cu = np.array([0, len(k1)], dtype=np.int32)
        cu_pools, _, P = K.count_pools(cu, c["kpool"])
        kd = torch.from_numpy(k.view(np.int16)).cuda()
        kp = K.pool_keys(kd, cu, torch.from_numpy(cu).cuda(), torch.from_numpy(cu_pools).cuda(),
                         c["kpool"])
        got = kp.cpu().numpy().view(np.uint16)
        want = np.array([int(x, 16) for x in c["pooled"]], dtype=np.uint16)
        assert np.array_equal(got, np.repeat(want[:, None], 8, axis=1)), c["name"]


@pytest.mark.parametrize("name,seed,variant", [
    ("tiny", 0, ""), ("sq4096", 1, ""), ("thd65536", 2, ""), ("sq4096", 3, "k_ternary"),
])
def test_pool_keys_bitexact(name, seed, variant):
    wl, r = _inputs(name, seed, variant=variant)
    cu = r["cu_seqlens"]
    cu_pools, _, _ = K.count_pools(cu, wl.kpool)
    kd = torch.from_numpy(r["k"].view(np.int16)).cuda()
    kp = K.pool_keys(kd, cu, torch.from_numpy(cu).cuda(), torch.from_numpy(cu_pools).cuda(), wl.kpool)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(kp.cpu().numpy().view(np.uint16), oracle.pool_keys(r["k"], cu, wl.kpool))


@pytest.mark.parametrize("kpool", [1, 2, 3, 5])
def test_pool_keys_other_pool_sizes(kpool):
    wl, r = _inputs("tiny", 4, T=203)
    cu = np.array([0, 1, 50, 50, 203], dtype=np.int32)
    cu_pools, _, _ = K.count_pools(cu, kpool)
    kd = torch.from_numpy(r["k"].view(np.int16)).cuda()
    kp = K.pool_keys(kd, cu, torch.from_numpy(cu).cuda(), torch.from_numpy(cu_pools).cuda(), kpool)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(kp.cpu().numpy().view(np.uint16), oracle.pool_keys(r["k"], cu, kpool))


# ---------------------------------------------------------------------------
# Whole path vs the oracle
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_workload(seed):
    wl, r = _inputs("tiny", seed)
    res = run_gpu(r, wl.kpool, wl.budget)
    _full_check(wl, r, res, where=f"tiny s{seed}")


@pytest.mark.parametrize("variant", ["", "w_neg", "k_ternary", "w_zero"])
def test_tiny_shapes_variants(variant):
    wl, r = _inputs("tiny", 7, T=300, variant=variant)
    r["cu_seqlens"] = np.array([0, 1, 2, 37, 37, 100, 300], dtype=np.int32)
    for budget in (1, 4, 13):
        res = run_gpu(r, wl.kpool, budget)
        _full_check(synth.workload("tiny", T=300, budget=budget), r, res, where=f"{variant} b{budget}")


def test_many_short_sequences_and_odd_pool_sizes():
    """More than 32 sequences in one chunk (the score launch splits its segment list),
    empty and one-token sequences, and pool sizes 2, 3 and 5 through the whole path."""
    wl, r = _inputs("sq4096", 12, T=3000)
    rng = np.random.default_rng(12)
    lens = rng.integers(0, 70, size=80)
    lens[::9] = 0
    lens[1::9] = 1
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cu = cu[cu <= 3000]
    if cu[-1] < 3000:
        cu = np.concatenate([cu, [3000]]).astype(np.int32)
    r["cu_seqlens"] = cu
    assert len(cu) - 1 > 64
    for kpool, budget in ((2, 9), (3, 5), (5, 3)):
        res = run_gpu(r, kpool, budget)
        _full_check(synth.workload("sq4096", T=3000, kpool=kpool, budget=budget), r, res,
                    where=f"many seqs kpool {kpool}")


@pytest.mark.parametrize("name", ["sq4096", "sq4096_k1"])
def test_sq4096_workload(name):
    wl, r = _inputs(name, 0)
    res = run_gpu(r, wl.kpool, wl.budget)
    _full_check(wl, r, res, where=name)


@pytest.mark.parametrize("name", ["thd65536", "thd65536_k1"])
def test_thd_workload_windows(name):
    wl, r = _inputs(name, 0)
    cu = r["cu_seqlens"]
    res = run_gpu(r, wl.kpool, wl.budget, want_scores=False)
    # windows at every sequence start and end plus a spread of interior rows
    rows = set()
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        rows.update(range(a, min(b, a + 6)))
        rows.update(range(max(a, b - 6), b))
    rows.update(np.linspace(0, wl.T - 1, 40).astype(int).tolist())
    rows = np.array(sorted(rows))
    # scores for those rows come from a second GPU call per row (same kernels, own range)
    q, k, w = device_tensors(r)
    sel = K.Selector(cu, wl.kpool, wl.budget, wl.H, wl.D)
    kp = K.pool_keys(k, cu, sel.cu_dev, sel.cu_pools_dev, wl.kpool)
    g_scores = np.empty((len(rows), sel.max_pools), dtype=np.float32)
    g_ids = np.empty((len(rows), wl.budget), dtype=np.int32)
    for i, row in enumerate(rows):
        ids, sc = K.score_topk(q, kp, w, cu, sel.cu_dev, wl.kpool, wl.budget, int(row), int(row) + 1,
                               want_scores=True)
        g_scores[i] = sc.cpu().numpy()[0]
        g_ids[i] = ids.cpu().numpy()[0]
    np.testing.assert_array_equal(g_ids, res["pool_ids"][rows])     # row split == full run
    kp_o, o_scores, t = oracle_rows(r, wl.kpool, rows, width=sel.max_pools)
    np.testing.assert_array_equal(res["kp"], kp_o)
    nvis = t // wl.kpool + 1
    check_scores(g_scores, o_scores, nvis, name)
    check_topk_self(g_scores, g_ids, nvis, wl.budget, name)
    check_selection_vs_oracle(g_ids, o_scores, nvis, wl.budget, name)
    check_tokens(res["token_ids"][rows], res["pool_ids"][rows], t, wl.kpool, where=name)


# ---------------------------------------------------------------------------
# Invariants of the whole path
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kpool,budget", [(4, 64), (1, 1100)])
def test_row_split_and_chunking_reassemble_bitwise(kpool, budget):
    """Slices [q_lo, q_hi) with a workspace of a few rows (many chunks, slice edges inside
    chunks and tiles) concatenate to the single full run, scores and ids alike
    (Megatron-LM PR #8299, 'Test plan': sharded == unsharded, small chunk cap)."""
    wl, r = _inputs("sq4096", 5, T=1500, kpool=kpool)
    r["cu_seqlens"] = np.array([0, 700, 701, 1500], dtype=np.int32)
    full = run_gpu(r, wl.kpool, budget)
    pitch = ((full["max_pools"] + 63) // 64) * 64
    row_bytes = (pitch + pitch // 16) * 4     # one score row plus its 16-pool group maxima
    for bounds, cap in [((0, 333, 334, 1000, 1500), 7 * row_bytes), ((0, 1, 700, 1499, 1500), row_bytes),
                        ((0, 750, 1500), 100 * row_bytes)]:
        parts = [run_gpu(r, wl.kpool, budget, q_lo=a, q_hi=b, workspace_cap=cap)
                 for a, b in zip(bounds[:-1], bounds[1:])]
        for key in ("pool_ids", "token_ids", "scores"):
            np.testing.assert_array_equal(np.concatenate([p[key] for p in parts]), full[key], err_msg=key)
    # the same chunks serialised on one stream (flags = 0) give the same bits
    serial = run_gpu(r, wl.kpool, budget, workspace_cap=7 * row_bytes, overlap=False)
    for key in ("pool_ids", "token_ids", "scores"):
        np.testing.assert_array_equal(serial[key], full[key], err_msg=key)


@pytest.mark.parametrize("budget", [2048, 1000, 600, 512])
def test_per_token_long_rows_use_group_pruning(budget):
    """kpool 1, rows that see more than 65536 pools (4100+ groups of 16): the top-k reads
    the score kernel's group maxima first and then only candidate groups, in each of its
    instances (budget 2048: 8 maxima per thread over 512 threads; 1000 and 600: 4 over
    512; 512: 4 over 256); checked against the oracle on a window of such rows, with a
    small workspace so the window spans several chunks."""
    wl, r = _inputs("sq4096_k1", 11, T=67000)
    lo, hi = 66000, 66090
    pitch = (67000 + 63) // 64 * 64
    res = run_gpu(r, 1, budget, q_lo=lo, q_hi=hi, workspace_cap=20 * (pitch + pitch // 16) * 4)
    rows = np.arange(lo, hi)
    kp, o_scores, t = oracle_rows(r, 1, rows, width=res["max_pools"])
    np.testing.assert_array_equal(res["kp"], kp)
    nvis = t + 1
    where = f"k1 long budget {budget}"
    check_scores(res["scores"], o_scores, nvis, where)
    check_topk_self(res["scores"], res["pool_ids"], nvis, budget, where)
    check_selection_vs_oracle(res["pool_ids"], o_scores, nvis, budget, where)
    check_tokens(res["token_ids"], res["pool_ids"], t, 1, where=where)


def test_thd_packing_invariance():
    wl, r = _inputs("sq4096", 6, T=2000)
    cu = np.array([0, 333, 1200, 2000], dtype=np.int32)
    r["cu_seqlens"] = cu
    packed = run_gpu(r, wl.kpool, 32)
    for s in range(3):
        a, b = int(cu[s]), int(cu[s + 1])
        alone = {"q": r["q"][a:b], "k": r["k"][a:b], "w": r["w"][a:b],
                 "cu_seqlens": np.array([0, b - a], dtype=np.int32)}
        res = run_gpu(alone, wl.kpool, 32)
        np.testing.assert_array_equal(res["pool_ids"], packed["pool_ids"][a:b])
        np.testing.assert_array_equal(res["token_ids"], packed["token_ids"][a:b])
        n = res["scores"].shape[1]
        np.testing.assert_array_equal(res["scores"], packed["scores"][a:b, :n])


def test_repeat_runs_are_bitwise_identical():
    wl, r = _inputs("sq4096", 8, T=3000)
    a = run_gpu(r, wl.kpool, wl.budget)
    b = run_gpu(r, wl.kpool, wl.budget)
    for key in ("kp", "pool_ids", "token_ids", "scores"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)


def test_weight_doubling_doubles_scores_exactly():
    wl, r = _inputs("sq4096", 9, T=1000)
    a = run_gpu(r, wl.kpool, 100)
    r2 = dict(r)
    r2["w"] = (r["w"] * np.float32(2)).astype(np.float32)
    b = run_gpu(r2, wl.kpool, 100)
    np.testing.assert_array_equal(b["scores"], 2 * a["scores"])
    np.testing.assert_array_equal(b["pool_ids"], a["pool_ids"])


def test_head_permutation_changes_scores_only_by_rounding():
    # Permuting the heads of q and w together leaves the formula unchanged; on the GPU it
    # only reorders the fp32 head sum.  Both runs must pass every oracle rule, and their
    # scores differ by at most a few fp32 roundings of the head sum.
    wl, r = _inputs("sq4096", 11, T=1500, budget=200)
    a = run_gpu(r, wl.kpool, wl.budget)
    perm = np.random.default_rng(5).permutation(wl.H)
    assert (perm != np.arange(wl.H)).any()
    r2 = dict(r)
    r2["q"] = np.ascontiguousarray(r["q"][:, perm, :])
    r2["w"] = np.ascontiguousarray(r["w"][:, perm])
    b = run_gpu(r2, wl.kpool, wl.budget)
    for res, where in ((a, "heads in order"), (b, "heads permuted")):
        _full_check(wl, r, res, where=where)
    vis = np.isfinite(a["scores"])
    np.testing.assert_array_equal(vis, np.isfinite(b["scores"]))
    # (w >= 0 here, so the head sum has no cancellation: each ordering is within
    # H * 2^-24 of the exact sum, relative)
    av, bv = a["scores"][vis], b["scores"][vis]
    diff = np.abs(av - bv)
    assert (diff <= 2 * wl.H * 2.0 ** -24 * np.abs(av)).all(), diff.max()
    print(f"[heads] permuted heads: max score change {diff.max():.2e}", flush=True)


def test_zero_weights_select_by_index():
    wl, r = _inputs("sq4096", 0, T=3000, variant="w_zero")
    res = run_gpu(r, wl.kpool, wl.budget)
    for i in range(3000):
        m = min(wl.budget, i // 4 + 1)
        assert res["pool_ids"][i, :m].tolist() == list(range(m))
        assert np.all(res["pool_ids"][i, m:] == -1)


# ---------------------------------------------------------------------------
# The selection and expansion steps on their own
# ---------------------------------------------------------------------------

def _topk_rows(rng):
    rows = []
    for n in (0, 1, 3, 511, 512, 513, 1000, 4095, 4096, 4097, 20000, 131072):
        rows.append(rng.standard_normal(n).astype(np.float32))
    rows.append(np.zeros(131072, dtype=np.float32))                                   # all tied
    rows.append(rng.integers(-2, 3, 70000).astype(np.float32))                        # 5 values
    x = rng.standard_normal(9000).astype(np.float32)
    x[rng.random(9000) < 0.3] = 0.0
    x[rng.random(9000) < 0.3] = -0.0
    rows.append(x)                                                                    # +-0 ties
    y = np.round(rng.random(60000), 3).astype(np.float32)
    y[::7] = -np.inf
    y[5::11] = np.nan
    rows.append(y)                                                                    # inf, nan, ties
    z = rng.standard_normal(50000).astype(np.float32)
    z[1000:6000] = z.max() + 1.0                                                      # 5000 tied on top
    rows.append(z)
    for t in (700, 2500):                  # ties on top between the budget and the list cap:
        u = rng.standard_normal(65536).astype(np.float32)  # the cut starts past 32 shared bits
        u[rng.choice(65536, t, replace=False)] = u.max() + 1.0
        rows.append(u)
    v = (1.0 + rng.integers(0, 4096, 65536) * 2.0 ** -20).astype(np.float32)
    rows.append(v)                         # narrow range: bound and best key share ~20 bits
    ramp = np.arange(30000, dtype=np.float32)                                         # sorted input
    rows.append(ramp)
    rows.append(ramp[::-1].copy())
    return rows


@pytest.mark.parametrize("budget", [1, 7, 512, 1024, 1025, 2048])
def test_topk_standalone_matches_oracle_selection(budget):
    rng = np.random.default_rng(budget)
    rows = _topk_rows(rng)
    ld = max(len(x) for x in rows)
    ld = (ld + 3) // 4 * 4
    buf = np.full((len(rows), ld), np.nan, dtype=np.float32)   # junk past n_valid
    for i, x in enumerate(rows):
        buf[i, :len(x)] = x
    nv = np.array([len(x) for x in rows], dtype=np.int32)
    got = K.topk(torch.from_numpy(buf).cuda(), torch.from_numpy(nv).cuda(), budget)
    got = got.cpu().numpy()
    for i, x in enumerate(rows):
        want = oracle.select_row_full_sort(x, budget)
        assert np.array_equal(got[i], want), f"row {i} (n={len(x)})"


def test_topk_standalone_clamps_row_counts():
    # counts outside [0, ld] are clamped: negative -> nothing selected, beyond ld -> the row
    rng = np.random.default_rng(17)
    ld = 5000
    buf = rng.standard_normal((4, ld)).astype(np.float32)
    for budget in (7, 600, 2048):
        nv = np.array([-5, ld + 1000, 0, ld], dtype=np.int32)
        got = K.topk(torch.from_numpy(buf).cuda(), torch.from_numpy(nv).cuda(), budget).cpu().numpy()
        assert np.all(got[0] == -1) and np.all(got[2] == -1), budget
        for i in (1, 3):
            assert np.array_equal(got[i], oracle.select_row_full_sort(buf[i], budget)), (budget, i)


def test_expand_standalone_matches_oracle():
    rng = np.random.default_rng(3)
    for kpool in (1, 3, 4):
        cu = np.array([0, 5, 5, 900, 1000], dtype=np.int32)
        T = int(cu[-1])
        budget = 17
        ids = rng.integers(-1, 230, size=(T, budget)).astype(np.int32)
        got = K.expand(torch.from_numpy(ids).cuda(), cu, torch.from_numpy(cu).cuda(), kpool, budget, 0, T)
        got = got.cpu().numpy()
        _, t = oracle.row_positions(np.arange(T), cu)
        for i in range(T):
            assert np.array_equal(got[i], oracle.expand_row(ids[i], int(t[i]), kpool)), (kpool, i)
        # a sub-range lands at offset 0 of its own output
        sub = K.expand(torch.from_numpy(ids[10:20]).cuda(), cu, torch.from_numpy(cu).cuda(), kpool,
                       budget, 10, 20).cpu().numpy()
        np.testing.assert_array_equal(sub, got[10:20])


@pytest.mark.parametrize("kpool,budget,variant", [(4, 512, "w_zero"), (4, 512, "k_const"),
                                                  (1, 1000, "w_zero"), (2, 1024, "k_const"),
                                                  (1, 2048, "w_zero"), (1, 2048, "k_const")])
def test_long_rows_all_tied_take_the_exact_path(kpool, budget, variant):
    """Rows long enough for group pruning (>= 1024 groups at budgets up to 512, >= 2048
    up to 1024, >= 4096 up to 2048) whose scores are all equal (zero weights, or
    identical pooled keys): every group max ties with the bound, the candidate list
    overflows and the exact radix path must return the first `budget` pools in index
    order (ties go to the smaller pool index)."""
    T = 70000
    wl = synth.workload("sq4096", T=T, kpool=kpool, budget=budget, variant=variant)
    inp = synth.device_inputs(wl, 0)
    sel = K.Selector(inp["cu_seqlens"], kpool, budget, wl.H, wl.D)
    out = sel.run(inp["q"], inp["k"], inp["w"])
    ids = out["pool_ids"].cpu().numpy()
    m = np.minimum(budget, np.arange(T) // kpool + 1)
    col = np.arange(budget)[None, :]
    expect = np.where(col < m[:, None], col, -1).astype(np.int32)
    np.testing.assert_array_equal(ids, expect)
    # the long rows did go through group pruning's overflow (not only short rows)
    assert (T - 1) // kpool + 1 >= (16 if budget <= 512 else 32 if budget <= 1024 else 64) * 1024
