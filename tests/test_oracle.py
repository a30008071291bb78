"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself: hand-derived values
(tests/golden), an exact-rational brute force, closed forms, invariants and
a library routine for the bf16 rounding.  test_oracle_mutants.py then plants
plausible mistakes in the oracle and checks that these pins catch them.
"""
import json
import os

import numpy as np
import pytest
import torch

import exact_brute as brute
import oracle
from pool_score_top_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hex_bits(xs):
    return np.array([int(x, 16) for x in xs], dtype=np.uint16)


# ---------------------------------------------------------------------------
# bf16 rounding
# ---------------------------------------------------------------------------

def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(1)
    with np.errstate(over="ignore"):  # draws past the fp32 range become +-inf, on purpose
        x = np.concatenate([
            rng.standard_normal(200000).astype(np.float32),
            (rng.standard_normal(20000) * 1e-38).astype(np.float32),   # subnormals
            (rng.standard_normal(20000) * 3e38).astype(np.float32),    # near overflow
            np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 1.0 + 2**-8, 1.0 + 3 * 2**-8],
                     dtype=np.float32),
        ])
    # every dropped-half pattern around a tie
    base = np.uint32(0x3F810000)
    x = np.concatenate([x, (base + np.arange(0, 0x10000, 7, dtype=np.uint32)).view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.f32_to_bf16_rne(x), ref)


def test_bf16_roundtrip_exact():
    bits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_to_f32(bits)
    finite = np.isfinite(f)
    np.testing.assert_array_equal(oracle.f32_to_bf16_rne(f[finite]), bits[finite])


# ---------------------------------------------------------------------------
# O1 pooling
# ---------------------------------------------------------------------------

def _pool_cases():
    with open(os.path.join(GOLDEN, "pool_pins.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _pool_cases(), ids=lambda c: c["name"])
def test_pool_hand_values(case):
    k = _hex_bits(case["keys"]).reshape(-1, 1)
    cu = np.array([0, len(k)], dtype=np.int32)
    kp = oracle.pool_keys(k, cu, case["kpool"])
    np.testing.assert_array_equal(kp[:, 0], _hex_bits(case["pooled"]))


def test_pool_closed_forms():
    rng = np.random.default_rng(2)
    T, D = 37, 8
    k = oracle.f32_to_bf16_rne(rng.standard_normal((T, D)).astype(np.float32))
    cu = np.array([0, 9, 9, 37], dtype=np.int32)          # includes an empty sequence
    # kpool = 1: the pooled keys are the keys
    np.testing.assert_array_equal(oracle.pool_keys(k, cu, 1), k)
    # partial last pools of one token are that token
    kp = oracle.pool_keys(k, cu, 4)
    cu_pools, maxp = oracle.count_pools(cu, 4)
    assert list(cu_pools) == [0, 3, 3, 10] and maxp == 7
    np.testing.assert_array_equal(kp[2], k[8])     # seq 0: L=9 -> pools of 4, 4, 1 tokens
    kp = oracle.pool_keys(k, cu, 3)
    cu_pools, maxp = oracle.count_pools(cu, 3)
    assert list(cu_pools) == [0, 3, 3, 13] and maxp == 10
    np.testing.assert_array_equal(kp[12], k[36])   # seq 2: L=28 -> 9 pools of 3, one of 1
    # constant keys pool to themselves for every pool size
    c = np.full((T, D), 0x3F33, dtype=np.uint16)
    for kp_ in (1, 2, 3, 4, 5):
        np.testing.assert_array_equal(oracle.pool_keys(c, cu, kp_), 0x3F33)


# ---------------------------------------------------------------------------
# Exact brute force (whole path on tiny inputs)
# ---------------------------------------------------------------------------

def _brute_case(T, H, D, kpool, budget, cu, seed, variant=""):
    wl = synth.Workload("t", T, H, D, kpool, budget, 1.0, variant=variant)
    r = synth.rows(wl, seed, 0, T)
    return r["q"], r["k"], r["w"], np.asarray(cu, dtype=np.int32)


BRUTE_CASES = [
    # T, H, D, kpool, budget, cu_seqlens, seed, variant
    (64, 4, 16, 4, 4, [0, 64], 0, ""),          # the tiny workload, seed 0
    (64, 4, 16, 4, 4, [0, 64], 1, ""),
    (40, 3, 16, 3, 5, [0, 7, 8, 23, 40], 2, ""),  # packed, ragged, partial pools
    (33, 2, 4, 2, 3, [0, 33], 3, "w_neg"),       # negative weights
    (30, 4, 16, 4, 3, [0, 17, 30], 4, "k_ternary"),  # duplicated pooled keys -> exact ties
    (24, 4, 16, 4, 4, [0, 24], 5, "w_zero"),     # all scores zero
    (20, 2, 9, 1, 6, [0, 20], 6, ""),            # kpool 1 (per-token indexer)
]


@pytest.mark.parametrize("case", BRUTE_CASES, ids=lambda c: f"T{c[0]}H{c[1]}D{c[2]}k{c[3]}b{c[4]}s{c[6]}{c[7]}")
def test_oracle_matches_exact_brute_force(case):
    T, H, D, kpool, budget, cu, seed, variant = case
    q, k, w, cu = _brute_case(*case)
    ex = brute.run(q.tolist(), k.tolist(), w.view(np.uint32).tolist(), cu.tolist(), kpool, budget)
    got = oracle.select(q, k, w, cu, kpool, budget)
    # pooled keys: bit-exact
    kp_exact = np.array([[float(v) for v in row] for row in ex["kp"]], dtype=np.float64)
    np.testing.assert_array_equal(oracle.bf16_to_f32(got["kp"]).astype(np.float64), kp_exact)
    # scores: fp64 within 1e-12 relative of the exact rational value; masked = -inf
    _, t = oracle.row_positions(np.arange(T), cu)
    for i in range(T):
        n = t[i] // kpool + 1
        exact = np.array([float(v) for v in ex["scores"][i]])
        assert len(exact) == n
        np.testing.assert_allclose(got["scores"][i, :n], exact, rtol=1e-12, atol=1e-300)
        assert np.all(np.isneginf(got["scores"][i, n:]))
    np.testing.assert_array_equal(got["pool_ids"], np.array(ex["pool_ids"], dtype=np.int32))
    np.testing.assert_array_equal(got["token_ids"], np.array(ex["token_ids"], dtype=np.int32))


# ---------------------------------------------------------------------------
# Closed forms and invariants of the score
# ---------------------------------------------------------------------------

def test_score_closed_form_one_hot():
    """One nonzero weight and one nonzero dim: S = w * max(0, scale * q_d * kp_d)."""
    H, D, kpool = 4, 16, 2
    T = 12
    q = np.zeros((T, H, D), dtype=np.float32)
    k = np.zeros((T, D), dtype=np.float32)
    w = np.zeros((T, H), dtype=np.float32)
    rng = np.random.default_rng(7)
    qv = rng.integers(-4, 5, size=T).astype(np.float32)
    kv = rng.integers(-4, 5, size=T).astype(np.float32)
    q[:, 2, 5] = qv
    k[:, 5] = kv
    w[:, 2] = 0.75
    cu = np.array([0, T], dtype=np.int32)
    out = oracle.select(oracle.f32_to_bf16_rne(q), oracle.f32_to_bf16_rne(k), w, cu, kpool, 3)
    kp = (kv[0::2] + kv[1::2]) / 2.0
    for i in range(T):
        for p in range(i // kpool + 1):
            want = 0.75 * max(0.0, 0.25 * qv[i] * kp[p])
            assert out["scores"][i, p] == want


def test_score_invariants_heads_and_weight_scaling():
    wl = synth.workload("tiny")
    r = synth.host_inputs(wl, 3)
    base = oracle.select(r["q"], r["k"], r["w"], r["cu_seqlens"], wl.kpool, wl.budget)
    perm = np.array([2, 0, 3, 1])
    pq = oracle.select(r["q"][:, perm], r["k"], r["w"][:, perm], r["cu_seqlens"], wl.kpool, wl.budget)
    np.testing.assert_allclose(pq["scores"], base["scores"], rtol=1e-14)
    np.testing.assert_array_equal(pq["pool_ids"], base["pool_ids"])
    w2 = (r["w"] * np.float32(2)).astype(np.float32)
    d2 = oracle.select(r["q"], r["k"], w2, r["cu_seqlens"], wl.kpool, wl.budget)
    np.testing.assert_array_equal(d2["scores"], 2 * base["scores"])
    np.testing.assert_array_equal(d2["pool_ids"], base["pool_ids"])


def test_masking_closed_form():
    wl = synth.workload("tiny")
    r = synth.host_inputs(wl, 0)
    out = oracle.select(r["q"], r["k"], r["w"], r["cu_seqlens"], 4, 16)
    for i in range(wl.T):
        nv = i // 4 + 1
        assert np.all(np.isfinite(out["scores"][i, :nv]))
        assert np.all(np.isneginf(out["scores"][i, nv:]))
        ids = out["pool_ids"][i]
        assert sorted(ids[ids >= 0].tolist()) == list(range(nv))   # budget 16 >= |V|: all visible
        assert np.all(ids[nv:] == -1)


# ---------------------------------------------------------------------------
# O3 selection
# ---------------------------------------------------------------------------

def _select_cases():
    with open(os.path.join(GOLDEN, "select_pins.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("i", range(5))
def test_select_hand_values(i):
    c = _select_cases()["select"][i]
    s = np.array([float(x) for x in c["scores"]])
    assert oracle.select_row(s, c["budget"]).tolist() == c["ids"]
    assert oracle.select_row_full_sort(s, c["budget"]).tolist() == c["ids"]


@pytest.mark.parametrize("i", range(3))
def test_expand_hand_values(i):
    c = _select_cases()["expand"][i]
    assert oracle.expand_row(c["ids"], c["t"], c["kpool"]).tolist() == c["tokens"]


def test_select_partition_path_equals_full_sort():
    rng = np.random.default_rng(11)
    for trial in range(60):
        n = int(rng.integers(1, 5000))
        budget = int(rng.integers(1, 700))
        kind = trial % 3
        if kind == 0:
            s = rng.standard_normal(n)
        elif kind == 1:
            s = rng.integers(-3, 4, size=n).astype(np.float64)   # heavy ties
        else:
            s = np.round(rng.random(n), 2) * rng.choice([1.0, -1.0], size=n)
            s[rng.random(n) < 0.1] = -0.0
        a = oracle.select_row(s, budget)
        b = oracle.select_row_full_sort(s, budget)
        np.testing.assert_array_equal(a, b)


def test_select_brute_permutation_property():
    """The selection is the first `budget` of the (score desc, index asc) order."""
    rng = np.random.default_rng(12)
    for _ in range(200):
        n = int(rng.integers(1, 12))
        s = rng.integers(-2, 3, size=n).astype(np.float64)
        budget = int(rng.integers(1, 14))
        want = sorted(range(n), key=lambda p: (-s[p], p))[:budget]
        want = want + [-1] * (budget - len(want))
        assert oracle.select_row(s, budget).tolist() == want


def test_select_zero_weights_is_the_tiebreak_alone():
    wl = synth.workload("sq4096", T=300, variant="w_zero")
    r = synth.host_inputs(wl, 0)
    out = oracle.select(r["q"], r["k"], r["w"], r["cu_seqlens"], 4, 16)
    for i in range(300):
        nv = i // 4 + 1
        m = min(16, nv)
        assert out["pool_ids"][i, :m].tolist() == list(range(m))


# ---------------------------------------------------------------------------
# O4 expansion, whole-path properties
# ---------------------------------------------------------------------------

def test_expand_count_closed_form():
    rng = np.random.default_rng(5)
    for _ in range(300):
        kpool = int(rng.integers(1, 6))
        t = int(rng.integers(0, 60))
        nv = t // kpool + 1
        budget = int(rng.integers(1, 10))
        sel = rng.permutation(nv)[:budget]
        ids = np.full(budget, -1)
        ids[:len(sel)] = sel
        tok = oracle.expand_row(ids, t, kpool)
        last = t // kpool
        full = sum(1 for p in sel if p < last)
        want = kpool * full + ((t % kpool) + 1) * int(last in sel)
        assert int((tok >= 0).sum()) == want
        assert np.all(tok[tok >= 0] <= t)


def test_row_split_reassembles_and_thd_packing_invariance():
    wl = synth.workload("tiny", T=96)
    r = synth.rows(wl, 9, 0, 96)
    cu = np.array([0, 30, 31, 96], dtype=np.int32)
    full = oracle.select(r["q"], r["k"], r["w"], cu, 4, 4)
    parts = [oracle.select(r["q"], r["k"], r["w"], cu, 4, 4, q_lo=a, q_hi=b)
             for a, b in [(0, 13), (13, 13), (13, 64), (64, 96)]]
    for key in ("pool_ids", "token_ids", "scores"):
        np.testing.assert_array_equal(np.concatenate([p[key] for p in parts]), full[key])
    # sequence 2 alone equals sequence 2 inside the pack
    alone = oracle.select(r["q"][31:], r["k"][31:], r["w"][31:], np.array([0, 65]), 4, 4)
    np.testing.assert_array_equal(alone["pool_ids"], full["pool_ids"][31:])
    np.testing.assert_array_equal(alone["token_ids"], full["token_ids"][31:])
    np.testing.assert_array_equal(alone["scores"][:, :17], full["scores"][31:, :17])


def test_selection_rows_are_unique_causal_and_ordered():
    wl = synth.workload("sq4096", T=700)
    r = synth.host_inputs(wl, 0)
    out = oracle.select(r["q"], r["k"], r["w"], r["cu_seqlens"], 4, 64)
    for i in range(700):
        ids = out["pool_ids"][i]
        v = ids[ids >= 0]
        assert len(set(v.tolist())) == len(v)
        assert np.all(v <= i // 4)
        s = out["scores"][i, v]
        for a, b, pa, pb in zip(s[:-1], s[1:], v[:-1], v[1:]):
            assert a > b or (a == b and pa < pb)
        # nothing unselected beats the cutoff
        nv = i // 4 + 1
        if len(v) == 64:
            rest = np.setdiff1d(np.arange(nv), v)
            if len(rest):
                assert out["scores"][i, rest].max() <= s[-1]
