"""Pins for the oracle's tail mode (no GPU).

"Tail append" is named on the pages (Megatron-LM PR #8299, "Change": pool
expansion, tail append and mask filtering run on the gathered selection) but
never defined.  The reading (oracle.count_pools / expand_row / select, tail=True):
pools are the full pools of each sequence (Atlas tp.rs module doc writes the pool
count as seq / kpool), and the L mod kpool tokens after them, the tail, are
appended to every row's expanded tokens and then filtered causally like them.
Parity against the pages' own operator is therefore unpinned; these pin the
reading:

  * hand-worked rows (tests/golden/tail_pins.json);
  * an exact-rational brute force of the whole path in tail mode on tiny packed
    inputs (pools, scores, ids, tokens);
  * a sequence whose length is a multiple of kpool is unchanged by tail mode
    (the tail slots are -1);
  * the tail slots of every row follow their closed form;
  * tail-mode ids are the selection over the default mode's scores restricted
    to the full pools (the full pools' keys are the same in both modes).
"""
import json
import os

import numpy as np
import pytest

import exact_brute as brute
import oracle
from pool_score_top_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tail_cases():
    with open(os.path.join(GOLDEN, "tail_pins.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", tail_cases(), ids=lambda c: f"L{c['L']}_k{c['kpool']}_t{c['t']}")
def test_tail_hand_rows(case):
    L, kp = case["L"], case["kpool"]
    got = oracle.expand_row(case["ids"], case["t"], kp, (L // kp * kp, L))
    assert got.tolist() == case["tokens"], case["why"]


BRUTE_CASES = [
    # T, H, D, kpool, budget, cu_seqlens, seed, variant
    (37, 3, 16, 4, 3, [0, 3, 3, 14, 37], 1, ""),
    (30, 2, 4, 3, 4, [0, 1, 2, 17, 30], 2, "w_neg"),
    (26, 4, 16, 5, 2, [0, 26], 3, "k_ternary"),
    (20, 2, 4, 1, 3, [0, 9, 20], 4, ""),
]


@pytest.mark.parametrize("case", BRUTE_CASES, ids=lambda c: f"T{c[0]}_k{c[3]}")
def test_tail_mode_matches_exact_brute_force(case):
    T, H, D, kpool, budget, cu, seed, variant = case
    wl = synth.Workload("t", T, H, D, kpool, budget, 1.0, variant=variant)
    r = synth.rows(wl, seed, 0, T)
    cu = np.array(cu)
    ex = brute.run(r["q"].tolist(), r["k"].tolist(), r["w"].view(np.uint32).tolist(), cu.tolist(),
                   kpool, budget, tail=True)
    got = oracle.select(r["q"], r["k"], r["w"], cu, kpool, budget, tail=True)
    kp_exact = np.array([[float(v) for v in row] for row in ex["kp"]]).reshape(-1, D)
    np.testing.assert_array_equal(oracle.bf16_to_f32(got["kp"]).astype(np.float64), kp_exact)
    for i in range(T):
        exact = np.array([float(v) for v in ex["scores"][i]])
        n = len(exact)
        np.testing.assert_allclose(got["scores"][i, :n], exact, rtol=1e-12, atol=0)
        assert np.all(np.isneginf(got["scores"][i, n:]))
    np.testing.assert_array_equal(got["pool_ids"], np.array(ex["pool_ids"]).reshape(T, budget))
    np.testing.assert_array_equal(got["token_ids"], np.array(ex["token_ids"]).reshape(T, -1))


def test_multiple_of_kpool_is_unchanged_by_tail_mode():
    wl = synth.workload("tiny", T=64)
    r = synth.host_inputs(wl, 5)
    cu = np.array([0, 16, 16, 40, 64])                 # every length a multiple of 4
    a = oracle.select(r["q"], r["k"], r["w"], cu, 4, 4)
    b = oracle.select(r["q"], r["k"], r["w"], cu, 4, 4, tail=True)
    np.testing.assert_array_equal(a["kp"], b["kp"])
    np.testing.assert_array_equal(a["pool_ids"], b["pool_ids"])
    np.testing.assert_array_equal(b["token_ids"][:, :16], a["token_ids"])
    assert np.all(b["token_ids"][:, 16:] == -1)


def test_tail_slots_closed_form_and_restriction_to_full_pools():
    wl = synth.workload("tiny", T=90)
    r = synth.host_inputs(wl, 6)
    cu = np.array([0, 2, 2, 27, 61, 90])
    kpool, budget = 4, 3
    dflt = oracle.select(r["q"], r["k"], r["w"], cu, kpool, budget)
    tl = oracle.select(r["q"], r["k"], r["w"], cu, kpool, budget, tail=True)
    seq, t = oracle.row_positions(np.arange(90), cu)
    for i in range(90):
        L = int(cu[seq[i] + 1] - cu[seq[i]])
        nfull = L // kpool
        a = nfull * kpool
        want_tail = [a + j if a + j < L and a + j <= t[i] else -1 for j in range(kpool - 1)]
        assert tl["token_ids"][i, budget * kpool:].tolist() == want_tail, i
        # the same selection as over the default scores of the full pools only
        nv = min(int(t[i]) // kpool + 1, nfull)
        want_ids = oracle.select_row(dflt["scores"][i, :nv], budget)
        np.testing.assert_array_equal(tl["pool_ids"][i], want_ids)
        np.testing.assert_array_equal(tl["scores"][i, :nv], dflt["scores"][i, :nv])
        assert np.all(np.isneginf(tl["scores"][i, nv:]))
