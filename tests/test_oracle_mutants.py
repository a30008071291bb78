"""Plant plausible mistakes in the oracle (on the CPU) and check the pins catch them.

Each mutant replaces one oracle step with a subtly wrong version (a dropped
term, a wrong sign, index or order, a transposed operand).  The pin battery
(hand-derived values, exact brute force, closed forms) must fail for every
one of them; the unmodified oracle must pass it.
"""
import json
import os

import numpy as np
import pytest

import exact_brute as brute
from oracle import kpool_oracle as ko
from pool_score_top_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _battery():
    """Return True iff every pin holds for the oracle as currently bound."""
    with open(os.path.join(GOLDEN, "pool_pins.json")) as f:
        for c in json.load(f)["cases"]:
            k = np.array([int(x, 16) for x in c["keys"]], dtype=np.uint16).reshape(-1, 1)
            kp = ko.pool_keys(k, np.array([0, len(k)]), c["kpool"])
            if kp[:, 0].tolist() != [int(x, 16) for x in c["pooled"]]:
                return False
    with open(os.path.join(GOLDEN, "select_pins.json")) as f:
        g = json.load(f)
    for c in g["select"]:
        if ko.select_row(np.array([float(x) for x in c["scores"]]), c["budget"]).tolist() != c["ids"]:
            return False
    for c in g["expand"]:
        if ko.expand_row(c["ids"], c["t"], c["kpool"]).tolist() != c["tokens"]:
            return False
    cases = [
        (40, 3, 16, 3, 5, [0, 7, 8, 23, 40], 2, ""),
        (33, 2, 4, 2, 3, [0, 33], 3, "w_neg"),
        (30, 4, 16, 4, 3, [0, 17, 30], 4, "k_ternary"),
    ]
    for T, H, D, kpool, budget, cu, seed, variant in cases:
        wl = synth.Workload("t", T, H, D, kpool, budget, 1.0, variant=variant)
        r = synth.rows(wl, seed, 0, T)
        cu = np.array(cu)
        ex = brute.run(r["q"].tolist(), r["k"].tolist(), r["w"].view(np.uint32).tolist(),
                       cu.tolist(), kpool, budget)
        got = ko.select(r["q"], r["k"], r["w"], cu, kpool, budget)
        kp_exact = np.array([[float(v) for v in row] for row in ex["kp"]])
        if not np.array_equal(ko.bf16_to_f32(got["kp"]).astype(np.float64), kp_exact):
            return False
        for i in range(T):
            exact = np.array([float(v) for v in ex["scores"][i]])
            n = len(exact)
            if not np.allclose(got["scores"][i, :n], exact, rtol=1e-12, atol=0):
                return False
            if not np.all(np.isneginf(got["scores"][i, n:])):
                return False
        if not np.array_equal(got["pool_ids"], np.array(ex["pool_ids"])):
            return False
        if not np.array_equal(got["token_ids"], np.array(ex["token_ids"])):
            return False
    return True


# --------------------------- mutant builders -------------------------------

def _pool_variant(divide="n_p", order=1, accum="f32", rounding="rne"):
    def pool_keys(k_bits, cu_seqlens, kpool):
        k = ko.bf16_to_f32(k_bits)
        D = k.shape[1]
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        cu_pools, _ = ko.count_pools(cu, kpool)
        out = np.zeros((int(cu_pools[-1]), D), dtype=np.uint16)
        for s in range(len(cu) - 1):
            start, L = int(cu[s]), int(cu[s + 1] - cu[s])
            for p in range((L + kpool - 1) // kpool):
                toks = list(range(start + p * kpool, start + min(L, (p + 1) * kpool)))[::order]
                if accum == "f32":
                    acc = np.zeros(D, np.float32)
                    for tk in toks:
                        acc = (acc + k[tk]).astype(np.float32)
                else:
                    acc = np.sum(k[toks].astype(np.float64), axis=0)
                n = {"n_p": len(toks), "kpool": kpool, "none": 1}[divide]
                m = (acc / n).astype(np.float32)
                if rounding == "rne":
                    out[cu_pools[s] + p] = ko.f32_to_bf16_rne(m)
                else:
                    out[cu_pools[s] + p] = (m.view(np.uint32) >> 16).astype(np.uint16)
        return out
    return pool_keys


def _scores_variant(relu=True, relu_after_w=False, use_scale=True, vis_shift=0,
                    base_zero=False, w_reversed=False, transpose_kp=False):
    def row_scores(q_rows_bits, w_rows, kp_bits, cu_pools, seq, t, kpool, scale=None, width=None):
        q = ko.bf16_to_f32(q_rows_bits).astype(np.float64)
        w = np.asarray(w_rows, np.float32).astype(np.float64)
        if w_reversed:
            w = w[:, ::-1]
        kp = ko.bf16_to_f32(kp_bits).astype(np.float64)
        r, H, D = q.shape
        sc = (1.0 / np.sqrt(D) if scale is None else scale) if use_scale else 1.0
        nv = np.asarray(t) // kpool + 1 + vis_shift
        if width is None:
            width = int(nv.max())
        out = np.full((r, width), -np.inf)
        for i in range(r):
            base = 0 if base_zero else int(cu_pools[seq[i]])
            n = max(0, min(int(nv[i]), width))
            keys = kp[base:base + n]
            if transpose_kp:
                keys = keys[:, ::-1]
            dots = q[i] @ keys.T
            if relu_after_w:
                out[i, :n] = np.maximum((w[i][:, None] * sc * dots), 0.0).sum(0)
            elif relu:
                out[i, :n] = w[i] @ np.maximum(sc * dots, 0.0)
            else:
                out[i, :n] = w[i] @ (sc * dots)
        return out
    return row_scores


def _select_variant(kind):
    def select_row(scores_row, budget):
        s = np.asarray(scores_row, np.float64)
        if kind != "signed_zero":
            s = s + 0.0
        isnan = np.isnan(s)
        s = np.where(isnan, -np.inf, s)
        idx = np.arange(len(s))
        if kind == "larger_index_first":
            order = np.lexsort((-idx, -s, isnan))
        elif kind == "ascending":
            order = np.lexsort((idx, s, isnan))
        elif kind == "signed_zero":
            sign = np.signbit(s).astype(np.int64)
            order = np.lexsort((idx, sign, -s, isnan))
        elif kind == "nan_first":
            order = np.lexsort((idx, -s, ~isnan))
        out = np.full(budget, -1, np.int32)
        out[:min(budget, len(s))] = order[:budget]
        return out
    return select_row


def _expand_variant(kind):
    def expand_row(ids, t, kpool):
        out = np.full(len(ids) * kpool, -1, np.int32)
        for b, p in enumerate(ids):
            if p < 0:
                continue
            for j in range(kpool):
                tok = p * kpool + j
                ok = {"strict": tok < t, "none": True, "by_pool_end": p * kpool + kpool - 1 <= t}[kind]
                if ok:
                    out[b * kpool + j] = tok
        return out
    return expand_row


MUTANTS = {
    "pool_divide_by_kpool": ("pool_keys", _pool_variant(divide="kpool")),
    "pool_sum_not_mean": ("pool_keys", _pool_variant(divide="none")),
    "pool_reversed_order": ("pool_keys", _pool_variant(order=-1)),
    "pool_fp64_accumulate": ("pool_keys", _pool_variant(accum="f64")),
    "pool_truncate_not_rne": ("pool_keys", _pool_variant(rounding="trunc")),
    "score_no_relu": ("row_scores", _scores_variant(relu=False)),
    "score_relu_after_weight": ("row_scores", _scores_variant(relu_after_w=True)),
    "score_no_scale": ("row_scores", _scores_variant(use_scale=False)),
    "score_visible_off_by_one_short": ("row_scores", _scores_variant(vis_shift=-1)),
    "score_visible_off_by_one_long": ("row_scores", _scores_variant(vis_shift=+1)),
    "score_wrong_sequence_base": ("row_scores", _scores_variant(base_zero=True)),
    "score_weights_reversed": ("row_scores", _scores_variant(w_reversed=True)),
    "score_key_dims_reversed": ("row_scores", _scores_variant(transpose_kp=True)),
    "select_larger_index_first": ("select_row", _select_variant("larger_index_first")),
    "select_ascending": ("select_row", _select_variant("ascending")),
    "select_signed_zero": ("select_row", _select_variant("signed_zero")),
    "select_nan_first": ("select_row", _select_variant("nan_first")),
    "expand_strict_filter": ("expand_row", _expand_variant("strict")),
    "expand_no_filter": ("expand_row", _expand_variant("none")),
    "expand_filter_by_pool_end": ("expand_row", _expand_variant("by_pool_end")),
}


def test_unmodified_oracle_passes_battery():
    assert _battery()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(ko, attr, fn)
    if attr == "select_row":
        monkeypatch.setattr(ko, "select_row_full_sort", fn)
    try:
        ok = _battery()
    except (ValueError, IndexError):
        ok = False
    assert not ok, f"mutant {name} survived the pins"


# --------------------------- gated pooling ---------------------------------

def _gated_battery():
    """True iff every pin of tests/test_oracle_gated.py holds for the bound oracle."""
    import test_oracle_gated as tg
    checks = [lambda c=c: tg.test_gated_hand_values(c) for c in tg.gated_cases()]
    checks += [lambda k=k: tg.test_equal_gates_give_the_exact_mean(k) for k in (1, 2, 3, 4, 5)]
    checks += [tg.test_common_shift_per_dim_changes_nothing, tg.test_dominant_slot_returns_that_key,
               tg.test_kpool_one_returns_the_keys]
    checks += [lambda k=k, s=s: tg.test_matches_high_precision_evaluation(k, s)
               for k, s in ((2, 0), (3, 1), (4, 2), (5, 3))]
    for c in checks:
        try:
            with np.errstate(all="ignore"):
                c()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            return False
    return True


def _gated_variant(axis_d=False, no_shift=False, ape_rev=False, ape_right=False, no_norm=False,
                   no_gate=False, no_ape=False, f32=False, via_f32=False, wrong_token=False,
                   softmin=False):
    def pool_keys_gated(k_bits, g_bits, ape, cu_seqlens, kpool, return_values=False):
        dt = np.float32 if f32 else np.float64
        k = ko.bf16_to_f32(k_bits).astype(dt)
        g = ko.bf16_to_f32(g_bits).astype(dt)
        a = np.asarray(ape, np.float32).astype(dt)
        D = k.shape[1]
        cu = np.asarray(cu_seqlens, np.int64)
        cu_pools, _ = ko.count_pools(cu, kpool)
        vals = np.zeros((int(cu_pools[-1]), D), dt)
        for s in range(len(cu) - 1):
            start, L = int(cu[s]), int(cu[s + 1] - cu[s])
            for p in range((L + kpool - 1) // kpool):
                t0 = start + p * kpool
                n = min(kpool, L - p * kpool)
                slots = np.arange(n)
                if ape_rev:
                    slots = kpool - 1 - slots
                if ape_right:
                    slots = kpool - n + slots
                z = (0 if no_gate else g[t0:t0 + n]) + (0 if no_ape else a[slots])
                z = np.broadcast_to(z, (n, D)).astype(dt)
                if softmin:
                    z = -z
                ax = 1 if axis_d else 0
                e = np.exp(z) if no_shift else np.exp(z - z.max(axis=ax, keepdims=True))
                wts = e if no_norm else e / e.sum(axis=ax, keepdims=True)
                kk = k[t0:t0 + n]
                if wrong_token:
                    kk = np.roll(kk, 1, axis=0)
                vals[int(cu_pools[s]) + p] = (wts * kk).sum(axis=0)
        if via_f32:
            bits = ko.f32_to_bf16_rne(vals.astype(np.float32))
        else:
            bits = ko.f64_to_bf16_rne(vals.astype(np.float64))
        return (bits, vals.astype(np.float64)) if return_values else bits
    return pool_keys_gated


GATED_MUTANTS = {
    "gated_softmax_over_dims": _gated_variant(axis_d=True),
    "gated_no_max_shift": _gated_variant(no_shift=True),
    "gated_embedding_slots_reversed": _gated_variant(ape_rev=True),
    "gated_embedding_right_aligned": _gated_variant(ape_right=True),
    "gated_not_normalised": _gated_variant(no_norm=True),
    "gated_gate_dropped": _gated_variant(no_gate=True),
    "gated_embedding_dropped": _gated_variant(no_ape=True),
    "gated_fp32_arithmetic": _gated_variant(f32=True),
    "gated_rounded_through_fp32": _gated_variant(via_f32=True),
    "gated_weights_on_wrong_token": _gated_variant(wrong_token=True),
    "gated_softmin": _gated_variant(softmin=True),
}


def test_unmodified_gated_oracle_passes_battery():
    assert _gated_battery()


@pytest.mark.parametrize("name", sorted(GATED_MUTANTS))
def test_gated_mutant_is_caught(name, monkeypatch):
    import oracle
    monkeypatch.setattr(ko, "pool_keys_gated", GATED_MUTANTS[name])
    monkeypatch.setattr(oracle, "pool_keys_gated", GATED_MUTANTS[name])
    assert not _gated_battery(), f"mutant {name} survived the pins"


# --------------------------- tail mode ---------------------------------------

def _tail_battery():
    """True iff every pin of tests/test_oracle_tail.py holds for the bound oracle."""
    import test_oracle_tail as tt
    checks = [lambda c=c: tt.test_tail_hand_rows(c) for c in tt.tail_cases()]
    checks += [lambda c=c: tt.test_tail_mode_matches_exact_brute_force(c) for c in tt.BRUTE_CASES]
    checks += [tt.test_multiple_of_kpool_is_unchanged_by_tail_mode,
               tt.test_tail_slots_closed_form_and_restriction_to_full_pools]
    for c in checks:
        try:
            c()
        except (AssertionError, ValueError, IndexError):
            return False
    return True


_orig_expand_row = ko.expand_row
_orig_count_pools = ko.count_pools
_orig_visible_pools = ko.visible_pools


def _tail_expand_variant(kind):
    def expand_row(ids, t, kpool, tail=None):
        if tail is None:
            return _orig_expand_row(ids, t, kpool)
        a, e = int(tail[0]), int(tail[1])
        if kind == "early":
            a -= 1
        base = _orig_expand_row(ids, t, kpool)
        tl = np.full(kpool - 1, -1, np.int32)
        for j in range(kpool - 1):
            tok = a + j
            ok = {"unfiltered": tok < e, "strict": tok < e and tok < t,
                  "early": tok < e and tok <= t, "front": tok < e and tok <= t}[kind]
            if ok:
                tl[j] = tok
        return np.concatenate([tl, base]) if kind == "front" else np.concatenate([base, tl])
    return expand_row


def _tail_count_ceil(cu_seqlens, kpool, tail=False):
    return _orig_count_pools(cu_seqlens, kpool, False)


def _tail_visibility_uncapped(t, kpool, npools=None):
    return _orig_visible_pools(t, kpool)


TAIL_MUTANTS = {
    "tail_unfiltered": ("expand_row", _tail_expand_variant("unfiltered")),
    "tail_strict_filter": ("expand_row", _tail_expand_variant("strict")),
    "tail_starts_one_early": ("expand_row", _tail_expand_variant("early")),
    "tail_before_the_pools": ("expand_row", _tail_expand_variant("front")),
    "tail_partial_pool_kept": ("count_pools", _tail_count_ceil),
    "tail_visibility_not_capped": ("visible_pools", _tail_visibility_uncapped),
}


def test_unmodified_tail_oracle_passes_battery():
    assert _tail_battery()


@pytest.mark.parametrize("name", sorted(TAIL_MUTANTS))
def test_tail_mutant_is_caught(name, monkeypatch):
    import oracle
    attr, fn = TAIL_MUTANTS[name]
    monkeypatch.setattr(ko, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    assert not _tail_battery(), f"mutant {name} survived the pins"
