"""Pins for the oracle's gated k-pool compression (no GPU).

The pages name the GLM-5.3 indexer's k-pool compression gate and slot
embedding (Atlas inference docs, glm5next_dsa/tp.rs, the indexer tensors of
the shard plan) and say the op takes gate scores as an input (Megatron-LM PR
#8299, "Mechanism"), but print no formula: the formula in
oracle.pool_keys_gated is a reading, and against the pages' own operator its
parity is unpinned.  These pins fix that reading with things other than the
oracle itself:

  * hand-derived values (tests/golden/gated_pins.json), including keys just
    above and below a bf16 rounding midpoint (one rounding from the exact
    value, not two through fp32), a dominant slot behind a large common
    shift, and partial pools;
  * the fp64 -> bf16 rounding against an exact-rational rounding;
  * equal gates and embeddings give the exact mean (exact rationals);
  * adding the same constant to every slot of a dim (in the embedding)
    changes nothing, also for shifts of +-1000;
  * a dominant slot (by embedding, or by gate score) returns that token's key;
  * kpool = 1 returns the keys;
  * a high-precision evaluation (Python's decimal module at 50 digits, its own
    exp) of the same reading agrees with the fp64 values to 1e-13 and gives the
    same bf16 bits.
test_oracle_mutants.py plants mistakes in this function and checks that these
pins catch every one.
"""
import json
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import exact_brute as brute
import oracle
from pool_score_top_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(xs):
    return np.array([int(x, 16) for x in xs], dtype=np.uint16)


def _bf16_bits_of_fraction(x: Fraction) -> int:
    """Exact RNE of a rational to bf16, as a bit pattern (finite, normal or subnormal)."""
    v = brute.bf16(x)
    return int(np.float32(float(v)).view(np.uint32) >> np.uint32(16)) if v != 0 else (
        0x8000 if x < 0 else 0)


def gated_cases():
    with open(os.path.join(GOLDEN, "gated_pins.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", gated_cases(), ids=lambda c: c["name"])
def test_gated_hand_values(case):
    k = _bits(case["keys"]).reshape(-1, 1)
    g = _bits(case["gates"]).reshape(-1, 1)
    ape = np.array(case["ape"], dtype=np.float32).reshape(-1, 1)
    got = oracle.pool_keys_gated(k, g, ape, np.array([0, len(k)]), case["kpool"])
    assert got[:, 0].tolist() == _bits(case["pooled"]).tolist(), case["why"]


def test_f64_to_bf16_matches_exact_rounding():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(3000),
                        rng.standard_normal(500) * 1e-39,          # bf16 subnormal range
                        rng.standard_normal(500) * 1e30])
    # values just around midpoints: a bf16 value + half its ulp +- a tiny amount
    base = oracle.bf16_to_f32(rng.integers(0x0080, 0x7F00, 400).astype(np.uint16)).astype(np.float64)
    ulp = np.ldexp(1.0, np.frexp(base)[1] - 8)
    x = np.concatenate([x, base + ulp / 2, base + ulp / 2 + ulp * 2.0 ** -30,
                        base + ulp / 2 - ulp * 2.0 ** -30, -(base + ulp / 2)])
    got = oracle.f64_to_bf16_rne(x)
    for xi, gi in zip(x, got):
        assert int(gi) == _bf16_bits_of_fraction(Fraction(float(xi))), xi


def _inputs(T, D, kpool, seed, cu):
    wl = synth.workload("tiny_gated", T=T, D=D, kpool=kpool)
    r = synth.host_inputs(wl, seed)
    r["cu_seqlens"] = np.asarray(cu)
    return r


@pytest.mark.parametrize("kpool", [1, 2, 3, 4, 5])
def test_equal_gates_give_the_exact_mean(kpool):
    """g constant and ape constant: every weight is 1/n, the key is the exact mean."""
    r = _inputs(41, 8, kpool, kpool, [0, 1, 17, 17, 41])
    g = np.full_like(r["g"], 0x4040)                   # 3.0 everywhere
    ape = np.full((kpool, 8), -0.5, dtype=np.float32)
    got = oracle.pool_keys_gated(r["k"], g, ape, r["cu_seqlens"], kpool)
    cu = r["cu_seqlens"]
    row = 0
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        for p0 in range(a, b, kpool):
            toks = range(p0, min(b, p0 + kpool))
            for d in range(8):
                mean = sum(brute.decode_bf16(r["k"][t, d]) for t in toks) / len(toks)
                # the fp64 weights 1/n are inexact for n = 3, 5: a mean within fp64's
                # error of a bf16 rounding midpoint may go to either neighbour
                eps = abs(mean) * Fraction(1, 2 ** 50)
                allowed = {_bf16_bits_of_fraction(mean - eps), _bf16_bits_of_fraction(mean + eps)}
                assert int(got[row, d]) in allowed, (s, p0, d)
                if len(toks) in (1, 2, 4):              # weights exact: one answer
                    assert int(got[row, d]) == _bf16_bits_of_fraction(mean), (s, p0, d)
            row += 1
    assert row == len(got)


def test_common_shift_per_dim_changes_nothing():
    """Adding c_d to ape[j, d] for every slot j leaves every softmax unchanged.  The
    embeddings are multiples of 2^-6 below 2^4 and the shifts integers up to 1000, so the
    shifted embeddings are exact in fp32 and the identity is exact."""
    kpool, D = 4, 16
    r = _inputs(70, D, kpool, 3, [0, 3, 30, 70])
    ape = (np.round(r["ape"] * 64.0) / 64.0).astype(np.float32)  # multiples of 2^-6
    base = oracle.pool_keys_gated(r["k"], r["g"], ape, r["cu_seqlens"], kpool)
    rng = np.random.default_rng(4)
    for shifts in (rng.integers(-20, 21, D), np.full(D, 1000), np.full(D, -1000),
                   np.where(np.arange(D) % 2, 1000, -1000)):
        shifted = (ape + shifts.astype(np.float32)[None, :]).astype(np.float32)
        assert np.array_equal(shifted.astype(np.float64) - shifts, ape.astype(np.float64))
        got = oracle.pool_keys_gated(r["k"], r["g"], shifted, r["cu_seqlens"], kpool)
        np.testing.assert_array_equal(got, base)


def test_dominant_slot_returns_that_key():
    kpool, D = 4, 8
    cu = [0, 13, 14, 30]                                # partial pools of 1 and 2 tokens
    r = _inputs(30, D, kpool, 6, cu)
    k32 = oracle.bf16_to_f32(r["k"])
    cu_pools, _ = oracle.count_pools(cu, kpool)
    for j in range(kpool):
        ape = r["ape"].copy()
        ape[j] += np.float32(300.0)                     # e^-300 for every other slot
        got = oracle.bf16_to_f32(oracle.pool_keys_gated(r["k"], r["g"], ape, cu, kpool))
        for s in range(len(cu) - 1):
            a, b = cu[s], cu[s + 1]
            for p, p0 in enumerate(range(a, b, kpool)):
                if p0 + j < b:                          # slot j exists in this pool
                    np.testing.assert_array_equal(got[cu_pools[s] + p], k32[p0 + j])
    # dominance by gate score: one token per pool gets gate +64 (bf16 0x4280), others 0
    g = np.zeros_like(r["g"])
    pick = []
    rng = np.random.default_rng(7)
    for s in range(len(cu) - 1):
        for p0 in range(cu[s], cu[s + 1], kpool):
            t = int(rng.integers(p0, min(cu[s + 1], p0 + kpool)))
            g[t] = 0x4280
            pick.append(t)
    ape = np.zeros((kpool, D), dtype=np.float32)
    got = oracle.bf16_to_f32(oracle.pool_keys_gated(r["k"], g, ape, cu, kpool))
    np.testing.assert_array_equal(got, k32[pick])


def test_kpool_one_returns_the_keys():
    r = _inputs(50, 16, 1, 8, [0, 20, 50])
    got = oracle.pool_keys_gated(r["k"], r["g"], r["ape"], r["cu_seqlens"], 1)
    np.testing.assert_array_equal(got, r["k"])


def _decimal_reference(k_bits, g_bits, ape, cu, kpool):
    """The same reading evaluated in 50-digit decimal arithmetic (its own exp)."""
    getcontext().prec = 50
    dec = lambda f: Decimal(f.numerator) / Decimal(f.denominator)  # noqa: E731
    D = k_bits.shape[1]
    out = []
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        for p0 in range(a, b, kpool):
            toks = list(range(p0, min(b, p0 + kpool)))
            row = []
            for d in range(D):
                z = [dec(brute.decode_bf16(g_bits[t, d]) + brute.decode_f32(
                    int(np.float32(ape[j, d]).view(np.uint32)))) for j, t in enumerate(toks)]
                m = max(z)
                e = [(zi - m).exp() for zi in z]
                num = sum(ei * dec(brute.decode_bf16(k_bits[t, d])) for ei, t in zip(e, toks))
                row.append(num / sum(e))
            out.append(row)
    return out


@pytest.mark.parametrize("kpool,seed", [(2, 0), (3, 1), (4, 2), (5, 3)])
def test_matches_high_precision_evaluation(kpool, seed):
    cu = [0, 9, 9, 22]
    r = _inputs(22, 6, kpool, seed, cu)
    bits, vals = oracle.pool_keys_gated(r["k"], r["g"], r["ape"], cu, kpool, return_values=True)
    ref = _decimal_reference(r["k"], r["g"], r["ape"], cu, kpool)
    assert len(ref) == len(vals)
    for i, row in enumerate(ref):
        for d, x in enumerate(row):
            xf = float(x)
            assert abs(vals[i, d] - xf) <= 1e-13 * abs(xf) + 1e-300, (i, d)
            exact_bits = _bf16_bits_of_fraction(Fraction(x))
            assert int(bits[i, d]) == exact_bits, (i, d)
