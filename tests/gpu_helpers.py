"""Shared helpers for the GPU parity tests (comparison rules and runners).

Comparison rules (GPU vs the fp64 CPU oracle):
  * pooled keys: bit-identical.
  * scores: every visible (row, pool) within |g - o| <= ATOL + RTOL*|o|;
    masked entries exactly -inf.
  * selection vs its own scores: the GPU ids are exactly the first `budget`
    pools of the GPU's fp32 scores ordered by (score desc, index asc), -0 == +0,
    -1 padded (checked here with a plain lexsort, a property of the output).
  * selection vs the oracle: the id sets may differ only in pools whose
    oracle score lies within tolerance of the row's cutoff, and the GPU order
    may only swap pools whose oracle scores are within tolerance.
  * token ids: equal to the oracle's where the pool ids are, and the expansion
    rule holds on every row.
"""
import numpy as np
import torch

import oracle
from pool_score_top_amd import kpool as K
from pool_score_top_amd import synth

RTOL = 1e-3
ATOL = 1e-4


def tol(o):
    return ATOL + RTOL * np.abs(o)


def device_tensors(inputs, device="cuda"):
    q = torch.from_numpy(inputs["q"].view(np.int16)).to(device)
    k = torch.from_numpy(inputs["k"].view(np.int16)).to(device)
    w = torch.from_numpy(inputs["w"]).to(device)
    return q, k, w


def run_gpu(inputs, kpool, budget, q_lo=0, q_hi=None, want_scores=True, workspace_cap=None,
            overlap=True):
    cu = np.asarray(inputs["cu_seqlens"], dtype=np.int32)
    q, k, w = device_tensors(inputs)
    H, D = inputs["q"].shape[1:]
    sel = K.Selector(cu, kpool, budget, H, D, q_lo=q_lo, q_hi=q_hi, workspace_cap=workspace_cap,
                     overlap=overlap)
    scores = None
    if want_scores:
        scores = torch.empty((sel.q_hi - sel.q_lo, sel.max_pools), dtype=torch.float32, device="cuda")
    out = sel.run(q, k, w, scores_out=scores)
    torch.cuda.synchronize()
    res = {
        "kp": out["kp"].cpu().numpy().view(np.uint16),
        "pool_ids": out["pool_ids"].cpu().numpy(),
        "token_ids": out["token_ids"].cpu().numpy(),
        "scores": None if scores is None else scores.cpu().numpy(),
        "max_pools": sel.max_pools,
    }
    return res


def lexsort_first(scores_f32, budget):
    """First `budget` indices of the (score desc, index asc) order of fp32 scores."""
    s = np.asarray(scores_f32, dtype=np.float64) + 0.0
    isnan = np.isnan(s)
    s = np.where(isnan, -np.inf, s)
    idx = np.arange(len(s))
    order = np.lexsort((idx, -s, isnan))[:budget]
    out = np.full(budget, -1, dtype=np.int32)
    out[:len(order)] = order
    return out


def check_scores(g, o, nvis, where="", bound=None):
    """g: fp32 [rows, width] GPU scores, o: fp64 oracle scores, nvis: visible per row.

    Gate: |g - o| <= ATOL + RTOL*|o| on every visible pool, -inf exactly where masked.
    With `bound` (fp64 [rows, width], see fp32_error_bound) every visible score must
    also lie within the error bound of the fp32 arithmetic, which is about a hundred
    times tighter than the gate, so an accuracy regression cannot hide under it.
    Returns the error figures (max abs, max relative, max err/tol, max err/bound)."""
    st = {"pairs": 0, "max_abs": 0.0, "max_rel": 0.0, "max_err_over_tol": 0.0,
          "max_err_over_bound": 0.0}
    for r in range(len(nvis)):
        n = int(nvis[r])
        d = np.abs(g[r, :n].astype(np.float64) - o[r, :n])
        bad = d > tol(o[r, :n])
        assert not bad.any(), (f"{where} row {r}: {bad.sum()} scores out of tolerance, "
                               f"max err {d.max():.3e}")
        assert np.all(np.isneginf(g[r, n:])), f"{where} row {r}: masked scores not -inf"
        if n == 0:
            continue
        st["pairs"] += n
        st["max_abs"] = max(st["max_abs"], float(d.max()))
        nz = o[r, :n] != 0
        if nz.any():
            st["max_rel"] = max(st["max_rel"], float((d[nz] / np.abs(o[r, :n][nz])).max()))
        st["max_err_over_tol"] = max(st["max_err_over_tol"], float((d / tol(o[r, :n])).max()))
        if bound is not None:
            b = bound[r, :n]
            over = d > b
            assert not over.any(), (f"{where} row {r}: {over.sum()} scores beyond the fp32 error "
                                    f"bound (max err {d.max():.3e}, bound there {b[over][0]:.3e})")
            st["max_err_over_bound"] = max(st["max_err_over_bound"],
                                           float((d / np.maximum(b, 1e-300)).max()))
    return st


def fp32_error_bound(q_bits, w, kp_bits, cu_pools, seq, t, kpool, D, H, width):
    """Forward error bound of the GPU's fp32 evaluation of one row's scores, fp64 [rows, width].

    The GPU forms each head's dot product from exact bf16 x bf16 products summed in
    fp32 (D terms), applies the ReLU, multiplies by the fp32 value of scale*w[h]
    (scale itself rounded to fp32) and sums the H heads in fp32.  With unit roundoff
    u = 2^-24 (doubled to allow accumulation that truncates), the standard first-order
    bound on such sums gives |g - S| <= 2 (D + H + 8) u A, where
        A[i,p] = sum_h |w[i,h]| * scale * sum_d |q[i,h,d]| |kp[p,d]|,
    the same expression as the score with every term made non-negative.  The ReLU only
    removes terms, and a dot product that rounds across zero costs at most its own
    error, which A already covers."""
    import oracle as O
    qa = np.abs(O.bf16_to_f32(q_bits).astype(np.float64))
    wa = np.abs(np.asarray(w, dtype=np.float32).astype(np.float64))
    kpa = np.abs(O.bf16_to_f32(kp_bits).astype(np.float64))
    scale = 1.0 / np.sqrt(D)
    u = 2.0 ** -24
    out = np.zeros((len(t), width))
    for i in range(len(t)):
        base = int(cu_pools[seq[i]])
        n = int(t[i]) // kpool + 1
        a = wa[i] @ (qa[i] @ kpa[base:base + n].T)
        out[i, :n] = 2.0 * (D + H + 8) * u * scale * a
    return out


def check_topk_self(g_scores, g_ids, nvis, budget, where=""):
    for r in range(len(nvis)):
        want = lexsort_first(g_scores[r, :int(nvis[r])], budget)  # (all -1 for a row with none)
        if not np.array_equal(want, g_ids[r]):
            bad = np.nonzero(want != g_ids[r])[0][:5]
            raise AssertionError(f"{where} row {r}: top-k differs from its own scores at slots "
                                 f"{bad.tolist()}: gpu {g_ids[r][bad].tolist()} want {want[bad].tolist()}")


def check_selection_vs_oracle(g_ids, o_scores, nvis, budget, where=""):
    """Set and order agreement with the fp64 oracle, up to pools tied within tolerance.

    Every pool in the symmetric difference of the GPU's and the oracle's id sets must
    score (in the oracle) within tau = tol(c) of the row's cutoff c, the oracle's
    budget-th best score.  Returns how close the rows came: the number of rows and
    pools that differ, the worst |o_p - c| / tau over the differing pools, and how
    many of those fall between tau and 2 tau (both sides carry error, so 2 tau is the
    strict bound; the gate is tau, and such pools are reported here)."""
    st = {"rows": len(nvis), "rows_differing": 0, "pools_differing": 0,
          "worst_cutoff_dist_over_tau": 0.0, "pools_between_tau_and_2tau": 0}
    for r in range(len(nvis)):
        n = int(nvis[r])
        o = o_scores[r, :n]
        ids = g_ids[r]
        sel = ids[ids >= 0]
        assert len(sel) == min(n, budget), f"{where} row {r}: {len(sel)} ids, want {min(n, budget)}"
        assert np.all(ids[len(sel):] == -1), f"{where} row {r}: padding not at the tail"
        if n == 0:          # no visible pool (tail mode, a sequence shorter than kpool)
            continue
        assert len(np.unique(sel)) == len(sel), f"{where} row {r}: duplicate ids"
        assert sel.max() < n, f"{where} row {r}: id beyond the visible pools"
        want = oracle.select_row(o, budget)
        want = want[want >= 0]
        if n <= budget:
            assert set(sel.tolist()) == set(range(n)), f"{where} row {r}: not every visible pool"
        else:
            c = np.sort(o)[::-1][budget - 1]
            diff = np.setxor1d(sel, want)
            if len(diff):
                err = np.abs(o[diff] - c)
                ratio = err / tol(c)
                st["rows_differing"] += 1
                st["pools_differing"] += len(diff)
                st["worst_cutoff_dist_over_tau"] = max(st["worst_cutoff_dist_over_tau"],
                                                      float(ratio.max()))
                st["pools_between_tau_and_2tau"] += int(((ratio > 1) & (ratio <= 2)).sum())
                assert np.all(err <= tol(c)), (f"{where} row {r}: pools {diff[err > tol(c)][:5]} "
                                               f"differ from the oracle away from the cutoff")
        # order: oracle scores non-increasing along the GPU order, within tolerance
        os_ = o[sel]
        drops = os_[1:] - os_[:-1]
        assert np.all(drops <= tol(os_[:-1])), f"{where} row {r}: order disagrees with the oracle"
    return st


def report(where, **stats):
    """One line of figures per check, printed (run pytest with -s or -v -rA to see them)."""
    parts = []
    for name, st in stats.items():
        parts.append(name + " " + " ".join(f"{k}={v:.3g}" if isinstance(v, float) else f"{k}={v}"
                                           for k, v in st.items()))
    print(f"[parity] {where}: " + "; ".join(parts), flush=True)


def check_tokens(g_tok, g_ids, t, kpool, o_ids=None, o_tok=None, where=""):
    """Token ids: equal to the oracle's where the pool ids agree with it, and for every row
    slot b*kpool+j holds p*kpool+j for p = ids[b] >= 0 with p*kpool+j <= t, else -1."""
    t = np.asarray(t, dtype=np.int64)
    p = np.repeat(g_ids.astype(np.int64), kpool, axis=1)
    j = np.tile(np.arange(kpool), g_ids.shape[1])[None, :]
    tok = p * kpool + j
    want = np.where((p >= 0) & (tok <= t[:, None]), tok, -1)
    bad = np.nonzero((g_tok != want).any(axis=1))[0]
    assert len(bad) == 0, f"{where} rows {bad[:5].tolist()}: token ids break the expansion rule"
    if o_ids is not None:
        same = (g_ids == o_ids).all(axis=1)
        assert np.array_equal(g_tok[same], o_tok[same]), f"{where}: token ids differ from the oracle"


def oracle_rows(inputs, kpool, rows, kp=None, width=None):
    """fp64 oracle scores for the given global rows (and the pooled keys)."""
    cu = np.asarray(inputs["cu_seqlens"])
    if kp is None:
        kp = oracle.pool_keys(inputs["k"], cu, kpool)
    cu_pools, max_pools = oracle.count_pools(cu, kpool)
    rows = np.asarray(rows)
    seq, t = oracle.row_positions(rows, cu)
    s = oracle.row_scores(inputs["q"][rows], inputs["w"][rows], kp, cu_pools, seq, t, kpool,
                          width=max_pools if width is None else width)
    return kp, s, t


def gated_allowed(vals, k_bits, g_bits, ape, cu_seqlens, kpool, u=2.0 ** -53, tail=False):
    """Bounds [lo, hi] (fp32 values of bf16 numbers) that the GPU's gated pooled keys may take.

    vals: the oracle's fp64 values of the gated pooled keys.  The GPU evaluates the
    same reading in floating point with unit roundoff u (fp64 in the kernel; the
    oracle's own fp64 evaluation errs the same way): z_j = g + ape, z_j - m, e_j = exp
    (an error of a few ulp), the slot sums and one divide.  First-order error analysis
    gives |gpu - value| <= delta = 2 (2 (eps_e + n u) + u) A, where
    eps_e = 4 u max_j |z_j| + 4 u bounds the relative error of each e_j,
    A = sum_j e_j |k_j| / sum_j e_j, and the factor 2 is a margin; it is doubled once
    more because the oracle's value carries an error of the same kind.  The GPU's bf16
    must then lie between the roundings of value - delta and value + delta: the
    rounding of the value itself, except where the value sits within delta of a
    rounding midpoint.  Returns (lo, hi, ambiguous mask)."""
    import oracle as O
    k = O.bf16_to_f32(k_bits).astype(np.float64)
    g = O.bf16_to_f32(g_bits).astype(np.float64)
    a = np.asarray(ape, np.float32).astype(np.float64)
    cu = np.asarray(cu_seqlens, np.int64)
    cu_pools, _ = O.count_pools(cu, kpool, tail)
    delta = np.zeros_like(vals)
    for s in range(len(cu) - 1):
        start, L = int(cu[s]), int(cu[s + 1] - cu[s])
        P = int(cu_pools[s + 1] - cu_pools[s])
        for j0 in range(0, P, 4096):                       # pools in blocks, vectorised
            ps = np.arange(j0, min(P, j0 + 4096))
            for n in np.unique(np.minimum(kpool, L - ps * kpool)):
                sel = ps[np.minimum(kpool, L - ps * kpool) == n]
                t = start + sel[:, None] * kpool + np.arange(n)[None, :]      # [np, n]
                z = g[t] + a[None, :n]                                        # [np, n, D]
                m = z.max(axis=1, keepdims=True)
                e = np.exp(z - m)
                A = (e * np.abs(k[t])).sum(axis=1) / e.sum(axis=1)
                eps_e = 4 * u * np.abs(z).max(axis=1) + 4 * u
                delta[int(cu_pools[s]) + sel] = 4 * (2 * (eps_e + n * u) + u) * A
    lo = O.bf16_to_f32(O.f64_to_bf16_rne(vals - delta))
    hi = O.bf16_to_f32(O.f64_to_bf16_rne(vals + delta))
    return lo, hi, lo != hi


def check_gated_keys(gpu_bits, vals, k_bits, g_bits, ape, cu_seqlens, kpool, where="", tail=False):
    """The GPU's gated pooled keys against the oracle's values (rule in gated_allowed)."""
    import oracle as O
    lo, hi, amb = gated_allowed(vals, k_bits, g_bits, ape, cu_seqlens, kpool, tail=tail)
    got = O.bf16_to_f32(gpu_bits)
    bad = (got < lo) | (got > hi)
    assert not bad.any(), (f"{where}: {bad.sum()} gated keys outside the error bound, first at "
                           f"{np.argwhere(bad)[0].tolist()}")
    exact = O.f64_to_bf16_rne(vals)
    st = {"keys": int(vals.size), "near_midpoint": int(amb.sum()),
          "differ_from_oracle_bits": int((gpu_bits != exact).sum())}
    assert st["differ_from_oracle_bits"] <= st["near_midpoint"]
    return st
