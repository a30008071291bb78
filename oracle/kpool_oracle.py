"""CPU oracle for the k-pool DSA indexer selection.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import, call or execute this
module.  The product path (the HIP library and its Python binding) never
imports it, and has no CPU fallback.

Plain, slow definitions of what the selection computes, evaluated one query
row at a time, with no chunking, tiling, fusion or reordering beyond what the
definition states.  It shares no code with the HIP path; the bf16 rounding
routine below is written here independently.

Steps, in the order the pages describe the selection op:

  O1  pool_keys     each pool's key = mean of its kpool consecutive keys
                    (fp32 sum in token order starting from +0, fp32 divide,
                    bf16 round-to-nearest-even)
  O1g pool_keys_gated  the gated alternative: per dim, a softmax over the
                    pool's slots of (gate score + slot embedding) weights the
                    keys (fp64, one bf16 rounding).  The formula is a reading:
                    parity against the pages' own operator is unpinned
  O2  row_scores    fp64  S[i,p] = sum_h w[i,h] * relu(scale * <q[i,h], kp[p]>)
                    over the pools visible to row i (p*kpool <= t)
  O3  select_row    order the visible pools by (score desc, pool index asc),
                    keep the first `budget`, pad with -1
  O4  expand_row    pool p -> tokens p*kpool + j, -1 where the token lies after
                    the row (token > t) or the slot is padding; in tail mode
                    (full pools only) the sequence's trailing L mod kpool tokens
                    are appended and filtered the same way.  "Tail append" is
                    named but not defined on the pages: this reading's parity
                    against the pages' own operator is unpinned

Sources (the pages this oracle follows):
  * Atlas inference docs, ``spark_model/layers/glm5next_dsa/tp.rs``, module
    doc "Why the indexer is REPLICATED, not sharded": the per-head score is a
    weighted ReLU of a scaled dot product summed over heads; pools are
    ``kpool`` consecutive tokens (``n_pools = seq / kpool``); the tie-break
    prefers the higher score and then the smaller pool index.
  * Megatron-LM PR #8299, "Mechanism": every query row scores the pooled keys;
    a row's selection depends only on that row and the pooled keys.
  * Megatron-LM PR #8299, "Change": selections are int32 pool ids per row;
    pools are then expanded to tokens and mask-filtered.
  * Megatron-LM PR #8299, "Test plan": causal mask and packed varlen bounds.

Readings taken where the pages are silent (stated once here, listed in the
design notes): the pooling operator is the mean with fp32 accumulation, the
scale is 1/sqrt(D), a pool is visible to the row at local position t iff its
first token p*kpool <= t, ids are sequence-local, unused slots hold -1, and
-0.0 ranks equal to +0.0.  NaN scores rank below every number (also below
-inf) and among themselves by pool index.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_to_f32",
    "f32_to_bf16_rne",
    "f64_to_bf16_rne",
    "count_pools",
    "pool_keys",
    "pool_keys_gated",
    "row_positions",
    "visible_pools",
    "row_scores",
    "select_row",
    "select_row_full_sort",
    "expand_row",
    "select",
]


# ---------------------------------------------------------------------------
# bf16 <-> fp32 (independent implementation; bf16 is stored as uint16 bits)
# ---------------------------------------------------------------------------

def bf16_to_f32(bits) -> np.ndarray:
    """Exact widening: a bf16 value is the upper half of an fp32 bit pattern."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_rne(x) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN.

    Adding 0x7FFF plus the lowest kept bit carries into the kept half exactly
    when the dropped half is above one half ulp, or equal to it with an odd
    kept half.  Finite values that round past the largest bf16 become inf,
    which is what round-to-nearest does.
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    if np.any(nan):
        r = np.where(nan, ((u >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint16), r)
    return r.astype(np.uint16)


# ---------------------------------------------------------------------------
# O1: pooled keys
# ---------------------------------------------------------------------------

def count_pools(cu_seqlens, kpool: int, tail: bool = False):
    """Pools per sequence; returns (cu_pools, max_pools).

    Default: ceil(L_s / kpool), a trailing partial pool (L_s not a multiple of
    kpool) kept as a pool of its own (reading).  tail=True: the full pools only,
    floor(L_s / kpool) -- the pool count of Atlas tp.rs module doc,
    ``n_pools = seq / kpool`` -- and the L_s mod kpool trailing tokens form the
    sequence's tail, which expand_row appends (reading of Megatron-LM PR #8299
    "Change": pool expansion, tail append, mask filtering).
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    lens = np.diff(cu)
    npools = lens // kpool if tail else (lens + kpool - 1) // kpool
    cu_pools = np.concatenate([[0], np.cumsum(npools)]).astype(np.int64)
    max_pools = int(npools.max()) if len(npools) else 0
    return cu_pools, max_pools


def pool_keys(k_bits, cu_seqlens, kpool: int, tail: bool = False) -> np.ndarray:
    """Pooled keys, bf16 bits ``[P_tot, D]``; pools of sequence s start at cu_pools[s].

    For pool p of sequence s with n_p = min(kpool, L_s - p*kpool) tokens:
        acc = +0 (fp32); acc = fp32(acc + k[token]) for the tokens in order;
        kp  = bf16_rne(fp32(acc / n_p)).
    Megatron-LM PR #8299 "Mechanism" (rows score the pooled keys); Atlas
    tp.rs module doc (pools of kpool consecutive tokens).  Mean with fp32
    accumulation and a bf16 result is the reading adopted here.  With
    tail=True only the full pools exist (count_pools).
    """
    k = bf16_to_f32(k_bits)
    if k.ndim != 2:
        raise ValueError("k must be [T, D]")
    D = k.shape[1]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    cu_pools, _ = count_pools(cu, kpool, tail)
    out = np.zeros((int(cu_pools[-1]), D), dtype=np.uint16)
    for s in range(len(cu) - 1):
        start, end = int(cu[s]), int(cu[s + 1])
        L = end - start
        nfull = L // kpool
        base = int(cu_pools[s])
        if nfull:
            blk = k[start:start + nfull * kpool].reshape(nfull, kpool, D)
            acc = np.zeros((nfull, D), dtype=np.float32)
            for j in range(kpool):  # token order within the pool
                acc = (acc + blk[:, j, :]).astype(np.float32)
            mean = (acc / np.float32(kpool)).astype(np.float32)
            out[base:base + nfull] = f32_to_bf16_rne(mean)
        rem = L - nfull * kpool
        if rem and not tail:
            acc = np.zeros(D, dtype=np.float32)
            for j in range(rem):
                acc = (acc + k[start + nfull * kpool + j]).astype(np.float32)
            mean = (acc / np.float32(rem)).astype(np.float32)
            out[base + nfull] = f32_to_bf16_rne(mean)
    return out


def f64_to_bf16_rne(x) -> np.ndarray:
    """fp64 -> bf16 bits, one round to nearest (ties to even) from the fp64 value.

    x = m * 2**e with 0.5 <= |m| < 1 (frexp); a bf16 number has 8 significant
    bits, so the result is rint(m * 2**8) * 2**(e - 8) (rint rounds half to
    even), with the quantum held at 2**-133 below the smallest normal bf16
    exponent (subnormals) and overflow past the largest bf16 going to inf.
    The value is exact in fp32, whose upper 16 bits are then the bf16 pattern.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    e = np.maximum(e, -125)                     # 2**(e-1) >= 2**-126: fixed quantum below
    q = np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)
    q = np.where(np.abs(q) >= 2.0 ** 128, np.copysign(np.inf, x), q)
    q = np.where(np.isfinite(x), q, x)
    with np.errstate(over="ignore"):
        f = q.astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def pool_keys_gated(k_bits, g_bits, ape, cu_seqlens, kpool: int, return_values: bool = False,
                    tail: bool = False):
    """Gated pooled keys, bf16 bits ``[P_tot, D]`` (and their fp64 values if asked).

    PARITY UNPINNED AGAINST THE PAGES: they name the GLM-5.3 indexer's k-pool
    compression tensors -- a gate projection [index_head_dim, hidden] and an
    absolute position embedding [index_kpool, index_head_dim] (Atlas inference
    docs, glm5next_dsa/tp.rs, the indexer tensors of the shard plan) -- and say
    the op takes gate scores as an input (Megatron-LM PR #8299, "Mechanism"),
    but give no formula.  This is the reading adopted (the pins in
    tests/test_oracle_gated.py fix this reading, not the pages' operator):

      for pool p of sequence s, tokens t_j = start_s + p*kpool + j, j < n_p,
      and every dim d:
        z_j   = g[t_j, d] + ape[j, d]                       (gate score + slot embedding)
        a_j   = exp(z_j - max_j z_j) / sum_j exp(z_j - max_j z_j)   (softmax over the slots)
        kp[p, d] = bf16_rne( sum_j a_j * k[t_j, d] )

    A trailing partial pool (n_p < kpool) uses the slot embeddings of the slots
    it has, ape[0 .. n_p - 1]; with tail=True only full pools exist.  Arithmetic in fp64 from the bf16 keys and gate
    scores (g = the gate projection's output, one value per token and dim) and
    the fp32 embeddings, rounded once to bf16.
    """
    k = bf16_to_f32(k_bits).astype(np.float64)
    g = bf16_to_f32(g_bits).astype(np.float64)
    a = np.asarray(ape, dtype=np.float32).astype(np.float64)
    if k.ndim != 2 or g.shape != k.shape or a.shape != (kpool, k.shape[1]):
        raise ValueError("need k, g [T, D] and ape [kpool, D]")
    D = k.shape[1]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    cu_pools, _ = count_pools(cu, kpool, tail)
    vals = np.zeros((int(cu_pools[-1]), D), dtype=np.float64)
    for s in range(len(cu) - 1):
        start, L = int(cu[s]), int(cu[s + 1] - cu[s])
        for p in range(int(cu_pools[s + 1] - cu_pools[s])):
            t0 = start + p * kpool
            n = min(kpool, L - p * kpool)
            z = g[t0:t0 + n] + a[:n]                   # [n, D]
            e = np.exp(z - z.max(axis=0))              # softmax over the n slots, per dim
            wts = e / e.sum(axis=0)
            vals[int(cu_pools[s]) + p] = (wts * k[t0:t0 + n]).sum(axis=0)
    bits = f64_to_bf16_rne(vals)
    return (bits, vals) if return_values else bits


# ---------------------------------------------------------------------------
# Row bookkeeping
# ---------------------------------------------------------------------------

def row_positions(rows, cu_seqlens):
    """Global packed row index -> (sequence s, local position t = i - start_s).

    Megatron-LM PR #8299 "Test plan": packed THD rows are bounded by
    cu_seqlens; positions, pool ids and token ids are sequence-local.
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    s = np.searchsorted(cu, rows, side="right") - 1
    if np.any(rows < 0) or np.any(rows >= cu[-1]):
        raise ValueError("row outside [0, T)")
    return s, rows - cu[s]


def visible_pools(t, kpool: int, npools=None):
    """Number of pools visible to local position t: pools p with p*kpool <= t (and,
    when the sequence has only npools pools, p < npools)."""
    nv = np.asarray(t, dtype=np.int64) // kpool + 1
    return nv if npools is None else np.minimum(nv, np.asarray(npools, dtype=np.int64))


# ---------------------------------------------------------------------------
# O2: scores (fp64)
# ---------------------------------------------------------------------------

def row_scores(q_rows_bits, w_rows, kp_bits, cu_pools, seq, t, kpool: int,
               scale: float | None = None, width: int | None = None) -> np.ndarray:
    """fp64 scores for a set of rows, ``[r, width]``, -inf where a pool is masked.

    S[i,p] = sum_h w[i,h] * max(0, scale * sum_d q[i,h,d] * kp[s,p,d])
    for p < visible_pools(t) (capped at the sequence's pool count, which
    cu_pools gives; only tail mode's count can be below it).  Atlas tp.rs module doc (the head-weighted
    ReLU sum); the scale 1/sqrt(D) is the reading adopted here.  Order of
    operations: dot, times scale, ReLU, times w, sum over heads.
    q_rows_bits: bf16 bits [r, H, D]; w_rows: fp32 [r, H]; kp_bits: [P_tot, D].
    """
    q = bf16_to_f32(q_rows_bits).astype(np.float64)
    w = np.asarray(w_rows, dtype=np.float32).astype(np.float64)
    kp = bf16_to_f32(kp_bits).astype(np.float64)
    r, H, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(np.float64(D))
    seq = np.asarray(seq, dtype=np.int64)
    t = np.asarray(t, dtype=np.int64)
    cu_pools = np.asarray(cu_pools, dtype=np.int64)
    nv = visible_pools(t, kpool, cu_pools[seq + 1] - cu_pools[seq])
    if width is None:
        width = int(nv.max()) if r else 0
    out = np.full((r, width), -np.inf, dtype=np.float64)
    for i in range(r):
        base = int(cu_pools[seq[i]])
        n = int(nv[i])
        keys = kp[base:base + n]                      # [n, D]
        dots = q[i] @ keys.T                          # [H, n], fp64
        act = np.maximum(scale * dots, 0.0)           # ReLU(scale * dot)
        out[i, :n] = w[i] @ act                       # sum_h w[h] * act[h, :]
    return out


# ---------------------------------------------------------------------------
# O3: selection with the deterministic tie-break
# ---------------------------------------------------------------------------

def _canon(scores_row) -> tuple[np.ndarray, np.ndarray]:
    s = np.asarray(scores_row, dtype=np.float64) + 0.0   # -0.0 -> +0.0
    isnan = np.isnan(s)
    return np.where(isnan, -np.inf, s), isnan


def select_row_full_sort(scores_row, budget: int) -> np.ndarray:
    """Reference selection by one full sort of the row's visible scores.

    Key (NaN last, score desc, pool index asc).  Atlas tp.rs module doc:
    the tie-break is higher score first, then the smaller pool index.
    Unused slots are -1 (reading).
    """
    s, isnan = _canon(scores_row)
    idx = np.arange(len(s), dtype=np.int64)
    order = np.lexsort((idx, -s, isnan))
    out = np.full(budget, -1, dtype=np.int32)
    take = order[:budget]
    out[:len(take)] = take
    return out


def select_row(scores_row, budget: int) -> np.ndarray:
    """Same result as select_row_full_sort, with a partition to find the cutoff.

    The budget-th best score c is found by partition; every pool scoring
    above c is kept and pools equal to c are ordered by index, by sorting
    only the pools that score at least c.
    """
    s, isnan = _canon(scores_row)
    n = len(s)
    if n <= 4 * budget or np.any(isnan):
        return select_row_full_sort(scores_row, budget)
    neg = -s
    c = np.partition(neg, budget - 1)[budget - 1]    # -(budget-th largest)
    cand = np.nonzero(neg <= c)[0]
    order = cand[np.lexsort((cand, neg[cand]))]
    return order[:budget].astype(np.int32)


# ---------------------------------------------------------------------------
# O4: expansion and causal filter
# ---------------------------------------------------------------------------

def expand_row(ids, t: int, kpool: int, tail=None) -> np.ndarray:
    """Token ids for one row: slot b*kpool+j holds p*kpool+j for p = ids[b].

    -1 where the slot is padding (p < 0) or the token comes after the row
    (p*kpool + j > t).  Megatron-LM PR #8299 "Change": pool expansion and
    mask filtering after the pool ids are known; filtered entries stay in
    place as -1 (reading).

    tail = (a, b): tail mode (see count_pools).  The sequence's tail tokens
    a .. b-1 (sequence-local, b - a < kpool) are appended after the expanded
    pools in kpool - 1 more slots, and the same causal filter applies to them:
    slot budget*kpool + j holds a + j if a + j < b and a + j <= t, else -1
    (the pages' order: expansion, tail append, mask filtering).
    """
    ids = np.asarray(ids, dtype=np.int64)
    n_tail = 0 if tail is None else kpool - 1
    out = np.full(len(ids) * kpool + n_tail, -1, dtype=np.int32)
    for b, p in enumerate(ids):
        if p < 0:
            continue
        for j in range(kpool):
            tok = p * kpool + j
            if tok <= t:
                out[b * kpool + j] = tok
    if tail is not None:
        a, e = int(tail[0]), int(tail[1])
        for j in range(n_tail):
            tok = a + j
            if tok < e and tok <= t:
                out[len(ids) * kpool + j] = tok
    return out


# ---------------------------------------------------------------------------
# Whole path on a row range
# ---------------------------------------------------------------------------

def select(q_bits, k_bits, w, cu_seqlens, kpool: int, budget: int,
           q_lo: int = 0, q_hi: int | None = None, scale: float | None = None,
           kp_bits=None, tail: bool = False):
    """Pool, score, select and expand the rows [q_lo, q_hi) of a packed batch.

    Megatron-LM PR #8299 "Change": a query-row range is scored on its own and
    gives, row for row, what the whole range gives.  Returns a dict with
    ``kp`` (bf16 bits), ``scores`` (fp64, -inf where masked, width = the
    largest pool count of any sequence), ``pool_ids`` (int32, [rows, budget])
    and ``token_ids`` (int32, [rows, budget*kpool], plus kpool - 1 tail slots
    in tail mode).  tail=True: full pools only and the tail appended (see
    count_pools and expand_row).
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T = int(cu[-1])
    if q_hi is None:
        q_hi = T
    if not (0 <= q_lo <= q_hi <= T):
        raise ValueError("bad row range")
    cu_pools, max_pools = count_pools(cu, kpool, tail)
    kp = pool_keys(k_bits, cu, kpool, tail) if kp_bits is None else kp_bits
    rows = np.arange(q_lo, q_hi, dtype=np.int64)
    n = len(rows)
    n_tail = kpool - 1 if tail else 0
    scores = np.full((n, max_pools), -np.inf, dtype=np.float64)
    pool_ids = np.full((n, budget), -1, dtype=np.int32)
    token_ids = np.full((n, budget * kpool + n_tail), -1, dtype=np.int32)
    if n:
        seq, t = row_positions(rows, cu)
        q = np.asarray(q_bits)[q_lo:q_hi]
        ww = np.asarray(w)[q_lo:q_hi]
        step = 64
        for a in range(0, n, step):
            b = min(n, a + step)
            scores[a:b] = row_scores(q[a:b], ww[a:b], kp, cu_pools, seq[a:b], t[a:b],
                                     kpool, scale, width=max_pools)
        nv = visible_pools(t, kpool, cu_pools[seq + 1] - cu_pools[seq])
        for i in range(n):
            pool_ids[i] = select_row(scores[i, :nv[i]], budget)
            tl = None
            if tail:
                L = int(cu[seq[i] + 1] - cu[seq[i]])
                tl = (L // kpool * kpool, L)
            token_ids[i] = expand_row(pool_ids[i], int(t[i]), kpool, tl)
    return {"kp": kp, "scores": scores, "pool_ids": pool_ids, "token_ids": token_ids,
            "cu_pools": cu_pools, "max_pools": max_pools}
