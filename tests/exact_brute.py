"""Exact-arithmetic brute force for tiny inputs (a pin for the oracle).

Pure Python with ``fractions.Fraction``; no numpy arithmetic.  Floats are
decoded from their bit patterns by hand and every rounding the method
specifies (fp32 sums and divide in pooling, bf16 storage of the pooled key) is
done by an explicit round-to-nearest-even on exact rationals.  Scores are the
exact rational value of the definition, so it needs a head dim D that is a
perfect square (scale = 1/sqrt(D) is then rational).
"""
from __future__ import annotations

from fractions import Fraction
from math import isqrt

F32_P, F32_EMIN = 24, -126
BF16_P, BF16_EMIN = 8, -126


def decode_bf16(b: int) -> Fraction:
    b = int(b) & 0xFFFF
    sign = -1 if b >> 15 else 1
    e = (b >> 7) & 0xFF
    m = b & 0x7F
    if e == 0xFF:
        raise ValueError("inf/nan not supported")
    if e == 0:
        return sign * Fraction(m, 128) * Fraction(2) ** (-126)
    return sign * (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)


def decode_f32(u: int) -> Fraction:
    u = int(u) & 0xFFFFFFFF
    sign = -1 if u >> 31 else 1
    e = (u >> 23) & 0xFF
    m = u & 0x7FFFFF
    if e == 0xFF:
        raise ValueError("inf/nan not supported")
    if e == 0:
        return sign * Fraction(m, 1 << 23) * Fraction(2) ** (-126)
    return sign * (1 + Fraction(m, 1 << 23)) * Fraction(2) ** (e - 127)


def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_rne(x: Fraction, p: int, emin: int) -> Fraction:
    """Nearest number with p significant bits (exponent >= emin), ties to even."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = max(_floor_log2(a), emin)
    quantum = Fraction(2) ** (e - p + 1)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * quantum


def f32(x: Fraction) -> Fraction:
    return round_rne(x, F32_P, F32_EMIN)


def bf16(x: Fraction) -> Fraction:
    return round_rne(x, BF16_P, BF16_EMIN)


def pooled_keys(k_bits, cu_seqlens, kpool, tail=False):
    """[P_tot][D] exact values of the stored pooled keys (tail: full pools only)."""
    out = []
    D = len(k_bits[0])
    for s in range(len(cu_seqlens) - 1):
        start, end = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        p = 0
        while (p + 1) * kpool <= end - start if tail else p * kpool < end - start:
            toks = range(start + p * kpool, min(end, start + (p + 1) * kpool))
            row = []
            for d in range(D):
                acc = Fraction(0)
                for tk in toks:
                    acc = f32(acc + decode_bf16(k_bits[tk][d]))
                row.append(bf16(f32(acc / len(toks))))
            out.append(row)
            p += 1
    return out


def run(q_bits, k_bits, w_f32_bits, cu_seqlens, kpool, budget, tail=False):
    """Exact pooled keys, scores, selections and token ids for every row.

    tail: only the full pools of each sequence are pools, and the sequence's
    remaining tokens are appended to every row's token list (kpool - 1 slots),
    causally filtered like the pools' tokens."""
    T = int(cu_seqlens[-1])
    H = len(q_bits[0])
    D = len(q_bits[0][0])
    r = isqrt(D)
    if r * r != D:
        raise ValueError("exact brute force needs a square head dim")
    scale = Fraction(1, r)
    kp = pooled_keys(k_bits, cu_seqlens, kpool, tail)
    pool_base, pool_count = [], []
    base = 0
    for s in range(len(cu_seqlens) - 1):
        pool_base.append(base)
        L = int(cu_seqlens[s + 1]) - int(cu_seqlens[s])
        pool_count.append(L // kpool if tail else (L + kpool - 1) // kpool)
        base += pool_count[-1]
    scores, ids, toks = [], [], []
    for i in range(T):
        s = max(j for j in range(len(cu_seqlens) - 1) if int(cu_seqlens[j]) <= i)
        t = i - int(cu_seqlens[s])
        nvis = len([p for p in range(pool_count[s]) if p * kpool <= t])
        qi = [[decode_bf16(q_bits[i][h][d]) for d in range(D)] for h in range(H)]
        wi = [decode_f32(w_f32_bits[i][h]) for h in range(H)]
        row = []
        for p in range(nvis):
            key = kp[pool_base[s] + p]
            tot = Fraction(0)
            for h in range(H):
                dot = sum(qi[h][d] * key[d] for d in range(D))
                tot += wi[h] * max(Fraction(0), scale * dot)
            row.append(tot)
        order = sorted(range(nvis), key=lambda p: (-row[p], p))[:budget]
        sel = order + [-1] * (budget - len(order))
        tk = []
        for p in sel:
            for j in range(kpool):
                tk.append(p * kpool + j if p >= 0 and p * kpool + j <= t else -1)
        if tail:
            L = int(cu_seqlens[s + 1]) - int(cu_seqlens[s])
            for tok in range(pool_count[s] * kpool, pool_count[s] * kpool + kpool - 1):
                tk.append(tok if tok < L and tok <= t else -1)
        scores.append(row)
        ids.append(sel)
        toks.append(tk)
    return {"kp": kp, "scores": scores, "pool_ids": ids, "token_ids": toks}
