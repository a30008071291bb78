"""Seeded synthetic inputs for the k-pool indexer selection.

This module only draws random numbers and lays them out.  It holds none of
the selection's arithmetic, and both the HIP path's tests and the CPU oracle
take their inputs from it.

Every tensor is generated per block of ``BLOCK_ROWS`` packed rows from
``numpy.random.SeedSequence([seed, tensor_id, block])`` with PCG64, so any row
window can be regenerated on its own without materialising the whole input.
fp32 draws are rounded to bf16 (round-to-nearest-even) by torch's dtype cast,
and bf16 tensors are returned as their uint16 bit patterns.

Workloads (the shapes of the pages' GLM-5.3-Flash indexer runs: 32 index
heads, index_topk 2048 with kpool 4, i.e. 512 pools per row, up to 512k
tokens; head dim 128):

  tiny       T=64, H=4, D=16, kpool 4, budget 4; w ~ U(0,1)
  sq4096     one sequence of 4096 tokens, H=32, D=128, budget 512; w ~ U(0,1)/H
  thd65536   two batches of 32768 tokens, each cut into 1..8 ragged sequences
  sq262144   one sequence of 262144 tokens
  sq524288   one sequence of 524288 tokens (and its last 1/8 row slice)
  *_k1       the same shapes with kpool 1 (the per-token indexer: every token is a
             pool) and budget 2048 = index_topk
  *_gated    the same shapes with gate scores g [T, D] (N(0,1) rounded to bf16)
             and slot embeddings ape [kpool, D] (fp32 N(0,1)) for the gated pooling

q and k are N(0,1) draws rounded to bf16; w is fp32.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BLOCK_ROWS = 4096

# tensor ids for the seed sequence
_Q, _K, _W, _CU, _G, _APE = 1, 2, 3, 4, 5, 6


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    D: int
    kpool: int
    budget: int
    w_div: float            # w ~ U(0,1) / w_div
    layout: str = "single"  # "single" sequence or "thd" packed batches
    thd_batch: int = 32768
    thd_max_seqs: int = 8
    q_lo: int = 0
    q_hi: int | None = None
    # test-only variants: "w_zero", "w_neg", "k_ternary", "k_const"
    variant: str = ""
    # "mean" pooling, or "gated" (gate scores g [T, D] and slot embeddings ape [kpool, D])
    pooling: str = "mean"
    extra: dict = field(default_factory=dict)

    @property
    def rows(self) -> tuple[int, int]:
        return self.q_lo, (self.T if self.q_hi is None else self.q_hi)


WORKLOADS = {
    "tiny": Workload("tiny", 64, 4, 16, 4, 4, 1.0),
    "sq4096": Workload("sq4096", 4096, 32, 128, 4, 512, 32.0),
    "thd65536": Workload("thd65536", 65536, 32, 128, 4, 512, 32.0, layout="thd"),
    "sq262144": Workload("sq262144", 262144, 32, 128, 4, 512, 32.0),
    "sq524288": Workload("sq524288", 524288, 32, 128, 4, 512, 32.0),
    "sq524288_slice": Workload("sq524288_slice", 524288, 32, 128, 4, 512, 32.0,
                               q_lo=7 * 524288 // 8, q_hi=524288),
    # kpool 1: index_topk 2048 tokens = 2048 pools per row
    "sq4096_k1": Workload("sq4096_k1", 4096, 32, 128, 1, 2048, 32.0),
    "thd65536_k1": Workload("thd65536_k1", 65536, 32, 128, 1, 2048, 32.0, layout="thd"),
    "sq262144_k1": Workload("sq262144_k1", 262144, 32, 128, 1, 2048, 32.0),
    "sq524288_k1": Workload("sq524288_k1", 524288, 32, 128, 1, 2048, 32.0),
    # gated k-pool compression: the same shapes with gate scores and slot embeddings
    "tiny_gated": Workload("tiny_gated", 64, 4, 16, 4, 4, 1.0, pooling="gated"),
    "sq4096_gated": Workload("sq4096_gated", 4096, 32, 128, 4, 512, 32.0, pooling="gated"),
    "thd65536_gated": Workload("thd65536_gated", 65536, 32, 128, 4, 512, 32.0, layout="thd",
                               pooling="gated"),
    "sq524288_gated": Workload("sq524288_gated", 524288, 32, 128, 4, 512, 32.0, pooling="gated"),
}


def workload(name: str, **overrides) -> Workload:
    base = WORKLOADS[name]
    if not overrides:
        return base
    d = dict(base.__dict__)
    d.update(overrides)
    return Workload(**d)


def _rng(seed: int, tensor: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor, block])))


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def cu_seqlens(wl: Workload, seed: int = 0) -> np.ndarray:
    """Packed sequence boundaries (int32, [nseq + 1])."""
    if wl.layout == "single":
        return np.array([0, wl.T], dtype=np.int32)
    if wl.layout != "thd":
        raise ValueError(wl.layout)
    nb = wl.T // wl.thd_batch
    bounds = [0]
    for b in range(nb):
        rng = _rng(seed, _CU, b)
        n = int(rng.integers(1, wl.thd_max_seqs + 1))
        cuts = np.sort(rng.choice(np.arange(1, wl.thd_batch), size=n - 1, replace=False))
        base = b * wl.thd_batch
        bounds += [base + int(c) for c in cuts] + [base + wl.thd_batch]
    return np.array(bounds, dtype=np.int32)


def _block_rows(wl: Workload, block: int) -> int:
    return min(BLOCK_ROWS, wl.T - block * BLOCK_ROWS)


def q_block(wl: Workload, seed: int, block: int) -> np.ndarray:
    rows = _block_rows(wl, block)
    x = _rng(seed, _Q, block).standard_normal((rows, wl.H, wl.D), dtype=np.float32)
    return _to_bf16_bits(x)


def k_block(wl: Workload, seed: int, block: int) -> np.ndarray:
    rows = _block_rows(wl, block)
    rng = _rng(seed, _K, block)
    if wl.variant == "k_ternary":
        x = rng.integers(-1, 2, size=(rows, wl.D)).astype(np.float32)
    elif wl.variant == "k_const":
        x = np.full((rows, wl.D), 0.7, dtype=np.float32)
    else:
        x = rng.standard_normal((rows, wl.D), dtype=np.float32)
    return _to_bf16_bits(x)


def w_block(wl: Workload, seed: int, block: int) -> np.ndarray:
    rows = _block_rows(wl, block)
    rng = _rng(seed, _W, block)
    if wl.variant == "w_zero":
        return np.zeros((rows, wl.H), dtype=np.float32)
    u = rng.random((rows, wl.H), dtype=np.float32)
    if wl.variant == "w_neg":
        u = (np.float32(2.0) * u - np.float32(1.0)).astype(np.float32)
    return (u / np.float32(wl.w_div)).astype(np.float32)


def g_block(wl: Workload, seed: int, block: int) -> np.ndarray:
    """Gate scores (the gate projection's output), N(0,1) rounded to bf16, [rows, D]."""
    rows = _block_rows(wl, block)
    x = _rng(seed, _G, block).standard_normal((rows, wl.D), dtype=np.float32)
    return _to_bf16_bits(x)


def ape(wl: Workload, seed: int) -> np.ndarray:
    """Slot embeddings of the gated pooling, fp32 N(0,1), [kpool, D]."""
    return _rng(seed, _APE, 0).standard_normal((wl.kpool, wl.D), dtype=np.float32)


def _blocks(lo: int, hi: int):
    return range(lo // BLOCK_ROWS, (hi + BLOCK_ROWS - 1) // BLOCK_ROWS)


def rows(wl: Workload, seed: int, lo: int, hi: int, which=("q", "k", "w")):
    """Regenerate rows [lo, hi) of q, k and/or w (host numpy arrays)."""
    gens = {"q": q_block, "k": k_block, "w": w_block, "g": g_block}
    out = {}
    for name in which:
        parts = []
        for b in _blocks(lo, hi):
            blk = gens[name](wl, seed, b)
            a = max(lo, b * BLOCK_ROWS) - b * BLOCK_ROWS
            e = min(hi, b * BLOCK_ROWS + len(blk)) - b * BLOCK_ROWS
            parts.append(blk[a:e])
        out[name] = np.concatenate(parts, axis=0) if parts else None
    return out


def host_inputs(wl: Workload, seed: int = 0) -> dict:
    """Whole workload on the host (small workloads only)."""
    gated = wl.pooling == "gated"
    r = rows(wl, seed, 0, wl.T, ("q", "k", "w", "g") if gated else ("q", "k", "w"))
    r["cu_seqlens"] = cu_seqlens(wl, seed)
    if gated:
        r["ape"] = ape(wl, seed)
    return r


def device_inputs(wl: Workload, seed: int = 0, device="cuda", threads: int | None = None) -> dict:
    """Whole workload generated block by block straight into device tensors.

    torch is used only to hold device memory.  Blocks are drawn in a thread
    pool (numpy releases the GIL while drawing) and copied as they finish.
    """
    import torch
    if threads is None:
        threads = max(1, min(16, len(os.sched_getaffinity(0))))
    q = torch.empty((wl.T, wl.H, wl.D), dtype=torch.int16, device=device)
    k = torch.empty((wl.T, wl.D), dtype=torch.int16, device=device)
    w = torch.empty((wl.T, wl.H), dtype=torch.float32, device=device)
    nblk = (wl.T + BLOCK_ROWS - 1) // BLOCK_ROWS

    gated = wl.pooling == "gated"
    g = torch.empty((wl.T, wl.D), dtype=torch.int16, device=device) if gated else None

    def make(b):
        return (b, q_block(wl, seed, b), k_block(wl, seed, b), w_block(wl, seed, b),
                g_block(wl, seed, b) if gated else None)

    with ThreadPoolExecutor(threads) as ex:
        for b, qb, kb, wb, gb in ex.map(make, range(nblk)):
            lo = b * BLOCK_ROWS
            hi = lo + len(qb)
            q[lo:hi].copy_(torch.from_numpy(qb.view(np.int16)))
            k[lo:hi].copy_(torch.from_numpy(kb.view(np.int16)))
            w[lo:hi].copy_(torch.from_numpy(wb))
            if gated:
                g[lo:hi].copy_(torch.from_numpy(gb.view(np.int16)))
    cu = cu_seqlens(wl, seed)
    out = {"q": q, "k": k, "w": w, "cu_seqlens": cu}
    if gated:
        out["g"] = g
        out["ape"] = torch.from_numpy(ape(wl, seed)).to(device)
    return out
