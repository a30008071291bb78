"""Python binding of libkpool (ctypes).  Argument marshalling only.

Every step of the selection runs in the HIP library; this module passes
torch tensors' device pointers and the current HIP stream through the C ABI
declared in include/kpool.h, allocates outputs with torch (device memory is
all torch is used for) and turns negative status codes into exceptions.
There is no CPU fallback: if libkpool.so is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkpool.so")

KPOOL_OK, KPOOL_EINVAL, KPOOL_EUNSUPPORTED, KPOOL_EWORKSPACE, KPOOL_EHIP = 0, -1, -2, -3, -4
KPOOL_FLAG_OVERLAP = 1
KPOOL_FLAG_TAIL = 2
PROFILE_KINDS = ("pool_keys", "score", "topk", "expand", "scores_copy")

_lib = None


class KpoolError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def lib():
    """The loaded libkpool.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libkpool.so is not built ({LIB_PATH}); run __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    u32 = ctypes.c_uint32
    sig = {
        "kpool_last_error": (ctypes.c_char_p, []),
        "kpool_version": (ctypes.c_int, []),
        "kpool_count_pools": (i64, [vp, i32, i32, u32, vp, vp]),
        "kpool_pool_keys": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, i32, u32, vp, vp]),
        "kpool_pool_keys_gated": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, i32, i32, i32, u32, vp, vp]),
        "kpool_workspace_bytes": (sz, [i64, i64, i32, i32]),
        "kpool_chunk_rows": (i64, [i32, sz, u32, vp]),
        "kpool_score_topk": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i64, i64,
                                            i32, vp, sz, u32, vp, vp, vp]),
        "kpool_score_topk_noalloc": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32,
                                                    i64, i64, i32, u32, vp, vp, vp]),
        "kpool_expand": (ctypes.c_int, [vp, vp, vp, i32, i32, i64, i64, i32, u32, vp, vp]),
        "kpool_topk": (ctypes.c_int, [vp, i64, vp, i64, i32, vp, vp]),
        "kpool_profile_enable": (ctypes.c_int, [ctypes.c_int]),
        "kpool_profile_collect": (ctypes.c_int, [vp, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(rc, fn):
    if rc != KPOOL_OK:
        raise KpoolError(fn, int(rc), lib().kpool_last_error().decode())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _host_i32(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Context in which the wrappers allocate: the stream the library call will run on.

    torch's caching allocator hands a freed block out again only to work ordered
    after the frees on the block's own stream; allocating on the call's stream
    keeps a workspace or output from being reused while the call still uses it."""
    import contextlib

    import torch
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _need(t, name, elem_size=None, dtype=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if elem_size is not None and t.element_size() != elem_size:
        raise ValueError(f"{name} must have {elem_size}-byte elements")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}")


# ---------------------------------------------------------------------------
# The C ABI, one wrapper per entry point
# ---------------------------------------------------------------------------

def version() -> int:
    return lib().kpool_version()


def _tail(tail):
    return KPOOL_FLAG_TAIL if tail else 0


def count_pools(cu_seqlens, kpool: int, tail: bool = False):
    """(cu_pools int32 [nseq+1], max_pools, P_tot) for a host cu_seqlens (tail: full pools)."""
    cu, cup = _host_i32(cu_seqlens)
    nseq = len(cu) - 1
    out = np.zeros(max(nseq, 0) + 1, dtype=np.int32)
    mx = ctypes.c_int32(0)
    tot = lib().kpool_count_pools(cup, nseq, kpool, _tail(tail), out.ctypes.data_as(ctypes.c_void_p),
                                  ctypes.byref(mx))
    _check(0 if tot >= 0 else tot, "kpool_count_pools")
    return out, int(mx.value), int(tot)


def workspace_bytes(q_lo: int, q_hi: int, max_pools: int, nbuf: int = 2) -> int:
    """Workspace of score_topk over rows [q_lo, q_hi): nbuf chunk buffers (2 for the
    chunk overlap, 1 without), each capped at 2 GiB of fp32 scores."""
    return int(lib().kpool_workspace_bytes(q_lo, q_hi, max_pools, nbuf))


def chunk_rows(max_pools: int, workspace_bytes: int, overlap: bool = False, tail: bool = False):
    """(rows per chunk, chunk buffers) of score_topk's chunk loop for this workspace."""
    nbuf = ctypes.c_int32(0)
    rows = lib().kpool_chunk_rows(max_pools, workspace_bytes,
                                  (KPOOL_FLAG_OVERLAP if overlap else 0) | _tail(tail), ctypes.byref(nbuf))
    _check(0 if rows >= 0 else rows, "kpool_chunk_rows")
    return int(rows), int(nbuf.value)


def pool_keys(k, cu_seqlens, cu_seqlens_dev, cu_pools_dev, kpool: int, out=None, stream=None,
              tail: bool = False):
    import torch
    _need(k, "k", 2)
    cu, cup = _host_i32(cu_seqlens)
    nseq = len(cu) - 1
    _, _, P_tot = count_pools(cu, kpool, tail)
    D = k.shape[-1]
    if out is None:
        with _on(stream):
            out = torch.empty((P_tot, D), dtype=k.dtype, device=k.device)
    rc = lib().kpool_pool_keys(_p(k), cup, _p(cu_seqlens_dev), _p(cu_pools_dev), nseq, D, kpool,
                               _tail(tail), _p(out), _stream(stream))
    _check(rc, "kpool_pool_keys")
    return out


def pool_keys_gated(k, g, ape, cu_seqlens, cu_seqlens_dev, cu_pools_dev, kpool: int, out=None,
                    stream=None, tail: bool = False):
    """Gated pooled keys: k, g bf16 [T, D] (int16 storage), ape fp32 [kpool, D]."""
    import torch
    _need(k, "k", 2)
    _need(g, "g", 2)
    _need(ape, "ape", dtype=torch.float32)
    cu, cup = _host_i32(cu_seqlens)
    nseq = len(cu) - 1
    _, _, P_tot = count_pools(cu, kpool, tail)
    D = k.shape[-1]
    if tuple(g.shape) != tuple(k.shape) or tuple(ape.shape) != (kpool, D):
        raise ValueError("need g shaped like k and ape [kpool, D]")
    if out is None:
        with _on(stream):
            out = torch.empty((P_tot, D), dtype=k.dtype, device=k.device)
    rc = lib().kpool_pool_keys_gated(_p(k), _p(g), _p(ape), cup, _p(cu_seqlens_dev), _p(cu_pools_dev),
                                     nseq, D, kpool, _tail(tail), _p(out), _stream(stream))
    _check(rc, "kpool_pool_keys_gated")
    return out


def score_topk(q, kp, w, cu_seqlens, cu_seqlens_dev, kpool: int, budget: int, q_lo: int = 0,
               q_hi: int | None = None, scale: float | None = None, workspace=None,
               pool_ids=None, scores_out=None, want_scores: bool = False, overlap: bool = False,
               stream=None, tail: bool = False):
    """Run the chunked score + top-k for rows [q_lo, q_hi).  Returns (pool_ids, scores_out).

    overlap=True passes KPOOL_FLAG_OVERLAP (two chunk buffers on two streams); a
    workspace allocated here then holds two chunk buffers, otherwise one."""
    import torch
    _need(q, "q", 2)
    _need(kp, "kp", 2)
    _need(w, "w", dtype=torch.float32)
    cu, cup = _host_i32(cu_seqlens)
    nseq = len(cu) - 1
    T = int(cu[-1])
    if q_hi is None:
        q_hi = T
    H, D = q.shape[-2], q.shape[-1]
    if scale is None:
        scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    _, max_pools, _ = count_pools(cu, kpool, tail)
    rows = max(0, q_hi - q_lo)
    with _on(stream):
        if pool_ids is None:
            pool_ids = torch.empty((rows, budget), dtype=torch.int32, device=q.device)
        if want_scores and scores_out is None:
            scores_out = torch.empty((rows, max_pools), dtype=torch.float32, device=q.device)
        if workspace is None:
            nb = workspace_bytes(q_lo, q_hi, max_pools, 2 if overlap else 1)
            workspace = torch.empty(max(nb, 16), dtype=torch.uint8, device=q.device)
    rc = lib().kpool_score_topk(_p(q), _p(kp), _p(w), cup, _p(cu_seqlens_dev), nseq, H, D, kpool,
                                ctypes.c_float(scale), q_lo, q_hi, budget, _p(workspace),
                                workspace.numel() * workspace.element_size(),
                                (KPOOL_FLAG_OVERLAP if overlap else 0) | _tail(tail), _p(pool_ids),
                                _p(scores_out), _stream(stream))
    _check(rc, "kpool_score_topk")
    return pool_ids, scores_out


def score_topk_noalloc(q, kp, w, cu_seqlens, cu_seqlens_dev, kpool: int, budget: int,
                       q_lo: int, q_hi: int, pool_ids, scores_out=None, scale: float | None = None,
                       stream=None, tail: bool = False):
    """score_topk through the library's static scratch (kpool_score_topk_noalloc): the
    caller passes every output; nothing is allocated here or in the library."""
    import torch
    _need(q, "q", 2)
    _need(kp, "kp", 2)
    _need(w, "w", dtype=torch.float32)
    cu, cup = _host_i32(cu_seqlens)
    H, D = q.shape[-2], q.shape[-1]
    if scale is None:
        scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    rc = lib().kpool_score_topk_noalloc(_p(q), _p(kp), _p(w), cup, _p(cu_seqlens_dev), len(cu) - 1,
                                        H, D, kpool, ctypes.c_float(scale), q_lo, q_hi, budget,
                                        _tail(tail), _p(pool_ids), _p(scores_out), _stream(stream))
    _check(rc, "kpool_score_topk_noalloc")
    return pool_ids, scores_out


def expand(pool_ids, cu_seqlens, cu_seqlens_dev, kpool: int, budget: int, q_lo: int = 0,
           q_hi: int | None = None, out=None, stream=None, tail: bool = False):
    """Token ids [rows, budget*kpool] (+ kpool - 1 tail slots in tail mode)."""
    import torch
    cu, cup = _host_i32(cu_seqlens)
    nseq = len(cu) - 1
    if q_hi is None:
        q_hi = int(cu[-1])
    rows = max(0, q_hi - q_lo)
    if out is None:
        with _on(stream):
            out = torch.empty((rows, budget * kpool + (kpool - 1 if tail else 0)), dtype=torch.int32,
                              device=pool_ids.device)
    rc = lib().kpool_expand(_p(pool_ids), cup, _p(cu_seqlens_dev), nseq, kpool, q_lo, q_hi, budget,
                            _tail(tail), _p(out), _stream(stream))
    _check(rc, "kpool_expand")
    return out


def topk(scores, n_valid, budget: int, out=None, stream=None):
    """Selection alone over fp32 scores [rows, ld] with n_valid int32 [rows] (device)."""
    import torch
    _need(scores, "scores", dtype=torch.float32)
    rows, ld = scores.shape
    if out is None:
        with _on(stream):
            out = torch.empty((rows, budget), dtype=torch.int32, device=scores.device)
    rc = lib().kpool_topk(_p(scores), ld, _p(n_valid), rows, budget, _p(out), _stream(stream))
    _check(rc, "kpool_topk")
    return out


def profile_enable(on: bool = True):
    _check(lib().kpool_profile_enable(1 if on else 0), "kpool_profile_enable")


def profile_collect():
    """{kind: (ms, launches)} accumulated since the last collect."""
    ms = (ctypes.c_double * 5)()
    n = (ctypes.c_int64 * 5)()
    _check(lib().kpool_profile_collect(ms, n), "kpool_profile_collect")
    return {k: (ms[i], int(n[i])) for i, k in enumerate(PROFILE_KINDS)}


# ---------------------------------------------------------------------------
# Whole path on one batch
# ---------------------------------------------------------------------------

class Selector:
    """Pool -> score/top-k -> expand for one packed batch layout (device tensors in, out).

    Holds the device copies of cu_seqlens / cu_pools and a workspace sized
    for the row range; `run` enqueues the three library calls on one stream.
    By default the workspace is one chunk buffer, so all fp32 scores in flight stay
    within the 2 GiB cap; overlap=True sizes it for two chunk buffers and runs the
    chunk loop with KPOOL_FLAG_OVERLAP (two chunks in flight on two streams);
    workspace_cap caps the workspace (smaller chunks); tail=True runs every step in
    tail mode (KPOOL_FLAG_TAIL).
    """

    def __init__(self, cu_seqlens, kpool: int, budget: int, H: int, D: int, device="cuda",
                 q_lo: int = 0, q_hi: int | None = None, workspace_cap: int | None = None,
                 scale: float | None = None, overlap: bool = False, tail: bool = False):
        import torch
        self.cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        self.T = int(self.cu[-1])
        self.kpool, self.budget, self.H, self.D = kpool, budget, H, D
        self.q_lo = q_lo
        self.q_hi = self.T if q_hi is None else q_hi
        self.overlap = overlap
        self.tail = tail
        self.cu_pools, self.max_pools, self.P_tot = count_pools(self.cu, kpool, tail)
        self.cu_dev = torch.from_numpy(self.cu).to(device)
        self.cu_pools_dev = torch.from_numpy(self.cu_pools).to(device)
        self.scale = float(np.float32(1.0) / np.sqrt(np.float32(D))) if scale is None else scale
        nb = workspace_bytes(self.q_lo, self.q_hi, self.max_pools, 2 if overlap else 1)
        if workspace_cap is not None:
            nb = min(nb, workspace_cap)
        self.workspace = torch.empty(max(nb, 16), dtype=torch.uint8, device=device)
        rows = self.q_hi - self.q_lo
        self.kp = torch.empty((self.P_tot, D), dtype=torch.int16, device=device)
        self.pool_ids = torch.empty((rows, budget), dtype=torch.int32, device=device)
        self.token_ids = torch.empty((rows, budget * kpool + (kpool - 1 if tail else 0)),
                                     dtype=torch.int32, device=device)

    @property
    def workspace_bytes(self) -> int:
        return self.workspace.numel()

    def chunk_rows(self, overlap: bool | None = None) -> int:
        """Rows per chunk of the chunk loop with this workspace (the library's plan)."""
        overlap = self.overlap if overlap is None else overlap
        return chunk_rows(self.max_pools, self.workspace_bytes, overlap, self.tail)[0]

    def chunk_buffers(self, overlap: bool | None = None) -> int:
        overlap = self.overlap if overlap is None else overlap
        return chunk_rows(self.max_pools, self.workspace_bytes, overlap, self.tail)[1]

    def run(self, q, k, w, scores_out=None, stream=None, overlap: bool | None = None, g=None,
            ape=None):
        """One pass of the path; with gate scores g and slot embeddings ape the keys are
        pooled by the gated compression, otherwise by the mean."""
        overlap = self.overlap if overlap is None else overlap
        if g is not None:
            pool_keys_gated(k, g, ape, self.cu, self.cu_dev, self.cu_pools_dev, self.kpool,
                            out=self.kp, stream=stream, tail=self.tail)
        else:
            pool_keys(k, self.cu, self.cu_dev, self.cu_pools_dev, self.kpool, out=self.kp,
                      stream=stream, tail=self.tail)
        score_topk(q, self.kp, w, self.cu, self.cu_dev, self.kpool, self.budget, self.q_lo, self.q_hi,
                   scale=self.scale, workspace=self.workspace, pool_ids=self.pool_ids,
                   scores_out=scores_out, overlap=overlap, stream=stream, tail=self.tail)
        expand(self.pool_ids, self.cu, self.cu_dev, self.kpool, self.budget, self.q_lo, self.q_hi,
               out=self.token_ids, stream=stream, tail=self.tail)
        return {"kp": self.kp, "pool_ids": self.pool_ids, "token_ids": self.token_ids}
