"""The C ABI without a GPU: the library loads, exports what include/kpool.h
declares, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import numpy as np
import pytest

from pool_score_top_amd import kpool as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kpool.h")

pytestmark = pytest.mark.skipif(not os.path.exists(K.LIB_PATH), reason="libkpool.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kpool_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("kpool_pool_keys", "kpool_score_topk", "kpool_expand", "kpool_topk",
                 "kpool_count_pools", "kpool_workspace_bytes", "kpool_last_error"):
        assert must in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(K.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing


def test_no_process_wide_switch_in_the_header():
    """Every setting is an argument of the call: the header declares no setter."""
    names = declared_functions()
    assert not [n for n in names if "set_" in n], names
    assert K.version() == 300


def test_count_pools_and_workspace():
    cu_pools, mx, tot = K.count_pools([0, 9, 9, 37], 4)
    assert cu_pools.tolist() == [0, 3, 3, 10] and mx == 7 and tot == 10
    # tail mode: full pools only (9 -> 2, 28 -> 7, a 3-token sequence -> none)
    cu_pools, mx, tot = K.count_pools([0, 9, 9, 37, 40], 4, tail=True)
    assert cu_pools.tolist() == [0, 2, 2, 9, 9] and mx == 7 and tot == 9
    # 512k tokens, kpool 4: pitch 131072 floats = 512 KiB per row -> 4096 rows per 2 GiB chunk,
    # plus one fp32 group maximum per 16 pools of each row; two chunk buffers when the
    # range needs more than one chunk
    assert K.workspace_bytes(0, 524288, 131072) == 2 * 4096 * (131072 + 8192) * 4
    assert K.workspace_bytes(0, 524288, 131072, 1) == 4096 * (131072 + 8192) * 4
    assert K.workspace_bytes(0, 6000, 131072) == 6000 * (131072 + 8192) * 4
    assert K.workspace_bytes(0, 6000, 131072, 1) == 4096 * (131072 + 8192) * 4
    assert K.workspace_bytes(0, 100, 131072) == 100 * (131072 + 8192) * 4
    assert K.workspace_bytes(5, 5, 10) == 0
    assert K.workspace_bytes(0, 3, 1) == 3 * (64 + 4) * 4   # pitch rounds up to 64
    assert K.workspace_bytes(0, 3, 1, 0) == 0 and K.workspace_bytes(0, 3, 1, 3) == 0


@pytest.mark.parametrize("max_pools", [1, 63, 64, 65, 7000, 131072, 262144])
@pytest.mark.parametrize("ws", [272, 4 << 20, 1 << 31, (1 << 32) + 12345, 40 << 30])
@pytest.mark.parametrize("overlap", [False, True])
def test_chunk_plan_properties(max_pools, ws, overlap):
    """The chunk plan: whole 64-float score rows plus one group maximum per 16 pools,
    each chunk's fp32 scores within 2 GiB, all chunk buffers within the workspace, and
    no room for one more row under either limit."""
    pitch = (max_pools + 63) // 64 * 64
    row = (pitch + pitch // 16) * 4
    if ws < row:
        with pytest.raises(K.KpoolError):
            K.chunk_rows(max_pools, ws, overlap)
        return
    rows, nbuf = K.chunk_rows(max_pools, ws, overlap)
    assert nbuf == (2 if overlap and ws >= 2 * row else 1)
    assert rows >= 1 and rows * pitch * 4 <= 1 << 31 and nbuf * rows * row <= ws
    assert (rows + 1) * pitch * 4 > 1 << 31 or nbuf * (rows + 1) * row > ws
    # the tail flag does not change the plan for the same pool count
    assert K.chunk_rows(max_pools, ws, overlap, tail=True) == (rows, nbuf)


def test_chunk_plan_rejects():
    L = K.lib()
    assert L.kpool_chunk_rows(0, 1 << 20, 0, None) == K.KPOOL_EINVAL
    assert L.kpool_chunk_rows(10, 1 << 20, 4, None) == K.KPOOL_EINVAL
    assert L.kpool_chunk_rows(10, 271, 0, None) == K.KPOOL_EWORKSPACE
    assert L.kpool_chunk_rows(10, 272, 0, None) == 1


def _call_score(**kw):
    L = K.lib()
    cu = np.array(kw.pop("cu", [0, 64]), dtype=np.int32)
    args = dict(q=16, kp=16, w=16, cu_dev=16, nseq=len(cu) - 1, H=4, D=16, kpool=4, scale=0.25,
                q_lo=0, q_hi=int(cu[-1]), budget=4, ws=16, ws_bytes=1 << 20, flags=0, ids=16)
    args.update(kw)
    vp = ctypes.c_void_p
    return L.kpool_score_topk(vp(args["q"]), vp(args["kp"]), vp(args["w"]),
                              cu.ctypes.data_as(vp), vp(args["cu_dev"]), args["nseq"], args["H"],
                              args["D"], args["kpool"], ctypes.c_float(args["scale"]), args["q_lo"],
                              args["q_hi"], args["budget"], vp(args["ws"]), args["ws_bytes"],
                              args["flags"], vp(args["ids"]), None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q_lo=5, q_hi=4), K.KPOOL_EINVAL),
    (dict(q_hi=65), K.KPOOL_EINVAL),
    (dict(q_lo=-1), K.KPOOL_EINVAL),
    (dict(budget=0), K.KPOOL_EINVAL),
    (dict(budget=2049), K.KPOOL_EINVAL),
    (dict(kpool=0), K.KPOOL_EINVAL),
    (dict(scale=0.0), K.KPOOL_EINVAL),
    (dict(scale=float("nan")), K.KPOOL_EINVAL),
    (dict(H=8), K.KPOOL_EUNSUPPORTED),
    (dict(D=64), K.KPOOL_EUNSUPPORTED),
    (dict(q=0), K.KPOOL_EINVAL),
    (dict(q=8), K.KPOOL_EINVAL),            # misaligned
    (dict(ws=0), K.KPOOL_EWORKSPACE),
    (dict(ws_bytes=100), K.KPOOL_EWORKSPACE),  # less than one 272-byte workspace row
    (dict(cu=[1, 64]), K.KPOOL_EINVAL),
    (dict(cu=[0, 40, 30, 64]), K.KPOOL_EINVAL),
    (dict(nseq=0), K.KPOOL_EINVAL),
    (dict(flags=4), K.KPOOL_EINVAL),         # unknown flag bit (1 overlap, 2 tail)
    (dict(flags=0x80000001), K.KPOOL_EINVAL),
    # one sequence whose pooled keys exceed the kernel's 32-bit byte offsets (2^24 pools at D=128)
    (dict(cu=[0, 1 << 24], kpool=1, H=32, D=128), K.KPOOL_EUNSUPPORTED),
])
def test_score_topk_rejects_bad_arguments(kw, code):
    rc = _call_score(**kw)
    assert rc == code
    assert K.lib().kpool_last_error().decode()


def test_empty_range_is_a_noop_without_pointers():
    assert _call_score(q_lo=10, q_hi=10, q=0, kp=0, w=0, ws=0, ids=0) == K.KPOOL_OK


def test_other_entry_points_reject_bad_arguments():
    L = K.lib()
    vp = ctypes.c_void_p
    cu = np.array([0, 64], dtype=np.int32)
    cup = cu.ctypes.data_as(vp)
    assert L.kpool_pool_keys(vp(16), cup, vp(16), vp(16), 1, 12, 4, 0, vp(16), None) == K.KPOOL_EINVAL
    assert L.kpool_pool_keys(vp(16), cup, vp(16), vp(16), 1, 16, 0, 0, vp(16), None) == K.KPOOL_EINVAL
    assert L.kpool_pool_keys(None, cup, vp(16), vp(16), 1, 16, 4, 0, vp(16), None) == K.KPOOL_EINVAL
    assert L.kpool_pool_keys(vp(16), cup, vp(16), vp(16), 1, 16, 4, 1, vp(16), None) == K.KPOOL_EINVAL  # flag
    assert L.kpool_expand(vp(16), cup, vp(16), 1, 4, 3, 2, 4, 0, vp(16), None) == K.KPOOL_EINVAL
    assert L.kpool_expand(vp(16), cup, vp(16), 1, 4, 0, 65, 4, 0, vp(16), None) == K.KPOOL_EINVAL
    assert L.kpool_expand(None, cup, vp(16), 1, 4, 0, 64, 4, 0, vp(16), None) == K.KPOOL_EINVAL
    assert L.kpool_expand(vp(16), cup, vp(16), 1, 4, 0, 64, 4, 0, vp(8), None) == K.KPOOL_EINVAL
    assert L.kpool_expand(vp(16), cup, vp(16), 1, 4, 0, 64, 4, 1, vp(16), None) == K.KPOOL_EINVAL   # flag
    assert L.kpool_topk(vp(16), 6, vp(16), 3, 4, vp(16), None) == K.KPOOL_EINVAL      # ld % 4
    assert L.kpool_topk(vp(16), 8, vp(16), 3, 0, vp(16), None) == K.KPOOL_EINVAL      # budget
    assert L.kpool_topk(vp(8), 8, vp(16), 3, 4, vp(16), None) == K.KPOOL_EINVAL       # alignment
    assert L.kpool_topk(None, 8, vp(16), 0, 4, None, None) == K.KPOOL_OK              # no rows
    assert L.kpool_count_pools(cup, 1, 0, 0, None, None) == K.KPOOL_EINVAL
    assert L.kpool_count_pools(cup, 1, 4, 1, None, None) == K.KPOOL_EINVAL           # overlap flag
    assert L.kpool_count_pools(cup, 1, 4, 2, None, None) == 16                        # tail: 64 // 4


def test_gated_pool_keys_rejects_bad_arguments():
    L = K.lib()
    vp = ctypes.c_void_p
    cu = np.array([0, 64], dtype=np.int32)
    cup = cu.ctypes.data_as(vp)
    ok = dict(k=16, g=16, ape=16, cud=16, cpd=16, D=16, kpool=4, flags=0, kp=16)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return L.kpool_pool_keys_gated(vp(a["k"]), vp(a["g"]), vp(a["ape"]), cup, vp(a["cud"]),
                                       vp(a["cpd"]), 1, a["D"], a["kpool"], a["flags"], vp(a["kp"]), None)
    for kw in (dict(g=0), dict(ape=0), dict(k=0), dict(kp=0), dict(g=8), dict(ape=4), dict(D=12),
               dict(kpool=0), dict(flags=1)):
        assert call(**kw) == K.KPOOL_EINVAL, kw
        assert K.lib().kpool_last_error().decode()
    # an empty batch needs no pointers
    cu0 = np.array([0, 0], dtype=np.int32)
    assert L.kpool_pool_keys_gated(None, None, None, cu0.ctypes.data_as(vp), None, None, 1, 16, 4, 0,
                                   None, None) == K.KPOOL_OK


C_USER = r"""
#include <stdio.h>
#include <stdlib.h>
#include "kpool.h"

/* the call sequence of one pass, as a C caller writes it (type-checked, not run) */
int one_pass(const uint16_t *q, const uint16_t *k, const float *w, const int32_t *cu_host,
             const int32_t *cu_dev, const int32_t *cu_pools_dev, int32_t nseq, int64_t T,
             uint16_t *kp, void *workspace, int32_t *pool_ids, float *scores, int32_t *token_ids,
             void *stream) {
  int32_t cu_pools_host[64];
  int32_t max_pools = 0;
  int32_t nbuf = 0;
  int64_t P = kpool_count_pools(cu_host, nseq, 4, 0, cu_pools_host, &max_pools);
  if (P < 0) return (int)P;
  int rc = kpool_pool_keys(k, cu_host, cu_dev, cu_pools_dev, nseq, 128, 4, 0, kp, stream);
  if (rc != KPOOL_OK) { fprintf(stderr, "%s\n", kpool_last_error()); return rc; }
  size_t ws = kpool_workspace_bytes(0, T, max_pools, 1);
  int64_t rows = kpool_chunk_rows(max_pools, ws, 0, &nbuf);
  (void)rows;
  rc = kpool_score_topk(q, kp, w, cu_host, cu_dev, nseq, 32, 128, 4, 0.08838835f, 0, T, 512,
                        workspace, ws, 0, pool_ids, scores, stream);
  if (rc != KPOOL_OK) return rc;
  rc = kpool_score_topk_noalloc(q, kp, w, cu_host, cu_dev, nseq, 32, 128, 4, 0.08838835f, 0, T,
                                512, KPOOL_FLAG_TAIL, pool_ids, NULL, stream);
  if (rc != KPOOL_OK) return rc;
  rc = kpool_expand(pool_ids, cu_host, cu_dev, nseq, 4, 0, T, 512, 0, token_ids, stream);
  if (rc != KPOOL_OK) return rc;
  rc = kpool_pool_keys_gated(k, k, w, cu_host, cu_dev, cu_pools_dev, nseq, 128, 4,
                             KPOOL_FLAG_TAIL, kp, stream);
  if (rc != KPOOL_OK) return rc;
  rc = kpool_topk(scores, 64, cu_dev, T, 512, pool_ids, stream);
  double ms[KPOOL_PROFILE_KINDS];
  int64_t launches[KPOOL_PROFILE_KINDS];
  kpool_profile_enable(1);
  kpool_profile_collect(ms, launches);
  return rc + kpool_version() * 0 + (int)KPOOL_NOALLOC_SCRATCH_BYTES * 0 + (int)KPOOL_FLAG_OVERLAP * 0;
}
"""


def test_header_is_plain_c_and_the_call_sequence_type_checks(tmp_path):
    """include/kpool.h is a C header (the boundary is a C ABI): a C99 caller that makes
    every call compiles with warnings as errors (syntax and types only; nothing is run)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = tmp_path / "user.c"
    src.write_text(C_USER)
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-fsyntax-only",
                        "-I", os.path.dirname(HEADER), str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_c_example_is_built_and_rejects_bad_usage(tmp_path):
    # the C example over the ABI (examples/select_file.c); these paths return before any
    # HIP call, so they run without a GPU
    import subprocess
    from pool_score_top_amd import build as B
    assert os.path.exists(B.EXAMPLE), "the C example is not built; run __graft_entry__.build()"
    p = subprocess.run([B.EXAMPLE], capture_output=True, text=True, timeout=60)
    assert p.returncode == 2 and "usage" in p.stderr
    short = tmp_path / "short.bin"
    np.array([64, 4, 16, 4, 4, 1, 0, 64], dtype="<i4").tofile(short)  # header and cu_seqlens only
    p = subprocess.run([B.EXAMPLE, str(short), str(tmp_path / "out.bin")], capture_output=True, text=True,
                       timeout=60)
    assert p.returncode == 2 and "short input" in p.stderr
