"""The C example (pool_score_top_amd/examples/select_file.c) on the GPU.

The example drives the whole selection through the C ABI with plain HIP runtime calls
and no framework: device buffers from hipMalloc, one stream, pool, score + select and
expand, the status of every call checked.  Its pool and token ids must equal those of
the Python binding on the same inputs bit for bit, and on the tiny workload also the
oracle's, so the ABI gives the same results without torch in the process.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
from gpu_helpers import run_gpu
from pool_score_top_amd import build as B
from pool_score_top_amd import synth

pytestmark = pytest.mark.gpu

# (workload, overrides, cu_seqlens or None for the workload's own)
CASES = [
    ("tiny", {}, None),
    ("sq4096", {"T": 3000, "budget": 64}, [0, 1100, 1100, 3000]),
    ("sq4096", {"T": 2500, "kpool": 1, "budget": 1025}, [0, 700, 2500]),
    ("sq4096", {"T": 2048, "kpool": 3, "budget": 513}, None),
]


def _write_input(path, wl, r, cu):
    with open(path, "wb") as f:
        np.array([wl.T, wl.H, wl.D, wl.kpool, wl.budget, len(cu) - 1], dtype="<i4").tofile(f)
        np.asarray(cu, dtype="<i4").tofile(f)
        np.ascontiguousarray(r["q"], dtype="<u2").tofile(f)
        np.ascontiguousarray(r["k"], dtype="<u2").tofile(f)
        np.ascontiguousarray(r["w"], dtype="<f4").tofile(f)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_c_example_matches_the_binding(case, tmp_path):
    assert os.path.exists(B.EXAMPLE), f"{B.EXAMPLE} is not built; run __graft_entry__.build()"
    name, over, cu = CASES[case]
    wl = synth.workload(name, **over)
    r = synth.host_inputs(wl, 500 + case)
    if cu is not None:
        r["cu_seqlens"] = np.asarray(cu, dtype=np.int32)
    cu = np.asarray(r["cu_seqlens"], dtype=np.int32)
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    _write_input(src, wl, r, cu)
    print(f"[c example] case {case}: {name} {over} nseq={len(cu) - 1}", flush=True)
    p = subprocess.run([B.EXAMPLE, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert p.returncode == 0, p.stderr
    out = np.fromfile(dst, dtype="<i4")
    n_ids = wl.T * wl.budget
    assert out.size == n_ids + n_ids * wl.kpool
    ids = out[:n_ids].reshape(wl.T, wl.budget)
    tok = out[n_ids:].reshape(wl.T, wl.budget * wl.kpool)
    ref = run_gpu(r, wl.kpool, wl.budget, want_scores=False, overlap=False)
    np.testing.assert_array_equal(ids, ref["pool_ids"])
    np.testing.assert_array_equal(tok, ref["token_ids"])
    if name == "tiny":
        o = oracle.select(r["q"], r["k"], r["w"], cu, wl.kpool, wl.budget)
        np.testing.assert_array_equal(ids, o["pool_ids"])
        np.testing.assert_array_equal(tok, o["token_ids"])
