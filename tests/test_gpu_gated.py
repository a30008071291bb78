"""GPU parity of the gated k-pool compression (kpool_pool_keys_gated) and of the
whole path on gated pooled keys, through the C ABI, against the oracle.

The formula is a reading of the pages (they name the gate and the slot
embedding but print no formula), so parity against the pages' own operator is
unpinned; the oracle's reading is pinned on the CPU (test_oracle_gated.py).
The kernel and the oracle both compute in fp64: the GPU's bf16 keys must equal
the oracle's rounding except where the oracle's value lies within the fp64
error bound (about 1e-14 relative) of a bf16 rounding midpoint, where either
neighbour is accepted (gpu_helpers.gated_allowed; the count is printed and is
zero for these inputs).  Scores, pool ids
and token ids then follow the rules of the other parity tests, against the
oracle run on the oracle's own gated keys.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (check_gated_keys, check_scores, check_selection_vs_oracle, check_tokens,
                         check_topk_self, device_tensors, report)
from pool_score_top_amd import kpool as K
from pool_score_top_amd import synth

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _gpu_gated_keys(k_bits, g_bits, ape, cu, kpool):
    cu = np.asarray(cu, dtype=np.int32)
    cu_pools, _, _ = K.count_pools(cu, kpool)
    k = torch.from_numpy(np.ascontiguousarray(k_bits).view(np.int16)).cuda()
    g = torch.from_numpy(np.ascontiguousarray(g_bits).view(np.int16)).cuda()
    a = torch.from_numpy(np.ascontiguousarray(ape, dtype=np.float32)).cuda()
    kp = K.pool_keys_gated(k, g, a, cu, torch.from_numpy(cu).cuda(), torch.from_numpy(cu_pools).cuda(),
                           kpool)
    torch.cuda.synchronize()
    return kp.cpu().numpy().view(np.uint16)


def test_gated_hand_values():
    with open(os.path.join(GOLDEN, "gated_pins.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        k = np.repeat(np.array([int(x, 16) for x in c["keys"]], np.uint16)[:, None], 8, axis=1)
        g = np.repeat(np.array([int(x, 16) for x in c["gates"]], np.uint16)[:, None], 8, axis=1)
        ape = np.repeat(np.array(c["ape"], np.float32)[:, None], 8, axis=1)
        cu = [0, len(k)]
        got = _gpu_gated_keys(k, g, ape, cu, c["kpool"])
        bits, vals = oracle.pool_keys_gated(k, g, ape, cu, c["kpool"], return_values=True)
        check_gated_keys(got, vals, k, g, ape, cu, c["kpool"], where=c["name"])
        # the hand values themselves, the two keys 2^-40 off a midpoint included
        want = np.repeat(np.array([int(x, 16) for x in c["pooled"]], np.uint16)[:, None], 8, axis=1)
        np.testing.assert_array_equal(got, want, err_msg=c["name"])


@pytest.mark.parametrize("name,seed", [("tiny_gated", 0), ("sq4096_gated", 1), ("thd65536_gated", 2)])
def test_gated_pool_keys_workloads(name, seed):
    wl = synth.workload(name)
    r = synth.host_inputs(wl, seed)
    cu = r["cu_seqlens"]
    got = _gpu_gated_keys(r["k"], r["g"], r["ape"], cu, wl.kpool)
    _, vals = oracle.pool_keys_gated(r["k"], r["g"], r["ape"], cu, wl.kpool, return_values=True)
    st = check_gated_keys(got, vals, r["k"], r["g"], r["ape"], cu, wl.kpool, where=name)
    report(name, gated_keys=st)
    np.testing.assert_array_equal(got, oracle.f64_to_bf16_rne(vals))   # no key near a midpoint here


@pytest.mark.parametrize("kpool", [1, 2, 3, 5, 8])
def test_gated_pool_keys_other_pool_sizes(kpool):
    wl = synth.workload("tiny_gated", T=203, D=16, kpool=kpool)
    r = synth.host_inputs(wl, 30 + kpool)
    cu = np.array([0, 1, 50, 50, 203], dtype=np.int32)
    got = _gpu_gated_keys(r["k"], r["g"], r["ape"], cu, kpool)
    _, vals = oracle.pool_keys_gated(r["k"], r["g"], r["ape"], cu, kpool, return_values=True)
    check_gated_keys(got, vals, r["k"], r["g"], r["ape"], cu, kpool, where=f"kpool {kpool}")
    if kpool == 1:     # one slot: weight 1, the keys themselves
        np.testing.assert_array_equal(got, r["k"])


def test_gated_large_gates_do_not_overflow():
    """Gate scores and embeddings near +-1000 (exp would overflow without the max shift)."""
    wl = synth.workload("tiny_gated", T=100, D=16, kpool=4)
    r = synth.host_inputs(wl, 5)
    g = oracle.f32_to_bf16_rne(oracle.bf16_to_f32(r["g"]) * np.float32(300.0))
    ape = (r["ape"] * np.float32(300.0)).astype(np.float32)
    cu = np.array([0, 37, 100], dtype=np.int32)
    got = _gpu_gated_keys(r["k"], g, ape, cu, 4)
    assert np.all(np.isfinite(oracle.bf16_to_f32(got)))
    _, vals = oracle.pool_keys_gated(r["k"], g, ape, cu, 4, return_values=True)
    check_gated_keys(got, vals, r["k"], g, ape, cu, 4, where="large gates")


@pytest.mark.parametrize("name,seed", [("tiny_gated", 0), ("tiny_gated", 3), ("sq4096_gated", 4)])
def test_gated_whole_path(name, seed):
    wl = synth.workload(name)
    r = synth.host_inputs(wl, seed)
    cu = r["cu_seqlens"]
    q, k, w = device_tensors(r)
    g = torch.from_numpy(r["g"].view(np.int16)).cuda()
    ape = torch.from_numpy(r["ape"]).cuda()
    sel = K.Selector(cu, wl.kpool, wl.budget, wl.H, wl.D)
    scores = torch.empty((wl.T, sel.max_pools), dtype=torch.float32, device="cuda")
    out = sel.run(q, k, w, scores_out=scores, g=g, ape=ape)
    torch.cuda.synchronize()
    kp_bits, vals = oracle.pool_keys_gated(r["k"], r["g"], r["ape"], cu, wl.kpool, return_values=True)
    st_k = check_gated_keys(out["kp"].cpu().numpy().view(np.uint16), vals, r["k"], r["g"], r["ape"],
                            cu, wl.kpool, where=name)
    ref = oracle.select(r["q"], r["k"], r["w"], cu, wl.kpool, wl.budget, kp_bits=kp_bits)
    rows = np.arange(wl.T)
    _, t = oracle.row_positions(rows, cu)
    nvis = t // wl.kpool + 1
    gs = scores.cpu().numpy()
    ids = out["pool_ids"].cpu().numpy()
    st_s = check_scores(gs, ref["scores"], nvis, name)
    check_topk_self(gs, ids, nvis, wl.budget, name)
    st_sel = check_selection_vs_oracle(ids, ref["scores"], nvis, wl.budget, name)
    check_tokens(out["token_ids"].cpu().numpy(), ids, t, wl.kpool, ref["pool_ids"], ref["token_ids"],
                 where=name)
    report(f"{name} seed {seed} (gated)", gated_keys=st_k, scores=st_s, selection=st_sel)
