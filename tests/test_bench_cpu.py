"""Host-side helpers of bench.py: the visible-pair count behind `value` and the
roofline flops, and the staleness rule of the committed traffic figure."""
import os
import shutil

import numpy as np
import pytest

import bench


def brute_pairs(cu, q_lo, q_hi, kpool):
    """Count (row, pool) pairs by testing every pool of the row's sequence."""
    n = 0
    for i in range(q_lo, q_hi):
        s = int(np.searchsorted(cu, i, side="right")) - 1
        t = i - int(cu[s])
        npool = (int(cu[s + 1]) - int(cu[s]) + kpool - 1) // kpool
        n += sum(1 for p in range(npool) if p * kpool <= t)
    return n


@pytest.mark.parametrize("seed", range(4))
def test_visible_pairs_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, 40, size=rng.integers(1, 6))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    for kpool in (1, 2, 3, 4, 5):
        lo = int(rng.integers(0, T + 1))
        hi = int(rng.integers(lo, T + 1))
        assert bench.visible_pairs(cu, lo, hi, kpool) == brute_pairs(cu, lo, hi, kpool)


def test_visible_pairs_closed_forms():
    # one sequence of T tokens, kpool k: sum over t of (t // k + 1); for T = k * P that is
    # k * P (P + 1) / 2
    for T, k in ((524288, 4), (262144, 4), (524288, 1)):
        P = T // k
        assert bench.visible_pairs(np.array([0, T]), 0, T, k) == k * P * (P + 1) // 2
    # the 512k last-1/8 slice: rows [458752, 524288)
    full = bench.visible_pairs(np.array([0, 524288]), 0, 524288, 4)
    head = bench.visible_pairs(np.array([0, 524288]), 0, 458752, 4)
    assert bench.visible_pairs(np.array([0, 524288]), 458752, 524288, 4) == full - head == 8053096448


def test_traffic_figure_goes_stale_with_the_kernel(tmp_path, monkeypatch):
    """The committed FETCH/WRITE figure is used only while score.hip and api.hip hash
    to the values it was measured on."""
    prof = os.path.join(bench.ROOT, "profiles", "score_kernel_sq524288_traffic.md")
    if not os.path.exists(prof):
        pytest.skip("no committed traffic summary")
    root = tmp_path / "repo"
    (root / "profiles").mkdir(parents=True)
    shutil.copytree(os.path.join(bench.ROOT, "pool_score_top_amd", "csrc"),
                    root / "pool_score_top_amd" / "csrc")
    shutil.copy(prof, root / "profiles")
    monkeypatch.setattr(bench, "ROOT", str(root))
    t = bench.score_traffic("sq524288")
    if t is not None:  # the summary matches the sources: a changed kernel must void it
        assert t["fetch"] > 0 and t["write"] > 0
    with open(root / "pool_score_top_amd" / "csrc" / "score.hip", "a") as f:
        f.write("\n// changed\n")
    assert bench.score_traffic("sq524288") is None
    assert bench.score_traffic("no_such_workload") is None
