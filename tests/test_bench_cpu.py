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


def _fake_repo(tmp_path, with_hashes=True):
    import hashlib
    root = tmp_path / "repo"
    (root / "profiles").mkdir(parents=True)
    csrc = root / "pool_score_top_amd" / "csrc"
    shutil.copytree(os.path.join(bench.ROOT, "pool_score_top_amd", "csrc"), csrc)
    lines = ["# counters", "```"]
    for name in bench.COUNTER_SOURCES:
        sha = hashlib.sha256((csrc / name).read_bytes()).hexdigest() if with_hashes else "0" * 64
        lines.append(f"sha256_{name}: {sha}")
    lines += ["score_fetch_bytes_per_launch: 341156430", "score_write_bytes_per_launch: 1174277950",
              "score_mfma_busy_frac: 0.716", "topk_fetch_bytes_per_launch: 404000000",
              "topk_write_bytes_per_launch: 8400000", "```"]
    (root / "profiles" / "counters_sqX.md").write_text("\n".join(lines) + "\n")
    return root


def test_counter_figures_go_stale_with_the_sources(tmp_path, monkeypatch):
    """Committed counter figures are used only while score.hip, topk.hip and api.hip hash
    to the values they were measured on."""
    root = _fake_repo(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(root))
    c = bench.committed_counters("sqX")
    assert c["score_fetch_bytes_per_launch"] == 341156430 and c["topk_write_bytes_per_launch"] == 8.4e6
    assert c["score_mfma_busy_frac"] == 0.716
    assert bench.committed_counters("no_such_workload") is None
    for name in bench.COUNTER_SOURCES:
        f = root / "pool_score_top_amd" / "csrc" / name
        orig = f.read_bytes()
        f.write_bytes(orig + b"\n// changed\n")
        assert bench.committed_counters("sqX") is None, name
        f.write_bytes(orig)
    assert bench.committed_counters("sqX") is not None


def test_counter_figures_with_wrong_hashes_are_ignored(tmp_path, monkeypatch):
    root = _fake_repo(tmp_path, with_hashes=False)
    monkeypatch.setattr(bench, "ROOT", str(root))
    assert bench.committed_counters("sqX") is None
