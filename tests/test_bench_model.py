"""CPU tests of the work model bench.py prices its rooflines with, and of the
guard that keeps stale traffic counters out of the bench line.

The closed forms for the number of (query, key) pairs in the selected
supports and of valid (query, block) slots are checked against brute force
over the oracle's own supports, on selections drawn at random (the count is
the same for every selection that keeps the query's own block and picks
other blocks only among the visible ones), and against the totals per
(batch, head) that follow from the same definitions at the full sizes."""

import json
import os

import numpy as np
import pytest

import bench
import msa_inputs
from oracle import msa_oracle as O


def _random_selection(N, block, topk, rng):
    """A valid causal selection per query: its own block plus up to topk-1
    other visible blocks chosen at random, padded with -1."""
    nblk = N // block
    sel = np.full((N, topk), -1, dtype=np.int64)
    for t in range(N):
        own = t // block
        others = rng.permutation(own)[: min(topk - 1, own)]
        row = np.sort(np.concatenate([[own], others]))
        sel[t, : len(row)] = row
        assert row.max() < nblk
    return sel


@pytest.mark.parametrize("N,block,topk", [(128, 128, 4), (640, 128, 1), (1024, 128, 3), (1152, 128, 16),
                                          (512, 64, 5)])
def test_support_pairs_and_slots_match_brute_force(N, block, topk):
    rng = np.random.default_rng(N + topk)
    sel = _random_selection(N, block, topk, rng)
    pairs = sum(len(O.support(sel[t], t, N, block, True)) for t in range(N))
    slots = int((sel >= 0).sum())
    assert bench.support_pairs(N, block, topk) == pairs
    assert bench.valid_slots(N, block, topk) == slots


@pytest.mark.parametrize("N,topk,expect", [(1024, 4, 3.61e5), (8192, 16, 1.429e7), (131072, 16, 2.581e8),
                                           (1048576, 16, 2.079e9)])
def test_support_pairs_full_sizes(N, topk, expect):
    # Totals of |S(t)| per (batch, head) at the four workload lengths, to the
    # four significant figures they are quoted with.
    got = bench.support_pairs(N, 128, topk)
    assert abs(got - expect) / expect < 5e-4, got


def test_headline_work_per_launch():
    # fwd+bwd at N = 128K, 64/8 heads, d = 128, d_idx = 64: the flop counts the
    # bench line divides by the measured launch time.
    w = msa_inputs.WORKLOADS["fwdbwd-bf16-n128k"]
    work = bench.algorithmic_work(w)
    pairs = bench.support_pairs(w.N, 128, 16)
    assert work["fwd_partial"] == ("flop", 4.0 * 128 * pairs * 64)
    assert work["bwd_main"][1] == pytest.approx((10.0 * 128 * 64 + 6.0 * 64 * 8) * pairs)
    assert work["index_topk"][1] == pytest.approx(2.0 * 64 * 8 * w.N * (w.N + 1) / 2)
    assert work["bwd_main"][1] == pytest.approx(2.194e13, rel=1e-3)
    assert work["fwd_partial"][1] == pytest.approx(8.46e12, rel=1e-3)


def test_stale_traffic_counters_are_not_reported(tmp_path, monkeypatch):
    rec = {"kernel": "bwd_main", "workload": "w", "source_sha256": bench.source_sha("bwd_main"),
           "bytes_per_launch": 123.0}
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic_bwd_main_w.json").write_text(json.dumps(rec))
    # ROOT locates both the profiles and the kernel sources: point it at a
    # temporary tree that holds copies of the two hashed sources.
    real_root = bench.ROOT
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    csrc = tmp_path / "block_sparse_attention_branch_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in ("sparse_bwd.hip", "msa_internal.h"):
        (csrc / name).write_bytes(open(os.path.join(real_root, "block_sparse_attention_branch_amd", "csrc",
                                                    name), "rb").read())
    assert bench.measured_traffic("bwd_main", "w") == 123.0
    # Any change to the kernel's source or the shared header voids the record.
    with open(csrc / "msa_internal.h", "ab") as f:
        f.write(b"\n// changed\n")
    assert bench.measured_traffic("bwd_main", "w") is None
    assert bench.measured_traffic("bwd_main", "absent") is None
