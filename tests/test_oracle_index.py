"""Pins of the oracle's index branch (scores, block max-pool, top-k) against
things other than itself: hand-derived values, pure-Python integer brute
force, brute-force sorting, special cases and the planted closed form.

Pages: "How to solve the memory problem with MiniMax Sparse Attention"
('How the indexer works', 'Two-stage process', 'Kernel optimizations');
"How Flash-MSA cuts million-token training cost with sparse-k"
('Block sparsity mechanism')."""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import msa_oracle as O
import msa_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f(x):
    return -math.inf if x == "-inf" else float(x)


def test_hand_example_index():
    fx = json.load(open(os.path.join(GOLDEN, "index_hand_example.json")))
    kvals = [3, -1, 2, 0, -2, 5, 1, 1]
    N, bs = 8, 2
    for case in fx["cases"]:
        q_idx = np.full((1, N, 1, 1), float(case["q"]))
        k_idx = np.array(kvals, dtype=np.float64).reshape(1, N, 1)
        sel, pooled = O.index_topk(q_idx, k_idx, bs, case["topk"], causal=True,
                                   rows=[(0, case["t"])], want_pooled=True)
        assert sel[0, 0].tolist() == case["block_idx"], case
        assert [float(x) for x in pooled[0, 0]] == [_f(x) for x in case["pooled"]], case


def _brute_scores_int(qi, ki, b, t, g, causal):
    """Pure-Python integer dot products (exact)."""
    N = ki.shape[1]
    last = t if causal else N - 1
    return {u: sum(int(a) * int(c) for a, c in zip(qi[b, t, g], ki[b, u])) for u in range(last + 1)}


def _brute_select(scores, t, N, bs, topk, causal):
    nb = (N + bs - 1) // bs
    pooled = {}
    for u, s in scores.items():
        j = u // bs
        pooled[j] = max(pooled.get(j, -math.inf), s)
    own = t // bs
    others = sorted((j for j in pooled if j != own), key=lambda j: (-pooled[j], j))
    sel = sorted([own] + others[: topk - 1])
    return sel + [-1] * (topk - len(sel)), pooled, nb


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("topk", [1, 2, 3, 5])
def test_integer_brute_force(causal, topk):
    rng = np.random.default_rng(7 + topk)
    B, N, H_kv, d_idx, bs = 2, 37, 2, 3, 4          # ragged last block
    qi = rng.integers(-2, 3, size=(B, N, H_kv, d_idx))
    ki = rng.integers(-2, 3, size=(B, N, d_idx))
    sel, pooled = O.index_topk(qi.astype(np.float64), ki.astype(np.float64), bs, topk,
                               causal=causal, want_pooled=True)
    for b in range(B):
        for t in range(N):
            for g in range(H_kv):
                sc = _brute_scores_int(qi, ki, b, t, g, causal)
                exp_sel, exp_pool, nb = _brute_select(sc, t, N, bs, topk, causal)
                assert sel[b, t, g].tolist() == exp_sel, (b, t, g)
                for j in range(nb):
                    assert pooled[b, t, g, j] == exp_pool.get(j, -math.inf)


def test_special_cases_k_covers_all_and_k1():
    rng = np.random.default_rng(3)
    B, N, H_kv, d_idx, bs = 1, 64, 1, 4, 8
    qi = rng.standard_normal((B, N, H_kv, d_idx))
    ki = rng.standard_normal((B, N, d_idx))
    nb = N // bs
    sel_all = O.index_topk(qi, ki, bs, nb, causal=True)
    sel_one = O.index_topk(qi, ki, bs, 1, causal=True)
    for t in range(N):
        own = t // bs
        assert sel_all[0, t, 0].tolist() == list(range(own + 1)) + [-1] * (nb - own - 1)
        assert sel_one[0, t, 0].tolist() == [own]


def test_own_block_forced_even_when_worst():
    # Own block gets the lowest score; it is kept anyway.
    N, bs, topk = 16, 4, 2
    ki = np.zeros((1, N, 1))
    ki[0, :12, 0] = 5.0
    ki[0, 12:, 0] = -9.0
    qi = np.ones((1, N, 1, 1))
    sel = O.index_topk(qi, ki, bs, topk, causal=True, rows=[(0, 15)])
    assert sel[0, 0].tolist() == [0, 3]       # tie among B0..B2 -> B0, plus own B3


def test_alternative_forcing_reading_agrees():
    """'own + top-(k-1) of others' equals 'top-k of all, and if own is missing
    replace the lowest pick with own' under the same (score desc, index asc)
    order."""
    rng = np.random.default_rng(11)
    B, N, H_kv, d_idx, bs, topk = 1, 96, 2, 3, 8, 4
    qi = rng.integers(-2, 3, size=(B, N, H_kv, d_idx)).astype(np.float64)
    ki = rng.integers(-2, 3, size=(B, N, d_idx)).astype(np.float64)
    sel, pooled = O.index_topk(qi, ki, bs, topk, causal=True, want_pooled=True)
    for t in range(N):
        for g in range(H_kv):
            own = t // bs
            vis = list(range(own + 1))
            order = sorted(vis, key=lambda j: (-pooled[0, t, g, j], j))
            pick = order[:topk]
            if own not in pick:
                pick = pick[:-1] + [own]
            exp = sorted(pick) + [-1] * (topk - len(pick))
            assert sel[0, t, g].tolist() == exp


def test_exp_free_selection_matches_softmax_selection():
    """Selecting on softmax-transformed pooled scores (any positive temperature)
    picks the same blocks as selecting on the raw pooled scores, because exp
    and normalisation are strictly increasing ('Kernel optimizations')."""
    rng = np.random.default_rng(5)
    B, N, H_kv, d_idx, bs, topk = 1, 128, 1, 8, 8, 4
    qi = rng.standard_normal((B, N, H_kv, d_idx))
    ki = rng.standard_normal((B, N, d_idx))
    sel, pooled = O.index_topk(qi, ki, bs, topk, causal=True, want_pooled=True)
    for t in range(N):
        p = pooled[0, t, 0]
        vis = np.isfinite(p)
        z = np.where(vis, 0.3 * p, -np.inf)
        sm = np.exp(z - z[vis].max())
        sm = sm / sm.sum()
        sel2 = O.select_blocks_row(np.where(vis, sm, -np.inf), t, bs, topk, True)
        assert sel2.tolist() == sel[0, t, 0].tolist()


def test_selection_shared_by_group_heads_and_budget():
    """k blocks per query at most, a budget of k*bs tokens: with bs=128 and
    k=16 the budget is 2048 tokens ('Two-stage process')."""
    fx = json.load(open(os.path.join(GOLDEN, "budget.json")))
    for row in fx["support_sizes"]:
        assert O.support_size(row["t"], fx["block_size"], fx["topk"]) == row["size"]
    assert fx["block_size"] * fx["topk"] == fx["budget_tokens"]
    # brute force the support size on a small causal selection
    rng = np.random.default_rng(2)
    N, bs, topk = 200, 8, 5
    qi = rng.standard_normal((1, N, 1, 4))
    ki = rng.standard_normal((1, N, 4))
    sel = O.index_topk(qi, ki, bs, topk, causal=True)
    for t in range(N):
        S = O.support(sel[0, t, 0], t, N, bs, True)
        brute = [u for u in range(t + 1) if (u // bs) in set(sel[0, t, 0].tolist())]
        assert S.tolist() == brute
        assert len(brute) == O.support_size(t, bs, topk)


def test_planted_closed_form():
    """Planted variant: every visible planted block other than the own block is
    selected when at most k-1 of them are visible."""
    w = msa_inputs.Workload("planted-small", B=1, N=64 * 128 * 2, H_q=2, H_kv=2, d=16,
                            d_idx=64, topk=4, dtype="f32", seed=9)
    x = msa_inputs.make_inputs(w, "planted")
    qi = msa_inputs.to_numpy64(x["q_idx"])
    ki = msa_inputs.to_numpy64(x["k_idx"])
    planted = msa_inputs.planted_blocks(w)              # [0, 64]
    rows = [(0, t) for t in (0, 127, 128, 5000, 8191, 8192, 8300, 16383)]
    sel = O.index_topk(qi, ki, w.block_size, w.topk, causal=True, rows=rows)
    for i, (_, t) in enumerate(rows):
        own = t // w.block_size
        vis_planted = [j for j in planted if j <= own and j != own]
        assert len(vis_planted) <= w.topk - 1
        for g in range(w.H_kv):
            s = set(sel[i, g].tolist())
            assert own in s
            assert set(vis_planted) <= s, (t, g, sel[i, g])


def test_integer_inputs_tie_break_on_random_data():
    """With values in {-2..2} exact ties are frequent; the oracle must break
    them to the lower block index (checked against a brute-force sort of
    integer pooled scores)."""
    w = msa_inputs.WORKLOADS["fwd-f32-n1k"]
    x = msa_inputs.make_inputs(w, "int")
    qi = x["q_idx"].numpy().astype(np.int64)
    ki = x["k_idx"].numpy().astype(np.int64)
    rows = [(0, t) for t in (0, 5, 127, 128, 300, 511, 640, 1000, 1023)]
    sel = O.index_topk(qi.astype(np.float64), ki.astype(np.float64), w.block_size, w.topk,
                       rows=rows)
    ties_seen = 0
    for i, (_, t) in enumerate(rows):
        sc = _brute_scores_int(qi, ki, 0, t, 0, True)
        exp_sel, pooled, _ = _brute_select(sc, t, w.N, w.block_size, w.topk, True)
        vals = [pooled[j] for j in pooled]
        ties_seen += len(vals) - len(set(vals))
        assert sel[i, 0].tolist() == exp_sel
    assert ties_seen > 0
