"""GPU parity of msa_sparse_fwd against the oracle run on the GPU's own
block_idx.

Bar: bf16 O max-relative error <= 2e-2 and cosine >= 0.999, LSE max abs
<= 2e-2; fp32 O max-relative <= 1e-4 and LSE max abs <= 1e-4.  Plus the
closed form q = 0 (O = mean of V over S(t), LSE = ln |S(t)|) at every row."""

import math

import numpy as np
import pytest
import torch

import msa_inputs
from oracle import msa_oracle as O
from tests.gpu_helpers import (cosine, f32, fwd_chunk_queries, max_rel, need_gpu, sample_rows, say)

pytestmark = pytest.mark.gpu


def _forward(w, variant, causal=True, zero_q=False):
    msa = need_gpu()
    say(f"[fwd] {w.name} variant={variant} causal={causal} B={w.B} N={w.N} H={w.H_q}/{w.H_kv} "
        f"d={w.d} topk={w.topk} dtype={w.dtype}")
    x = msa_inputs.make_inputs(w, variant, device="cuda")
    if zero_q:
        x["q"].zero_()
    sel = msa.index_topk(x["q_idx"], x["k_idx"], topk=w.topk, causal=causal)
    o, lse = msa.sparse_fwd(x["q"], x["k"], x["v"], sel, d_idx=w.d_idx, causal=causal)
    torch.cuda.synchronize()
    return x, sel, o, lse


def _bar(w):
    return (1e-4, 1.0 - 1e-7, 1e-4) if w.dtype == "f32" else (2e-2, 0.999, 2e-2)


def _check_full(w, variant="normal", causal=True):
    x, sel, o, lse = _forward(w, variant, causal)
    ref_o, ref_l = O.sparse_fwd(f32(x["q"]), f32(x["k"]), f32(x["v"]), sel.cpu().numpy().astype(np.int64),
                                w.block_size, causal)
    rel_tol, cos_tol, lse_tol = _bar(w)
    got = f32(o)
    r, c, dl = max_rel(got, ref_o), cosine(got, ref_o), float(np.abs(f32(lse) - ref_l).max())
    say(f"  O maxrel {r:.3e} cos {c:.7f}  LSE maxabs {dl:.3e}")
    assert r <= rel_tol and c >= cos_tol and dl <= lse_tol


C1 = msa_inputs.WORKLOADS["fwd-f32-n1k"]


def test_f32_forward_normal():
    _check_full(C1, "normal")


def test_f32_forward_integer():
    _check_full(C1, "int")


def test_f32_forward_noncausal():
    _check_full(C1.replace(name="f32-noncausal"), "normal", causal=False)


@pytest.mark.parametrize("G,d", [(1, 128), (2, 64), (4, 128), (8, 128), (16, 64)])
def test_bf16_forward_group_sizes(G, d):
    H_kv = 2
    w = msa_inputs.Workload(f"bf16-G{G}-d{d}", B=2, N=1536, H_q=G * H_kv, H_kv=H_kv, d=d, d_idx=64, topk=5,
                            seed=50 + G)
    _check_full(w)


def test_bf16_forward_noncausal():
    w = msa_inputs.Workload("bf16-noncausal", B=1, N=1024, H_q=8, H_kv=2, d=128, d_idx=32, topk=3, seed=61)
    _check_full(w, causal=False)


def test_bf16_forward_topk_edges():
    for topk in (1, 2, 32):
        w = msa_inputs.Workload(f"bf16-k{topk}", B=1, N=1024, H_q=8, H_kv=4, d=128, d_idx=64, topk=topk,
                                seed=70 + topk)
        _check_full(w)


@pytest.mark.parametrize("B,N", [(3, 128), (2, 1152)])
def test_bf16_forward_single_block_and_ragged(B, N):
    # N = 128: one block, the own block, under the causal mask, every other
    # slot padding.  N = 1152: the last index tile and work items are partial.
    w = msa_inputs.Workload(f"bf16-ragged-{N}", B=B, N=N, H_q=8, H_kv=2, d=128, d_idx=64, topk=16, seed=91 + N)
    _check_full(w)


def test_zero_query_closed_form():
    """q = 0: every score is 0, so O is the mean of V over S(t) and the LSE
    is ln |S(t)| - for every row, which pins the mask and the support."""
    w = msa_inputs.Workload("bf16-zero-q", B=1, N=2048, H_q=8, H_kv=2, d=128, d_idx=64, topk=4, seed=80)
    x, sel, o, lse = _forward(w, "normal", zero_q=True)
    s = sel.cpu().numpy()
    v = f32(x["v"]).astype(np.float64)
    got_o, got_l = f32(o), f32(lse)
    cs = np.cumsum(np.concatenate([np.zeros((1, w.B, w.H_kv, w.d)), v.transpose(1, 0, 2, 3)]), axis=0)
    worst_o = worst_l = 0.0
    for t in range(w.N):
        for g in range(w.H_kv):
            S = O.support(s[0, t, g], t, w.N, w.block_size, True)
            mean = v[0, S, g].mean(0)
            for h in range(g * 4, g * 4 + 4):
                worst_o = max(worst_o, float(np.abs(got_o[0, t, h] - mean).max()))
                worst_l = max(worst_l, abs(float(got_l[0, t, h]) - math.log(len(S))))
    say(f"  zero-q: O maxabs {worst_o:.3e}, LSE maxabs {worst_l:.3e}")
    assert worst_o <= 2e-2 and worst_l <= 1e-4


def test_bf16_forward_full_multi_tile():
    w = msa_inputs.Workload("bf16-2k", B=2, N=2048, H_q=16, H_kv=4, d=128, d_idx=64, topk=8, seed=90)
    _check_full(w)


def _check_sampled(w, variant, n_rows, seed, causal=True):
    x, sel, o, lse = _forward(w, variant, causal=causal)
    chunk = fwd_chunk_queries(w)
    seams = [c + dt for c in range(chunk, w.N, chunk) for dt in (-1, 0, 1)]
    rows = sample_rows(w.B, w.N, n_rows, seed, extra=seams)
    bt = torch.tensor(rows, dtype=torch.long)
    q_rows = f32(x["q"][bt[:, 0], bt[:, 1]])
    ref_o, ref_l = O.sparse_fwd(q_rows, f32(x["k"]), f32(x["v"]), sel.cpu().numpy().astype(np.int64),
                                w.block_size, causal, rows=rows)
    got = f32(o[bt[:, 0], bt[:, 1]])
    got_l = f32(lse[bt[:, 0], bt[:, 1]])
    r, c, dl = max_rel(got, ref_o), cosine(got, ref_o), float(np.abs(got_l - ref_l).max())
    say(f"  chunk {chunk}, {len(rows)} rows: O maxrel {r:.3e} cos {c:.7f}  LSE maxabs {dl:.3e}")
    assert r <= 2e-2 and c >= 0.999 and dl <= 2e-2


def test_bf16_forward_8k_sampled():
    _check_sampled(msa_inputs.WORKLOADS["fwd-bf16-n8k"], "normal", 256, 2)


def test_bf16_forward_b4_8k_sampled():
    _check_sampled(msa_inputs.WORKLOADS["fwdbwd-bf16-b4-n8k"], "normal", 96, 3)


def test_bf16_forward_128k_sampled():
    _check_sampled(msa_inputs.WORKLOADS["fwd-bf16-n128k"], "normal", 96, 4)


def test_bf16_forward_128k_planted_sampled():
    _check_sampled(msa_inputs.WORKLOADS["fwd-bf16-n128k"], "planted", 64, 104)


def test_bf16_forward_topk64_sampled():
    # topk 64 over 72 blocks: 64 slots per row to merge (two chunks of loads).
    w = msa_inputs.Workload("bf16-k64", B=1, N=9216, H_q=8, H_kv=2, d=128, d_idx=64, topk=64, seed=98)
    _check_sampled(w, "normal", 96, 98)


def test_bf16_forward_d64_sampled():
    # d = 64, d_idx = 32 with multi-item lists.
    w = msa_inputs.Workload("bf16-d64-8k", B=2, N=8192, H_q=16, H_kv=4, d=64, d_idx=32, topk=16, seed=97)
    _check_sampled(w, "normal", 96, 97)


def test_bf16_forward_noncausal_sampled():
    # Every query sees every block (its own block unmasked too).
    w = msa_inputs.Workload("bf16-nc-8k", B=1, N=8192, H_q=32, H_kv=8, d=128, d_idx=64, topk=16, seed=96)
    _check_sampled(w, "normal", 128, 96, causal=False)


def test_bf16_forward_1m_sampled():
    _check_sampled(msa_inputs.WORKLOADS["fwdbwd-bf16-n1m"], "normal", 24, 5)
