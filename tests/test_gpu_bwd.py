"""GPU parity of msa_sparse_bwd against the oracle run on the GPU's own
block_idx.

Bar: every gradient tensor (dq, dk, dv, dq_idx, dk_idx) and dscore at cosine
>= 0.999 against the fp64 oracle (max-relative error reported); the KL value
per row within 2e-2 absolute.  Properties checked at any size: per row the
index-logit gradient sums to zero (sum p_px = sum pbar = 1)."""

import numpy as np
import pytest
import torch

import msa_inputs
from oracle import msa_oracle as O
from tests.gpu_helpers import bwd_chunk_queries, cosine, f32, max_rel, need_gpu, sample_rows, say

pytestmark = pytest.mark.gpu

COS = 0.999


def _run(w, variant="normal", causal=True, want_dscore=False, want_kl=False, lam=1.0):
    msa = need_gpu()
    say(f"[bwd] {w.name} variant={variant} causal={causal} B={w.B} N={w.N} H={w.H_q}/{w.H_kv} d={w.d} "
        f"d_idx={w.d_idx} topk={w.topk}")
    x = msa_inputs.make_inputs(w, variant, device="cuda", with_grad_out=True)
    sel = msa.index_topk(x["q_idx"], x["k_idx"], topk=w.topk, causal=causal)
    o, lse = msa.sparse_fwd(x["q"], x["k"], x["v"], sel, d_idx=w.d_idx, causal=causal)
    gr = msa.sparse_bwd(x["q"], x["k"], x["v"], o, x["dO"], lse, sel, x["q_idx"], x["k_idx"], kl_weight=lam,
                        causal=causal, want_dscore=want_dscore, want_kl=want_kl)
    torch.cuda.synchronize()
    return x, sel, gr


def _cmp(name, got, ref, cos_min=COS):
    c, r = cosine(got, ref), max_rel(got, ref)
    say(f"  {name:7s} cos {c:.6f} maxrel {r:.3e}")
    assert c >= cos_min, name
    return c


def _full(w, causal=True, lam=1.0):
    x, sel, gr = _run(w, causal=causal, want_dscore=True, want_kl=True, lam=lam)
    h = {k: f32(v) for k, v in x.items()}
    ref = O.sparse_bwd(h["q"], h["k"], h["v"], h["dO"], h["q_idx"], h["k_idx"],
                       sel.cpu().numpy().astype(np.int64), w.block_size, causal, kl_weight=lam, want_dscore=True)
    for name in ("dq", "dk", "dv", "dq_idx", "dk_idx", "dscore"):
        _cmp(name, f32(gr[name]), ref[name])
    dkl = float(np.abs(f32(gr["kl"]) - ref["kl"]).max())
    say(f"  kl maxabs {dkl:.3e}")
    assert dkl <= 2e-2
    # Property: per (b, t, g) the index-logit gradient sums to zero.
    zsum = f32(gr["dscore"]).sum(axis=(3, 4))
    assert np.abs(zsum).max() <= 1e-3 * max(1.0, abs(lam))


@pytest.mark.parametrize("G,d,d_idx", [(1, 128, 64), (2, 64, 32), (4, 128, 64), (8, 128, 64), (16, 64, 64),
                                       (8, 64, 32)])
def test_bwd_group_sizes(G, d, d_idx):
    H_kv = 2
    w = msa_inputs.Workload(f"bwd-G{G}-d{d}-i{d_idx}", B=2, N=1536, H_q=G * H_kv, H_kv=H_kv, d=d, d_idx=d_idx,
                            topk=5, backward=True, seed=200 + G)
    _full(w)


def test_bwd_noncausal():
    w = msa_inputs.Workload("bwd-noncausal", B=1, N=1024, H_q=8, H_kv=2, d=128, d_idx=64, topk=3, backward=True,
                            seed=210)
    _full(w, causal=False)


@pytest.mark.parametrize("topk", [1, 2, 12])
def test_bwd_topk_edges(topk):
    # topk = 12 > 8 blocks: rows of early blocks carry -1 padding.
    w = msa_inputs.Workload(f"bwd-k{topk}", B=1, N=1024, H_q=8, H_kv=2, d=128, d_idx=64, topk=topk, backward=True,
                            seed=220 + topk)
    _full(w)


@pytest.mark.parametrize("B,N", [(3, 128), (2, 1152)])
def test_bwd_single_block_and_ragged(B, N):
    # N = 128: every row's support is its own causal prefix and p_px, pbar
    # live on the one block; N = 1152: partial last items and index tiles.
    w = msa_inputs.Workload(f"bwd-ragged-{N}", B=B, N=N, H_q=8, H_kv=2, d=128, d_idx=64, topk=16,
                            backward=True, seed=250 + N)
    _full(w)


def test_bwd_kl_weight_scales_index_gradients():
    w = msa_inputs.Workload("bwd-lam", B=1, N=1024, H_q=16, H_kv=2, d=128, d_idx=64, topk=4, backward=True, seed=230)
    _full(w, lam=0.37)


def test_bwd_multi_tile_full():
    w = msa_inputs.Workload("bwd-2k", B=2, N=2048, H_q=16, H_kv=4, d=128, d_idx=64, topk=8, backward=True, seed=240)
    _full(w)


def _sampled(w, variant, n_rows, seed, blocks):
    """Rows: dq, dq_idx, kl, dscore of sampled rows.  Blocks: dk, dv (group 0)
    and dk_idx of sampled KV blocks of batch 0, recomputed from every row that
    selected them."""
    x, sel, gr = _run(w, variant, want_kl=True)
    chunk = bwd_chunk_queries(w)
    seams = [c + dt for c in range(chunk, w.N, chunk) for dt in (-1, 0, 1)]
    rows = sample_rows(w.B, w.N, n_rows, seed, extra=seams)
    say(f"  main-kernel chunk {chunk} queries, {len(seams)} seam rows")
    bt = torch.tensor(rows, dtype=torch.long)
    s = sel.cpu().numpy().astype(np.int64)
    k_h, v_h, ki_h = f32(x["k"]), f32(x["v"]), f32(x["k_idx"])
    ref = O.sparse_bwd(f32(x["q"][bt[:, 0], bt[:, 1]]), k_h, v_h, f32(x["dO"][bt[:, 0], bt[:, 1]]),
                       f32(x["q_idx"][bt[:, 0], bt[:, 1]]), ki_h, s, w.block_size, True, rows=rows)
    _cmp("dq", f32(gr["dq"][bt[:, 0], bt[:, 1]]), ref["dq"])
    _cmp("dq_idx", f32(gr["dq_idx"][bt[:, 0], bt[:, 1]]), ref["dq_idx"])
    dkl = float(np.abs(f32(gr["kl"][bt[:, 0], bt[:, 1]]) - ref["kl"]).max())
    say(f"  kl maxabs {dkl:.3e} over {len(rows)} rows")
    assert dkl <= 2e-2
    for j in blocks:
        sel_rows = np.nonzero((s[0] == j).any(axis=(1, 2)))[0]
        brow = [(0, int(t)) for t in sel_rows]
        bti = torch.tensor(brow, dtype=torch.long)
        say(f"  block {j}: {len(brow)} selecting rows")
        rb = O.sparse_bwd(f32(x["q"][bti[:, 0], bti[:, 1]]), k_h, v_h, f32(x["dO"][bti[:, 0], bti[:, 1]]),
                          f32(x["q_idx"][bti[:, 0], bti[:, 1]]), ki_h, s, w.block_size, True, rows=brow)
        ks = slice(j * w.block_size, (j + 1) * w.block_size)
        for name in ("dk", "dv"):
            _cmp(f"{name}[{j}]", f32(gr[name][0, ks]), rb[name][0, ks])
        _cmp(f"dki[{j}]", f32(gr["dk_idx"][0, ks]), rb["dk_idx"][0, ks])


# The sampled KV blocks are late ones, chosen by a few hundred to about a
# thousand rows, so the fp64 recomputation of their dk/dv stays within seconds
# (block 5 at 8K is chosen by ~7300 rows: minutes).  Lists long enough to
# span several work items, whose dk/dv add up across items, are compared in
# full by test_bwd_multi_tile_full (its longest lists hold ~1550 entries past
# the own block, beyond one item's 1024).
def test_bwd_b4_8k_sampled():
    w = msa_inputs.WORKLOADS["fwdbwd-bf16-b4-n8k"]
    _sampled(w, "normal", 96, 3, blocks=[w.nblk - 1, w.nblk - 8])


def test_bwd_128k_sampled():
    w = msa_inputs.WORKLOADS["fwdbwd-bf16-n128k"]
    _sampled(w, "normal", 48, 4, blocks=[w.nblk - 1, w.nblk - 20])


def test_bwd_128k_planted_sampled():
    w = msa_inputs.WORKLOADS["fwdbwd-bf16-n128k"]
    _sampled(w, "planted", 32, 104, blocks=[w.nblk - 1])


def test_bwd_1m_sampled():
    w = msa_inputs.WORKLOADS["fwdbwd-bf16-n1m"]
    _sampled(w, "normal", 16, 5, blocks=[w.nblk - 1])


def test_bwd_dq_and_forward_deterministic():
    """dq is summed from per-block partials in a fixed order, and the forward
    merges its partials in slot order: both are bit-identical across calls
    (dk, dv and the index gradients use fp32 atomics and are not)."""
    msa = need_gpu()
    w = msa_inputs.WORKLOADS["fwdbwd-bf16-b4-n8k"]
    say(f"[determinism] {w.name}")
    x = msa_inputs.make_inputs(w, "normal", device="cuda", with_grad_out=True)
    sel = msa.index_topk(x["q_idx"], x["k_idx"], topk=w.topk)
    runs = []
    for _ in range(2):
        o, lse = msa.sparse_fwd(x["q"], x["k"], x["v"], sel, d_idx=w.d_idx)
        gr = msa.sparse_bwd(x["q"], x["k"], x["v"], o, x["dO"], lse, sel, x["q_idx"], x["k_idx"])
        runs.append((o, lse, gr["dq"]))
    torch.cuda.synchronize()
    for name, a, b in zip(("o", "lse", "dq"), runs[0], runs[1]):
        same = torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))
        say(f"  {name} bit-identical: {same}")
        assert same, name
