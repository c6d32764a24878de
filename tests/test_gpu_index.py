"""GPU parity of msa_index_topk against the oracle.

Bar: block_idx bit-exact for integer-valued inputs (exact scores, many exact
ties broken to the lower block); for N(0,1) inputs bit-exact except rows the
oracle flags as near ties under the fp32 accumulation bound, where the GPU
selection must be equivalent up to those ties; the top-k stage alone is
bit-exact when re-run by the oracle on the kernel's own pooled scores."""

import numpy as np
import pytest
import torch

import msa_inputs
from oracle import msa_oracle as O
from tests.gpu_helpers import (U_FP8, U_MFMA, f32, need_gpu, row_tolerance, sample_rows, say, score_bounds,
                               selection_equivalent)

pytestmark = pytest.mark.gpu


def _host(t: torch.Tensor):
    """Exact host values of index inputs: FP8 E4M3 through the oracle's own
    decoding of the bytes, other dtypes by an exact upcast."""
    if t.dtype == torch.float8_e4m3fn:
        return O.decode_e4m3(t.view(torch.uint8).cpu().numpy())
    return f32(t)


def _run(w, variant, want_pooled=True, causal=True, fp8=False):
    msa = need_gpu()
    say(f"[index] {w.name} variant={variant} causal={causal} N={w.N} H_kv={w.H_kv} topk={w.topk} fp8={fp8}")
    x = msa_inputs.make_inputs(w, variant, device="cuda", index_fp8=fp8)
    out = msa.index_topk(x["q_idx"], x["k_idx"], topk=w.topk, causal=causal, return_pooled=want_pooled)
    torch.cuda.synchronize()
    return x, out


def _check_full(w, variant, causal=True, exact=True, fp8=False):
    u = U_FP8 if fp8 else U_MFMA      # unit roundoff of the matrix unit's accumulation
    x, (sel, pooled) = _run(w, variant, True, causal, fp8)
    qi, ki = _host(x["q_idx"]), _host(x["k_idx"])
    ref_sel, ref_pool = O.index_topk(qi, ki, w.block_size, w.topk, causal=causal, want_pooled=True)
    gsel = sel.cpu().numpy().astype(np.int64)
    gpool = pooled.cpu().numpy()
    # The top-k stage alone: the oracle's selection on the GPU's pooled scores.
    nb = w.N // w.block_size
    for b in range(w.B):
        for t in range(w.N):
            for g in range(w.H_kv):
                st = O.select_blocks_row(gpool[b, t, g].astype(np.float64), t, w.block_size, w.topk, causal)
                assert st.tolist() == gsel[b, t, g].tolist(), ("top-k stage", b, t, g)
    if exact:
        np.testing.assert_array_equal(gpool, ref_pool)
        np.testing.assert_array_equal(gsel, ref_sel)
        return 0
    # Near ties allowed only under the accumulation bound.
    fin = np.isfinite(ref_pool)
    assert (np.isfinite(gpool) == fin).all()
    # Pooled values: each within the accumulation bound of the row's scores.
    worst = 0.0
    for b in range(w.B):
        bound = score_bounds(qi[b], ki[b], causal, w.d_idx, u=u)                  # [N, H_kv]
        err = np.where(fin[b], np.abs(gpool[b].astype(np.float64) - np.where(fin[b], ref_pool[b], 0.0)), 0.0)
        err = err.max(axis=2)
        bad = np.argwhere(err > bound)
        assert bad.size == 0, ("pooled value", b, bad[:4].tolist())
        worst = max(worst, float((err / np.maximum(bound, 1e-300)).max()))
    say(f"  pooled scores: worst error {worst:.3f} of the accumulation bound")
    flagged = 0
    for b in range(w.B):
        for t in range(w.N):
            for g in range(w.H_kv):
                if (gsel[b, t, g] == ref_sel[b, t, g]).all():
                    continue
                tol = row_tolerance(qi[b, t, g], ki[b], t, causal, w.d_idx, u)
                assert selection_equivalent(gsel[b, t, g], ref_sel[b, t, g], ref_pool[b, t, g], t,
                                            w.block_size, tol), (b, t, g, gsel[b, t, g], ref_sel[b, t, g])
                flagged += 1
    say(f"  near-tie rows {flagged} of {w.B * w.N * w.H_kv}")
    assert flagged <= max(2, w.B * w.N * w.H_kv // 1000)
    return flagged


C1 = msa_inputs.WORKLOADS["fwd-f32-n1k"]


def test_f32_integer_inputs_bit_exact():
    _check_full(C1, "int", exact=True)


def test_f32_normal_inputs():
    _check_full(C1, "normal", exact=False)


def test_f32_noncausal_integer():
    _check_full(C1.replace(name="f32-noncausal"), "int", causal=False, exact=True)


def test_bf16_integer_multi_tile_groups():
    w = msa_inputs.Workload("bf16-int-4k", B=2, N=4096, H_q=8, H_kv=8, d=128, d_idx=64, topk=16, seed=21)
    _check_full(w, "int", exact=True)


@pytest.mark.parametrize("topk", [1, 2, 5, 9, 32])
def test_bf16_integer_topk_edges(topk):
    w = msa_inputs.Workload(f"bf16-int-k{topk}", B=1, N=2048, H_q=4, H_kv=2, d=64, d_idx=32, topk=topk,
                            seed=30 + topk)
    _check_full(w, "int", exact=True)


@pytest.mark.parametrize("fp8", [False, True])
def test_integer_topk64_full_lists(fp8):
    # 72 blocks: rows past block 63 keep a full list of 63 other blocks (the
    # largest topk the library takes), earlier rows carry padding.
    w = msa_inputs.Workload(f"int-k64-fp8{int(fp8)}", B=1, N=9216, H_q=4, H_kv=2, d=64, d_idx=64, topk=64,
                            seed=97)
    _check_full(w, "int", exact=True, fp8=fp8)


def test_topk_larger_than_blocks_pads():
    w = msa_inputs.Workload("pad", B=1, N=512, H_q=1, H_kv=1, d=64, d_idx=64, topk=8, seed=5)
    x, (sel, pooled) = _run(w, "normal")
    s = sel.cpu().numpy()[0, :, 0]
    for t in range(w.N):
        own = t // 128
        assert s[t].tolist() == list(range(own + 1)) + [-1] * (8 - own - 1)


@pytest.mark.parametrize("B,N,H_kv", [(3, 128, 2), (2, 1152, 2), (1, 640, 1)])
def test_bf16_integer_ragged_query_tiles(B, N, H_kv):
    # A workgroup covers 64 queries per wave (256 at H_kv = 2, 512 at H_kv = 1):
    # these lengths leave whole waves past the end of the sequence, and N = 128
    # is the one-block sequence whose rows hold the own block and padding only.
    w = msa_inputs.Workload(f"bf16-int-ragged-{N}", B=B, N=N, H_q=2 * H_kv, H_kv=H_kv, d=64, d_idx=64, topk=4,
                            seed=43 + N)
    _check_full(w, "int", exact=True)
    if N == 128:
        sel = _run(w, "int", True, True, False)[1][0].cpu().numpy()
        assert (sel[..., 0] == 0).all() and (sel[..., 1:] == -1).all()


def test_bf16_integer_h_kv_odd_groups():
    # H_kv = 3 (groups per workgroup fall back to 1) and a non-causal pass.
    w = msa_inputs.Workload("bf16-int-hkv3", B=1, N=1536, H_q=6, H_kv=3, d=64, d_idx=64, topk=4, seed=41)
    _check_full(w, "int", exact=True)
    _check_full(w, "int", causal=False, exact=True)


def test_bf16_normal_8k():
    _check_full(msa_inputs.WORKLOADS["fwd-bf16-n8k"], "normal", exact=False)


def _sampled(w, variant, n_rows, seed, fp8=False):
    msa = need_gpu()
    say(f"[index sampled] {w.name} variant={variant} fp8={fp8}")
    x = msa_inputs.make_inputs(w, variant, device="cuda", index_fp8=fp8)
    sel = msa.index_topk(x["q_idx"], x["k_idx"], topk=w.topk)
    torch.cuda.synchronize()
    rows = sample_rows(w.B, w.N, n_rows, seed)
    bt = torch.tensor(rows, dtype=torch.long)
    qi_rows = _host(x["q_idx"][bt[:, 0], bt[:, 1]])
    ki = _host(x["k_idx"])
    ref_sel, ref_pool = O.index_topk(qi_rows, ki, w.block_size, w.topk, rows=rows, want_pooled=True)
    gsel = sel[bt[:, 0], bt[:, 1]].cpu().numpy().astype(np.int64)
    flagged = 0
    for i, (b, t) in enumerate(rows):
        for g in range(w.H_kv):
            if (gsel[i, g] == ref_sel[i, g]).all():
                continue
            tol = row_tolerance(qi_rows[i, g], ki[b], t, True, w.d_idx, U_FP8 if fp8 else U_MFMA)
            assert selection_equivalent(gsel[i, g], ref_sel[i, g], ref_pool[i, g], t, w.block_size, tol), \
                (b, t, g, gsel[i, g], ref_sel[i, g])
            flagged += 1
    say(f"  sampled rows {len(rows)}, near-tie rows {flagged}")
    assert flagged <= max(2, len(rows) * w.H_kv // 200)
    return x, sel, rows


def test_bf16_128k_sampled():
    _sampled(msa_inputs.WORKLOADS["fwd-bf16-n128k"], "normal", 96, 4)


def test_bf16_128k_planted_closed_form():
    w = msa_inputs.WORKLOADS["fwd-bf16-n128k"]
    x, sel, rows = _sampled(w, "planted", 64, 104)
    planted = set(msa_inputs.planted_blocks(w))
    s = sel.cpu().numpy()
    # Every row: every visible planted block other than its own is selected
    # when at most k-1 of them are visible; otherwise k-1 planted blocks are.
    for t in range(0, w.N, 97):
        own = t // w.block_size
        want = {j for j in planted if j < own}
        for g in range(w.H_kv):
            got = set(s[0, t, g].tolist())
            if len(want) <= w.topk - 1:
                assert want <= got, (t, g)
            else:
                assert len(want & got) == w.topk - 1, (t, g)


def test_bf16_1m_sampled():
    _sampled(msa_inputs.WORKLOADS["fwdbwd-bf16-n1m"], "normal", 32, 5)


# FP8 E4M3 index inputs (d_idx = 64): the same bar, with the oracle run on the
# decoded E4M3 values.  Products of E4M3 values are exact in fp32, so integer
# inputs give exact scores and bit-exact pooled scores and selections.
def test_fp8_integer_inputs_bit_exact():
    w = msa_inputs.Workload("fp8-int-4k", B=2, N=4096, H_q=8, H_kv=8, d=128, d_idx=64, topk=16, seed=121)
    _check_full(w, "int", exact=True, fp8=True)


@pytest.mark.parametrize("topk", [1, 5, 32])
def test_fp8_integer_topk_edges_and_noncausal(topk):
    w = msa_inputs.Workload(f"fp8-int-k{topk}", B=1, N=2048, H_q=6, H_kv=3, d=64, d_idx=64, topk=topk,
                            seed=130 + topk)
    _check_full(w, "int", exact=True, fp8=True)
    _check_full(w, "int", causal=False, exact=True, fp8=True)


def test_fp8_normal_8k():
    _check_full(msa_inputs.WORKLOADS["fwd-bf16-n8k"], "normal", exact=False, fp8=True)


def test_fp8_128k_sampled():
    _sampled(msa_inputs.WORKLOADS["fwd-bf16-n128k"], "normal", 96, 14, fp8=True)


@pytest.mark.parametrize("softmax", [False, True])
def test_torch_topk_pipeline_selects_the_same_blocks(softmax):
    """The materialise-then-torch.topk pipeline that bench.py --compare-topk
    times against the fused kernel computes the same selection (fp32 scores
    here): rows differ only at near ties under the accumulation bound."""
    import bench
    w = msa_inputs.Workload("bf16-cmp-topk", B=1, N=2048, H_q=16, H_kv=4, d=128, d_idx=64, topk=16, seed=95)
    x, sel = _run(w, "normal", want_pooled=False)
    ref_t = bench.torch_index_topk(x["q_idx"], x["k_idx"], w.topk, w.block_size, softmax=softmax, chunk=512,
                                   score_dtype=torch.float32)
    torch.cuda.synchronize()
    qi, ki = f32(x["q_idx"]), f32(x["k_idx"])
    ref_sel, ref_pool = O.index_topk(qi, ki, w.block_size, w.topk, causal=True, want_pooled=True)
    gsel, tsel = sel.cpu().numpy().astype(np.int64), ref_t.cpu().numpy().astype(np.int64)
    differ = 0
    for t in range(w.N):
        for g in range(w.H_kv):
            if (tsel[0, t, g] == gsel[0, t, g]).all():
                continue
            tol = row_tolerance(qi[0, t, g], ki[0], t, True, w.d_idx)
            assert selection_equivalent(tsel[0, t, g], ref_sel[0, t, g], ref_pool[0, t, g], t, w.block_size,
                                        tol), (t, g, tsel[0, t, g], gsel[0, t, g])
            differ += 1
    say(f"  torch pipeline (softmax={softmax}) rows differing from the kernel: {differ} of {w.N * w.H_kv}")
    assert differ <= max(2, w.N * w.H_kv // 1000)
