"""GPU parity of msa_sparse_bwd against the oracle run on the GPU's own
block_idx.

Bar: every gradient tensor (dq, dk, dv, dq_idx, dk_idx) and dscore at cosine
>= 0.999 against the fp64 oracle, both over the whole tensor and on every
slice where a local error would hide: per (query row, group) for dq, dq_idx
and dscore, per (KV block, group) for dk and dv, per KV block for dk_idx.  A
slice whose oracle value is zero must be (near) zero on the GPU too.  The KL
value per row within 2e-2 absolute.  Properties checked at any size: per row
the index-logit gradient sums to zero (sum p_px = sum pbar = 1).  The small
full cases also run the kernel instance without the per-score outputs (the
one a training step runs, which skips the causal test off the diagonal) and
hold it to the same per-slice bar.

The backward forms D = rowsum(dO * o) from the o it is given, as the
FlashAttention backward does.  The per-row dq bar therefore runs with the
oracle's own o (rounded to the dtype) as the input of both sides, so that
both form the same D; fed the GPU forward's o instead (the chained pass of
the small cases), D carries that o's rounding, which dominates the rare rows
whose dq nearly cancels (e.g. |dq| = 0.03 against a typical 2), so there dq
is held to the whole-tensor bar and every other slice check still applies.

At the full sizes (8K with B = 4, 128K, 1M) the heavy-list tests compare the
whole dk, dv and dk_idx tensors: off a seeded sample of rows dO and q_idx are
zero, so only the sampled rows add to them (exactly zero elsewhere), while
those zero index queries make every row select blocks 0 .. topk-2, whose
inverted lists then span many work items (and every main-kernel chunk)."""

import numpy as np
import pytest
import torch

import msa_inputs
from oracle import msa_oracle as O
from tests.gpu_helpers import bwd_chunk_queries, cosine, f32, fwd_chunk_queries, max_rel, need_gpu, \
    sample_rows, say

pytestmark = pytest.mark.gpu

COS = 0.999
DEV = "cuda"   # device of the test tensors
# A slice whose oracle value is exactly zero may hold rounding residue on the
# GPU (e.g. t = 0, where p_px = pbar = 1 in exact arithmetic): it must stay
# below this fraction of the largest slice norm of the tensor.
ZERO_FRAC = 1e-4


def _fwd(w, variant="normal", causal=True, x=None):
    msa = need_gpu()
    say(f"[bwd] {w.name} variant={variant} causal={causal} B={w.B} N={w.N} H={w.H_q}/{w.H_kv} d={w.d} "
        f"d_idx={w.d_idx} topk={w.topk}")
    if x is None:
        x = msa_inputs.make_inputs(w, variant, device=DEV, with_grad_out=True)
    sel = msa.index_topk(x["q_idx"], x["k_idx"], topk=w.topk, causal=causal)
    o, lse = msa.sparse_fwd(x["q"], x["k"], x["v"], sel, d_idx=w.d_idx, causal=causal)
    return x, sel, o, lse


def _bwd(w, x, sel, o, lse, causal=True, want_dscore=False, want_kl=False, lam=1.0):
    msa = need_gpu()
    gr = msa.sparse_bwd(x["q"], x["k"], x["v"], o, x["dO"], lse, sel, x["q_idx"], x["k_idx"], kl_weight=lam,
                        causal=causal, want_dscore=want_dscore, want_kl=want_kl)
    torch.cuda.synchronize()
    return gr


def _oracle_output(w, x, sel_np, rows=None, causal=True):
    """The oracle's forward output and LSE (for all rows, or for `rows`), as
    the backward's inputs: o rounded to the workload dtype, lse to fp32."""
    if rows is None:
        q = f32(x["q"])
    else:
        bt = torch.tensor(rows, dtype=torch.long)
        q = f32(x["q"][bt[:, 0], bt[:, 1]])
    o, lse = O.sparse_fwd(q, f32(x["k"]), f32(x["v"]), sel_np, w.block_size, causal, rows=rows)
    o_in = torch.from_numpy(o).to(x["q"].dtype)
    return o_in, torch.from_numpy(lse).float()


def _slices_cos(name, got, ref, what, cos_min=COS, norm_scale=None):
    """got, ref: [S, L] (one slice per row).  cos >= cos_min on every slice
    with a nonzero reference; near zero where the reference is zero."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    rn = np.sqrt((r * r).sum(axis=1))
    gn = np.sqrt((g * g).sum(axis=1))
    scale = float(rn.max()) if norm_scale is None else norm_scale
    live = rn > 0
    cos = (g[live] * r[live]).sum(axis=1) / np.maximum(gn[live] * rn[live], 1e-300)
    worst = float(cos.min()) if cos.size else 1.0
    zero_res = float(gn[~live].max()) / scale if (~live).any() and scale > 0 else 0.0
    say(f"  {name:9s} per {what}: {int(live.sum())} slices, worst cos {worst:.6f}; "
        f"{int((~live).sum())} zero slices, largest residue {zero_res:.1e} of the top norm")
    if cos.size:
        i = int(np.argmin(cos))
        assert worst >= cos_min, (name, what, "slice", int(np.nonzero(live)[0][i]), worst)
    assert zero_res <= ZERO_FRAC, (name, what, "nonzero where the oracle is zero", zero_res)


def _cmp(name, got, ref, cos_min=COS):
    c, r = cosine(got, ref), max_rel(got, ref)
    say(f"  {name:9s} cos {c:.6f} maxrel {r:.3e}")
    assert c >= cos_min, name
    return c


def _per_row_group(a, H_kv):
    """[..., H(_q or _kv), X] rows -> [rows * H_kv, rest]: one slice per (row, group)."""
    a = np.asarray(a)
    lead = int(np.prod(a.shape[: a.ndim - 2])) if a.ndim > 2 else 1
    return a.reshape(lead * H_kv, -1)


def _per_block_group(a, bs):
    """[B, N, H_kv, d] -> [(b, j, g), bs * d]."""
    B, N, H, D = a.shape
    return np.asarray(a).reshape(B, N // bs, bs, H, D).transpose(0, 1, 3, 2, 4).reshape(-1, bs * D)


def _per_block(a, bs):
    """[B, N, d_idx] -> [(b, j), bs * d_idx]."""
    B, N, D = a.shape
    return np.asarray(a).reshape(B * (N // bs), bs * D)


def _full(w, causal=True, lam=1.0):
    """Two passes over the same inputs.
    Chained: the GPU forward's o and lse feed the GPU backward, against the
    oracle's exact D = sum_u P dP.  Every tensor and every slice is compared
    except dq per row: there D carries the stored o's rounding, which
    dominates the few rows whose dq nearly cancels.
    Isolated: the oracle's own o (in the dtype) and lse feed the GPU backward,
    and the oracle forms D from the same o: every slice is compared, dq per
    row included."""
    x, sel, o, lse = _fwd(w, causal=causal)
    s = sel.cpu().numpy().astype(np.int64)
    h = {k: f32(v) for k, v in x.items()}
    bs, H = w.block_size, w.H_kv
    o_in, lse_in = _oracle_output(w, x, s, causal=causal)
    for mode in ("chained", "isolated"):
        if mode == "chained":
            gr = _bwd(w, x, sel, o, lse, causal, want_dscore=True, want_kl=True, lam=lam)
            o_ref = None
        else:
            gr = _bwd(w, x, sel, o_in.to(DEV), lse_in.to(DEV), causal, want_dscore=True, want_kl=True, lam=lam)
            o_ref = f32(o_in)
        say(f" {mode}:")
        ref = O.sparse_bwd(h["q"], h["k"], h["v"], h["dO"], h["q_idx"], h["k_idx"], s, bs, causal, kl_weight=lam,
                           want_dscore=True, o=o_ref)
        got = {n: f32(gr[n]) for n in ("dq", "dk", "dv", "dq_idx", "dk_idx", "dscore")}
        for name in got:
            _cmp(name, got[name], ref[name])
        if mode == "isolated":
            _slices_cos("dq", _per_row_group(got["dq"].reshape(w.B, w.N, H, -1), H),
                        _per_row_group(ref["dq"].reshape(w.B, w.N, H, -1), H), "(row, group)")
        _slices_cos("dq_idx", _per_row_group(got["dq_idx"], H), _per_row_group(ref["dq_idx"], H), "(row, group)")
        _slices_cos("dscore", got["dscore"].reshape(w.B * w.N * H, -1), ref["dscore"].reshape(w.B * w.N * H, -1),
                    "(row, group)")
        for name in ("dk", "dv"):
            _slices_cos(name, _per_block_group(got[name], bs), _per_block_group(ref[name], bs), "(block, group)")
        _slices_cos("dk_idx", _per_block(got["dk_idx"], bs), _per_block(ref["dk_idx"], bs), "block")
        dkl = float(np.abs(f32(gr["kl"]) - ref["kl"]).max())
        say(f"  kl maxabs {dkl:.3e}")
        assert dkl <= 2e-2
        # Property: per (b, t, g) the index-logit gradient sums to zero.
        zsum = got["dscore"].sum(axis=(3, 4))
        assert np.abs(zsum).max() <= 1e-3 * max(1.0, abs(lam))
        if mode == "isolated":
            # The kernel instance without the per-score outputs (the one a
            # training step runs) against the same reference.
            gp = _bwd(w, x, sel, o_in.to(DEV), lse_in.to(DEV), causal, lam=lam)
            say(" isolated, without dscore / kl:")
            gotp = {n: f32(gp[n]) for n in ("dq", "dk", "dv", "dq_idx", "dk_idx")}
            for name in gotp:
                _cmp(name, gotp[name], ref[name])
            _slices_cos("dq", _per_row_group(gotp["dq"].reshape(w.B, w.N, H, -1), H),
                        _per_row_group(ref["dq"].reshape(w.B, w.N, H, -1), H), "(row, group)")
            _slices_cos("dq_idx", _per_row_group(gotp["dq_idx"], H), _per_row_group(ref["dq_idx"], H),
                        "(row, group)")
            for name in ("dk", "dv"):
                _slices_cos(name, _per_block_group(gotp[name], bs), _per_block_group(ref[name], bs),
                            "(block, group)")
            _slices_cos("dk_idx", _per_block(gotp["dk_idx"], bs), _per_block(ref["dk_idx"], bs), "block")


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


def _seams(w):
    """Rows on both sides of every launch seam of the forward and of the
    backward main kernel."""
    out = []
    for chunk in (fwd_chunk_queries(w), bwd_chunk_queries(w)):
        out += [c + dt for c in range(chunk, w.N, chunk) for dt in (-1, 0, 1)]
    return out


def _check_rows(w, gr, ref, bt):
    H = w.H_kv
    dq = f32(gr["dq"][bt[:, 0], bt[:, 1]])
    dqi = f32(gr["dq_idx"][bt[:, 0], bt[:, 1]])
    _cmp("dq", dq, ref["dq"])
    _cmp("dq_idx", dqi, ref["dq_idx"])
    _slices_cos("dq", _per_row_group(dq.reshape(len(bt), H, -1), H),
                _per_row_group(ref["dq"].reshape(len(bt), H, -1), H), "(row, group)")
    _slices_cos("dq_idx", _per_row_group(dqi, H), _per_row_group(ref["dq_idx"], H), "(row, group)")


def _sampled(w, variant, n_rows, seed, blocks, causal=True):
    """Rows: dq, dq_idx, kl of sampled rows.  Blocks: dk, dv and dk_idx of
    sampled KV blocks of batch 0, recomputed from every row that selected
    them."""
    x, sel, o, lse = _fwd(w, variant, causal=causal)
    seams = _seams(w)
    rows = sample_rows(w.B, w.N, n_rows, seed, extra=seams)
    say(f"  {len(seams)} seam rows")
    bt = torch.tensor(rows, dtype=torch.long)
    s = sel.cpu().numpy().astype(np.int64)
    # The sampled rows' o and lse come from the oracle, so that both sides
    # form those rows' D from the same o.
    o_in, lse_in = _oracle_output(w, x, s, rows=rows, causal=causal)
    o[bt[:, 0], bt[:, 1]] = o_in.to(DEV)
    lse[bt[:, 0], bt[:, 1]] = lse_in.to(DEV)
    gr = _bwd(w, x, sel, o, lse, causal, want_kl=True)
    k_h, v_h, ki_h = f32(x["k"]), f32(x["v"]), f32(x["k_idx"])
    ref = O.sparse_bwd(f32(x["q"][bt[:, 0], bt[:, 1]]), k_h, v_h, f32(x["dO"][bt[:, 0], bt[:, 1]]),
                       f32(x["q_idx"][bt[:, 0], bt[:, 1]]), ki_h, s, w.block_size, causal, rows=rows,
                       o=f32(o_in))
    _check_rows(w, gr, ref, bt)
    dkl = float(np.abs(f32(gr["kl"][bt[:, 0], bt[:, 1]]) - ref["kl"]).max())
    say(f"  kl maxabs {dkl:.3e} over {len(rows)} rows")
    assert dkl <= 2e-2
    bs = w.block_size
    for j in blocks:
        sel_rows = np.nonzero((s[0] == j).any(axis=(1, 2)))[0]
        brow = [(0, int(t)) for t in sel_rows]
        bti = torch.tensor(brow, dtype=torch.long)
        say(f"  block {j}: {len(brow)} selecting rows")
        rb = O.sparse_bwd(f32(x["q"][bti[:, 0], bti[:, 1]]), k_h, v_h, f32(x["dO"][bti[:, 0], bti[:, 1]]),
                          f32(x["q_idx"][bti[:, 0], bti[:, 1]]), ki_h, s, bs, causal, rows=brow)
        ks = slice(j * bs, (j + 1) * bs)
        for name in ("dk", "dv"):
            g_, r_ = f32(gr[name][0, ks]), rb[name][0, ks]
            _cmp(f"{name}[{j}]", g_, r_)
            _slices_cos(f"{name}[{j}]", g_.transpose(1, 0, 2).reshape(w.H_kv, -1),
                        r_.transpose(1, 0, 2).reshape(w.H_kv, -1), "group")
        _cmp(f"dki[{j}]", f32(gr["dk_idx"][0, ks]), rb["dk_idx"][0, ks])


# The sampled KV blocks are late ones, chosen by a few hundred to about a
# thousand rows, so the fp64 recomputation of their dk/dv stays within seconds.
# Long lists that span many work items and chunks are compared in full by the
# heavy-list tests below.
def test_bwd_b4_8k_sampled():
    w = msa_inputs.WORKLOADS["fwdbwd-bf16-b4-n8k"]
    _sampled(w, "normal", 96, 3, blocks=[w.nblk - 1, w.nblk - 8])


def test_bwd_128k_sampled():
    w = msa_inputs.WORKLOADS["fwdbwd-bf16-n128k"]
    _sampled(w, "normal", 48, 4, blocks=[w.nblk - 1, w.nblk - 20])


def test_bwd_128k_planted_sampled():
    w = msa_inputs.WORKLOADS["fwdbwd-bf16-n128k"]
    _sampled(w, "planted", 32, 104, blocks=[w.nblk - 1])


def test_bwd_topk64_sampled():
    # topk 64 over 72 blocks: 64-slot dQ merges and index log-sum-exps.
    w = msa_inputs.Workload("bwd-k64", B=1, N=9216, H_q=8, H_kv=2, d=128, d_idx=64, topk=64, backward=True,
                            seed=99)
    _sampled(w, "normal", 48, 99, blocks=[w.nblk - 1, w.nblk - 8])


def test_bwd_1m_sampled():
    w = msa_inputs.WORKLOADS["fwdbwd-bf16-n1m"]
    _sampled(w, "normal", 16, 5, blocks=[w.nblk - 1])


PLANT = 10.0


def _heavy_inputs(w, rows, seed):
    """The workload's N(0,1) tensors, then: off the sampled rows, dO = 0 and
    q_idx = 0; on them, q_idx gets a seeded unit direction c with weight
    PLANT (its component along c replaced), and the index keys of block 0 get
    + PLANT c, so every sampled row past block 0 also selects block 0."""
    x = msa_inputs.make_inputs(w, "normal", device=DEV, with_grad_out=True)
    keep = torch.zeros((w.B, w.N), dtype=torch.bool, device=DEV)
    bt = torch.tensor(rows, dtype=torch.long, device=DEV)
    keep[bt[:, 0], bt[:, 1]] = True
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    c = torch.randn((w.d_idx,), generator=gen, device=DEV, dtype=torch.float32)
    c = c / c.norm()
    qi = x["q_idx"].float()
    qi = qi - (qi @ c)[..., None] * c + PLANT * c
    x["q_idx"] = torch.where(keep[:, :, None, None], qi, 0.0).to(x["q_idx"].dtype)
    ki = x["k_idx"].float()
    ki[:, : w.block_size] += PLANT * c
    x["k_idx"] = ki.to(x["k_idx"].dtype)
    x["dO"] = torch.where(keep[:, :, None, None], x["dO"], torch.zeros_like(x["dO"]))
    return x


def _heavy(w, n_rows, seed, causal=True):
    rows = sample_rows(w.B, w.N, n_rows, seed, extra=_seams(w))
    x = _heavy_inputs(w, rows, seed)
    x, sel, o, lse = _fwd(w, "normal", causal=causal, x=x)
    bs, H = w.block_size, w.H_kv
    s = sel.cpu().numpy().astype(np.int64)
    # Only the sampled rows have dO != 0 (D = 0 elsewhere); their o and lse
    # come from the oracle, so that both sides form D from the same o.
    bt = torch.tensor(rows, dtype=torch.long)
    o_in, lse_in = _oracle_output(w, x, s, rows=rows, causal=causal)
    o[bt[:, 0], bt[:, 1]] = o_in.to(DEV)
    lse[bt[:, 0], bt[:, 1]] = lse_in.to(DEV)
    gr = _bwd(w, x, sel, o, lse, causal)
    # The construction: every row past block 0 selected block 0, so block 0's
    # list holds N - bs entries per (batch, group).
    t = torch.arange(w.N, device=DEV)
    assert bool((sel == 0).any(dim=-1)[:, t >= bs].all()), "block 0 must be in every row's selection"
    lens = [int((sel[:, bs:] == j).any(dim=-1).sum()) for j in (0, 1, w.topk - 2)]
    say(f"  {len(rows)} sampled rows; list lengths over (batch, group) of blocks 0, 1, {w.topk - 2}: {lens}")
    ref = O.sparse_bwd(f32(x["q"][bt[:, 0], bt[:, 1]]), f32(x["k"]), f32(x["v"]), f32(x["dO"][bt[:, 0], bt[:, 1]]),
                       f32(x["q_idx"][bt[:, 0], bt[:, 1]]), f32(x["k_idx"]), s, bs, causal, rows=rows, o=f32(o_in))
    _check_rows(w, gr, ref, bt)
    # dk, dv per (batch, block, group); dk_idx per (batch, block).  Only
    # slices some sampled row selected can be nonzero: those are compared with
    # the oracle on the host; every other slice must be exactly zero, which is
    # checked on the device over the whole tensor.
    nblk = w.N // bs
    touched = np.zeros((w.B, nblk, H), dtype=bool)
    for (b, t_) in rows:
        for g in range(H):
            js = s[b, t_, g]
            touched[b, js[js >= 0], g] = True
    touched_b = touched.any(axis=2)
    tb = torch.from_numpy(touched).to(DEV)
    for name in ("dk", "dv"):
        a = gr[name].view(w.B, nblk, bs, H, w.d).float().abs().amax(dim=(2, 4))     # [B, nblk, H]
        resid = float(torch.where(tb, torch.zeros_like(a), a).max())
        say(f"  {name}: {int(touched.sum())} touched (block, group) slices; largest value elsewhere {resid}")
        assert resid == 0.0, name
        idx = np.argwhere(touched)
        ii = torch.from_numpy(idx).to(DEV)
        g_ = f32(gr[name].view(w.B, nblk, bs, H, w.d)[ii[:, 0], ii[:, 1], :, ii[:, 2]]).reshape(len(idx), -1)
        r_ = ref[name].reshape(w.B, nblk, bs, H, w.d)[idx[:, 0], idx[:, 1], :, idx[:, 2]].reshape(len(idx), -1)
        _cmp(name, g_, r_)
        _slices_cos(name, g_, r_, "(block, group)")
        j0 = np.nonzero((idx[:, 1] == 0))[0]
        _slices_cos(f"{name}[0]", g_[j0], r_[j0], "(batch, group) of block 0")
    a = gr["dk_idx"].view(w.B, nblk, bs * w.d_idx).abs().amax(dim=2)
    tbb = torch.from_numpy(touched_b).to(DEV)
    resid = float(torch.where(tbb, torch.zeros_like(a), a).max())
    say(f"  dk_idx: {int(touched_b.sum())} touched blocks; largest value elsewhere {resid}")
    assert resid == 0.0
    idx = np.argwhere(touched_b)
    ii = torch.from_numpy(idx).to(DEV)
    g_ = f32(gr["dk_idx"].view(w.B, nblk, bs * w.d_idx)[ii[:, 0], ii[:, 1]])
    r_ = ref["dk_idx"].reshape(w.B, nblk, bs * w.d_idx)[idx[:, 0], idx[:, 1]]
    _cmp("dk_idx", g_, r_)
    _slices_cos("dk_idx", g_, r_, "block")


def test_bwd_b4_8k_heavy_lists():
    # Block 0's list: 8064 entries per (batch, group), eight main-kernel items.
    _heavy(msa_inputs.WORKLOADS["fwdbwd-bf16-b4-n8k"], 64, 31)


def test_bwd_128k_heavy_lists():
    # 131,008 entries per group in each of the lists of blocks 0 .. 14: about
    # 128 work items each, all adding into the same dk / dv / dk_idx rows.
    _heavy(msa_inputs.WORKLOADS["fwdbwd-bf16-n128k"], 160, 41)


def test_bwd_1m_heavy_lists_across_chunks():
    # Block 0's list spans every main-kernel chunk (4 at this size), and the
    # sampled rows sit in all of them, so its dk / dv / dk_idx add up across
    # launches.
    w = msa_inputs.WORKLOADS["fwdbwd-bf16-n1m"]
    chunk = bwd_chunk_queries(w)
    say(f"  main-kernel chunk {chunk} queries: {(w.N + chunk - 1) // chunk} launches")
    _heavy(w, 64, 51)


def test_bwd_d64_heavy_lists():
    # d = 64, d_idx = 32: each wave's dQ product covers half the keys and the
    # halves meet in an LDS tile; blocks 0 .. 14 hold every query of their
    # (batch, group), 8064 entries, several work items each.
    w = msa_inputs.Workload("bwd-heavy-d64", B=2, N=8192, H_q=16, H_kv=4, d=64, d_idx=32, topk=16,
                            backward=True, seed=61)
    _heavy(w, 64, 61)


def test_bwd_g16_heavy_lists():
    # 16 query heads per group: the index work runs once per 8 steps, over
    # lists of 16256 entries.
    w = msa_inputs.Workload("bwd-heavy-g16", B=1, N=16384, H_q=32, H_kv=2, d=128, d_idx=64, topk=16,
                            backward=True, seed=62)
    _heavy(w, 64, 62)


def test_bwd_noncausal_sampled():
    # Every query sees every block; rows only (a block is chosen by most rows
    # here, which the heavy-list case below covers in full).
    w = msa_inputs.Workload("bwd-nc-8k", B=1, N=8192, H_q=32, H_kv=8, d=128, d_idx=64, topk=16,
                            backward=True, seed=63)
    _sampled(w, "normal", 96, 63, blocks=[], causal=False)


def test_bwd_noncausal_heavy_lists():
    w = msa_inputs.Workload("bwd-nc-heavy", B=2, N=8192, H_q=32, H_kv=8, d=128, d_idx=64, topk=16,
                            backward=True, seed=64)
    _heavy(w, 64, 64, causal=False)


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
