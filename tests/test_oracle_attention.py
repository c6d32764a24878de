"""Pins of the oracle's main branch (sparse softmax attention + LSE) and of its
backward with the KL index-score gradient, against things other than itself:
hand-derived values, PyTorch's fp64 CPU attention and autograd (independent
library routines), central finite differences, the streaming recurrence and
closed forms.

Pages: "How FlashAttention cuts GPU memory traffic without approximation"
('The online softmax trick', 'Exactness versus approximation', 'Training and
the backward pass', 'Architectural compatibility'); "How Flash-MSA cuts
million-token training cost with sparse-k" ('Removing the KL-divergence
bottleneck'); "How to solve the memory problem with MiniMax Sparse Attention"
('Training sparse attention')."""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import msa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _case(seed, B=2, N=40, H_q=4, H_kv=2, d=8, d_idx=4, bs=8, topk=3, causal=True, ints=False):
    rng = np.random.default_rng(seed)
    draw = (lambda s: rng.integers(-2, 3, size=s).astype(np.float64)) if ints else rng.standard_normal
    x = dict(q=draw((B, N, H_q, d)), k=draw((B, N, H_kv, d)), v=draw((B, N, H_kv, d)),
             q_idx=draw((B, N, H_kv, d_idx)), k_idx=draw((B, N, d_idx)),
             dO=draw((B, N, H_q, d)))
    x["sel"] = O.index_topk(x["q_idx"], x["k_idx"], bs, topk, causal=causal)
    x.update(B=B, N=N, H_q=H_q, H_kv=H_kv, d=d, d_idx=d_idx, bs=bs, topk=topk, causal=causal)
    return x


def _brute_mask(sel, N, bs, causal):
    """allowed[b, g, t, u]: u visible to t and blk(u) selected for (t, g)."""
    B, _, H_kv, _ = sel.shape
    m = np.zeros((B, H_kv, N, N), dtype=bool)
    for b in range(B):
        for t in range(N):
            for g in range(H_kv):
                chosen = set(int(j) for j in sel[b, t, g] if j >= 0)
                for u in range(N):
                    if (u <= t or not causal) and (u // bs) in chosen:
                        m[b, g, t, u] = True
    return m


def _torch_attention(x, mask):
    """PyTorch fp64 CPU scaled-dot-product attention with a boolean mask, GQA
    expanded by repeating each KV head over its group."""
    G = x["H_q"] // x["H_kv"]
    q = torch.tensor(x["q"]).permute(0, 2, 1, 3).requires_grad_(True)            # B,H,N,d
    k = torch.tensor(x["k"]).permute(0, 2, 1, 3).requires_grad_(True)
    v = torch.tensor(x["v"]).permute(0, 2, 1, 3).requires_grad_(True)
    kk = k.repeat_interleave(G, dim=1)
    vv = v.repeat_interleave(G, dim=1)
    am = torch.tensor(mask).repeat_interleave(G, dim=1)
    o = F.scaled_dot_product_attention(q, kk, vv, attn_mask=am)
    return q, k, v, o


def test_hand_example_forward_backward_kl():
    fx = json.load(open(os.path.join(GOLDEN, "attention_hand_example.json")))
    e = fx["expected"]
    q = np.array([0.0, 1.0]).reshape(1, 2, 1, 1)
    k = np.array([0.0, math.log(3.0)]).reshape(1, 2, 1, 1)
    v = np.array([4.0, 8.0]).reshape(1, 2, 1, 1)
    dO = np.ones((1, 2, 1, 1))
    qi = np.zeros((1, 2, 1, 1))
    ki = np.array([5.0, -7.0]).reshape(1, 2, 1)
    sel = np.zeros((1, 2, 1, 1), dtype=np.int64)
    o, lse = O.sparse_fwd(q, k, v, sel, 2, True, scale=1.0)
    np.testing.assert_allclose(o.ravel(), e["O"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse.ravel(), e["LSE"], rtol=0, atol=1e-12)
    g = O.sparse_bwd(q, k, v, dO, qi, ki, sel, 2, True, scale=1.0, scale_idx=1.0,
                     kl_weight=1.0, want_dscore=True)
    for name in ("dq", "dk", "dv", "kl", "dq_idx", "dk_idx"):
        np.testing.assert_allclose(g[name].ravel(), e[name], rtol=0, atol=1e-12, err_msg=name)
    np.testing.assert_allclose(g["dscore"][0, 1, 0, 0], e["dscore_t1"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_dense_special_case_matches_torch_sdpa(causal):
    """With k >= number of blocks the selection covers every visible block and
    the sparse branch is plain dense (causal) attention."""
    x = _case(1, N=32, bs=8, topk=4, causal=causal)
    o, lse = O.sparse_fwd(x["q"], x["k"], x["v"], x["sel"], x["bs"], causal)
    G = x["H_q"] // x["H_kv"]
    q = torch.tensor(x["q"]).permute(0, 2, 1, 3)
    kk = torch.tensor(x["k"]).permute(0, 2, 1, 3).repeat_interleave(G, 1)
    vv = torch.tensor(x["v"]).permute(0, 2, 1, 3).repeat_interleave(G, 1)
    ref = F.scaled_dot_product_attention(q, kk, vv, is_causal=causal).permute(0, 2, 1, 3)
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-12)
    s = torch.einsum("bhtd,bhud->bhtu", q, kk) / math.sqrt(x["d"])
    if causal:
        s = s.masked_fill(torch.ones(32, 32, dtype=torch.bool).triu(1), -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).permute(0, 2, 1).numpy(),
                               rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_sparse_forward_matches_masked_torch(causal):
    x = _case(2, N=56, bs=8, topk=3, causal=causal)
    o, lse = O.sparse_fwd(x["q"], x["k"], x["v"], x["sel"], x["bs"], causal)
    mask = _brute_mask(x["sel"], x["N"], x["bs"], causal)
    _, _, _, ref = _torch_attention(x, mask)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).detach().numpy(), rtol=1e-11, atol=1e-12)


def test_recurrence_equals_direct_softmax():
    x = _case(3, N=48, bs=8, topk=3)
    o1, l1 = O.sparse_fwd(x["q"], x["k"], x["v"], x["sel"], x["bs"], True)
    o2, l2 = O.sparse_fwd_recurrence(x["q"], x["k"], x["v"], x["sel"], x["bs"], True)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=1e-12, atol=1e-12)


def test_zero_query_closed_form():
    """q = 0 makes every score 0: O is the mean of V over S(t) and
    LSE = ln |S(t)|."""
    x = _case(4, N=40, bs=8, topk=3)
    q0 = np.zeros_like(x["q"])
    o, lse = O.sparse_fwd(q0, x["k"], x["v"], x["sel"], x["bs"], True)
    G = x["H_q"] // x["H_kv"]
    for b in range(x["B"]):
        for t in range(x["N"]):
            for h in range(x["H_q"]):
                g = h // G
                allowed = [u for u in range(t + 1) if (u // x["bs"]) in set(x["sel"][b, t, g].tolist())]
                np.testing.assert_allclose(o[b, t, h], x["v"][b, allowed, g].mean(0), atol=1e-12)
                assert abs(lse[b, t, h] - math.log(len(allowed))) < 1e-12


def test_probabilities_normalised():
    x = _case(5, N=40, bs=8, topk=2)
    o, lse = O.sparse_fwd(x["q"], x["k"], x["v"], x["sel"], x["bs"], True)
    scale = 1 / math.sqrt(x["d"])
    for t in (0, 7, 8, 39):
        S = O.support(x["sel"][1, t, 1], t, x["N"], x["bs"], True)
        s = scale * x["k"][1, S, 1] @ x["q"][1, t, 3]
        assert abs(np.exp(s - lse[1, t, 3]).sum() - 1) < 1e-12


def _torch_kl_grads(x, lam, scale_idx):
    """Autograd of lam * sum KL(pbar || softmax(scale_idx r)) over the support,
    with pbar the detached mean over the group's heads of the main softmax."""
    mask = torch.tensor(_brute_mask(x["sel"], x["N"], x["bs"], x["causal"]))     # B,g,t,u
    G = x["H_q"] // x["H_kv"]
    q = torch.tensor(x["q"]).permute(0, 2, 1, 3)
    k = torch.tensor(x["k"]).permute(0, 2, 1, 3).repeat_interleave(G, 1)
    s = (q @ k.transpose(-1, -2)) / math.sqrt(x["d"])
    s = s.masked_fill(~mask.repeat_interleave(G, 1), -math.inf)
    P = torch.softmax(s, -1)
    B, H_kv, N = x["B"], x["H_kv"], x["N"]
    pbar = P.reshape(B, H_kv, G, N, N).mean(2).detach()
    qi = torch.tensor(x["q_idx"]).permute(0, 2, 1, 3).requires_grad_(True)       # B,g,t,di
    ki = torch.tensor(x["k_idx"]).requires_grad_(True)                           # B,u,di
    z = scale_idx * (qi @ ki[:, None].transpose(-1, -2))
    z.retain_grad()
    zm = z.masked_fill(~mask, -math.inf)
    logp = torch.log_softmax(zm, -1)
    term = torch.where(mask, pbar * (torch.log(pbar.clamp_min(1e-300)) - logp), torch.zeros(()))
    kl = term.sum(-1)                                                          # B,g,t
    (lam * kl.sum()).backward()
    return qi.grad.permute(0, 2, 1, 3).numpy(), ki.grad.numpy(), kl.permute(0, 2, 1).detach().numpy(), z.grad, mask


@pytest.mark.parametrize("causal", [True, False])
def test_backward_matches_torch_autograd(causal):
    x = _case(6, N=48, bs=8, topk=3, causal=causal)
    lam, scale_idx = 0.7, 1 / math.sqrt(x["d_idx"])
    g = O.sparse_bwd(x["q"], x["k"], x["v"], x["dO"], x["q_idx"], x["k_idx"], x["sel"], x["bs"],
                     causal, kl_weight=lam, want_dscore=True)
    mask = _brute_mask(x["sel"], x["N"], x["bs"], causal)
    q, k, v, o = _torch_attention(x, mask)
    o.backward(torch.tensor(x["dO"]).permute(0, 2, 1, 3))
    np.testing.assert_allclose(g["dq"], q.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(g["dk"], k.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(g["dv"], v.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-10, atol=1e-11)
    dqi, dki, kl, zgrad, tmask = _torch_kl_grads(x, lam, scale_idx)
    np.testing.assert_allclose(g["dq_idx"], dqi, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(g["dk_idx"], dki, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(g["kl"], kl, rtol=1e-10, atol=1e-12)
    # dscore is the gradient w.r.t. the index logit z, laid out per (slot, offset).
    bs = x["bs"]
    for b in range(x["B"]):
        for t in range(x["N"]):
            for gg in range(x["H_kv"]):
                for slot, j in enumerate(x["sel"][b, t, gg]):
                    if j < 0:
                        assert not g["dscore"][b, t, gg, slot].any()
                        continue
                    for c in range(bs):
                        u = j * bs + c
                        want = zgrad[b, gg, t, u].item() if (u < x["N"] and tmask[b, gg, t, u]) else 0.0
                        assert abs(g["dscore"][b, t, gg, slot, c] - want) < 1e-12


def test_kl_gradient_identity_and_zero_sum():
    """Per row the index-logit gradient is lam*(p_px - pbar): it sums to zero,
    and vanishes when the student equals the teacher."""
    x = _case(7, N=32, bs=8, topk=2, B=1)
    g = O.sparse_bwd(x["q"], x["k"], x["v"], x["dO"], x["q_idx"], x["k_idx"], x["sel"], x["bs"],
                     True, kl_weight=1.0, want_dscore=True)
    np.testing.assert_allclose(g["dscore"].sum(axis=(3, 4)), 0.0, atol=1e-12)
    # teacher == student: with q = 0 the main softmax is uniform on S(t); with
    # q_idx = 0 so is the index softmax, so every gradient of the KL is zero.
    z = O.sparse_bwd(np.zeros_like(x["q"]), x["k"], x["v"], x["dO"], np.zeros_like(x["q_idx"]),
                     x["k_idx"], x["sel"], x["bs"], True, want_dscore=True)
    assert np.abs(z["dscore"]).max() < 1e-15
    assert np.abs(z["dq_idx"]).max() < 1e-12 and np.abs(z["dk_idx"]).max() < 1e-12
    assert np.abs(z["kl"]).max() < 1e-15


def test_finite_differences_all_gradients():
    """Central differences (fp64, h = 1e-6) of L = sum dO*O for q, k, v and of
    lam*sum KL for q_idx, k_idx, with the selection held fixed."""
    x = _case(8, B=1, N=24, H_q=2, H_kv=1, d=4, d_idx=3, bs=4, topk=3)
    lam = 1.3
    g = O.sparse_bwd(x["q"], x["k"], x["v"], x["dO"], x["q_idx"], x["k_idx"], x["sel"], x["bs"],
                     True, kl_weight=lam)

    def main_loss(q, k, v):
        o, _ = O.sparse_fwd(q, k, v, x["sel"], x["bs"], True)
        return float((o * x["dO"]).sum())

    def kl_loss(qi, ki):
        r = O.sparse_bwd(x["q"], x["k"], x["v"], x["dO"], qi, ki, x["sel"], x["bs"], True)
        return lam * float(r["kl"].sum())

    h = 1e-6
    rng = np.random.default_rng(0)
    for name, grad, f, args, pos in [
        ("q", g["dq"], main_loss, ("q", "k", "v"), 0),
        ("k", g["dk"], main_loss, ("q", "k", "v"), 1),
        ("v", g["dv"], main_loss, ("q", "k", "v"), 2),
        ("q_idx", g["dq_idx"], kl_loss, ("q_idx", "k_idx"), 0),
        ("k_idx", g["dk_idx"], kl_loss, ("q_idx", "k_idx"), 1),
    ]:
        base = [x[a].copy() for a in args]
        flat = base[pos].reshape(-1)
        for idx in rng.choice(flat.size, size=12, replace=False):
            old = flat[idx]
            flat[idx] = old + h
            fp = f(*base)
            flat[idx] = old - h
            fm = f(*base)
            flat[idx] = old
            fd = (fp - fm) / (2 * h)
            assert abs(fd - grad.reshape(-1)[idx]) < 1e-6 * max(1.0, abs(fd)), (name, idx, fd)


def test_sampled_rows_agree_with_full():
    """The row-sampled entry points give the same rows as the full run."""
    x = _case(9, N=40, bs=8, topk=3)
    rows = [(1, 0), (0, 17), (1, 39)]
    full_o, full_l = O.sparse_fwd(x["q"], x["k"], x["v"], x["sel"], x["bs"], True)
    o, l = O.sparse_fwd(x["q"], x["k"], x["v"], x["sel"], x["bs"], True, rows=rows)
    for i, (b, t) in enumerate(rows):
        np.testing.assert_array_equal(o[i], full_o[b, t])
        np.testing.assert_array_equal(l[i], full_l[b, t])
    sel_rows = O.index_topk(x["q_idx"], x["k_idx"], x["bs"], x["topk"], rows=rows)
    for i, (b, t) in enumerate(rows):
        assert sel_rows[i].tolist() == x["sel"][b, t].tolist()


def test_backward_D_from_the_stored_output():
    """D = rowsum(dO * o) when the forward's output is passed in, as the
    FlashAttention backward forms it ('Training and the backward pass').
    With the exact output it equals sum_u P dP, so every gradient matches the
    default; an error E in o shifts only the main-branch gradients, by the
    closed form dS_u -> dS_u - (dO . E) P_u: dq moves by
    -scale (dO . E) sum_u P_u k_u (sum_u P_u k_u = attention with the keys as
    values, from torch's SDPA), dv and the index gradients do not move."""
    x = _case(12, N=48, bs=8, topk=3)
    args = (x["q"], x["k"], x["v"], x["dO"], x["q_idx"], x["k_idx"], x["sel"], x["bs"], True)
    base = O.sparse_bwd(*args)
    o, _ = O.sparse_fwd(x["q"], x["k"], x["v"], x["sel"], x["bs"], True)
    same = O.sparse_bwd(*args, o=o)
    for name in ("dq", "dk", "dv", "dq_idx", "dk_idx", "kl"):
        np.testing.assert_allclose(same[name], base[name], rtol=1e-10, atol=1e-12)
    rng = np.random.default_rng(3)
    E = 1e-3 * rng.standard_normal(o.shape)
    moved = O.sparse_bwd(*args, o=o + E)
    mask = _brute_mask(x["sel"], x["N"], x["bs"], True)
    xk = dict(x, v=x["k"])
    _, _, _, pk = _torch_attention(xk, mask)                                    # B,H,N,d: sum_u P k_u
    pk = pk.detach().permute(0, 2, 1, 3).numpy()
    delta = (x["dO"] * E).sum(axis=-1, keepdims=True)                           # B,N,H_q,1
    scale = 1 / math.sqrt(x["d"])
    np.testing.assert_allclose(moved["dq"] - base["dq"], -scale * delta * pk, rtol=1e-8, atol=1e-13)
    np.testing.assert_allclose(moved["dv"], base["dv"], rtol=0, atol=1e-13)
    for name in ("dq_idx", "dk_idx", "kl"):
        np.testing.assert_allclose(moved[name], base[name], rtol=0, atol=1e-13)
    assert np.abs(moved["dk"] - base["dk"]).max() > 1e-6      # dk moves too (by -scale (dO.E) P_u q)
