"""Shared helpers of the GPU parity tests: device gate, metrics, near-tie
analysis of block selections and row sampling.  Imported by the gpu tests
only (not collected by pytest itself)."""

from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import msa_inputs
from oracle import msa_oracle as O

# Unit roundoff assumed for the matrix unit's fp32 accumulation.  The order
# and the rounding mode of the sums inside an MFMA instruction are not
# documented; a directed (truncating) rounding has unit roundoff 2^-23,
# twice the 2^-24 of round-to-nearest, so the bounds below use 2^-23.
U_MFMA = 2.0 ** -23
# The FP8 (E4M3) matrix unit accumulates its products with less precision
# than an fp32 sum (its internal format is not documented either): on gfx950,
# N(0,1) inputs rounded to E4M3 gave score errors up to 2^-21.3 * d_idx *
# sum_i |q_i k_i| (3.2 times the 2^-23 bound; bf16 inputs stay within 1% of
# it).  FP8 index scores are held to u = 2^-20, the measurement with a 2.5x
# margin.
U_FP8 = 2.0 ** -20


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_sparse_attention_branch_amd as msa
    msa.load_library()          # loud failure if the library is missing
    return msa


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def cosine(a, b):
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    return float(a @ b / math.sqrt((a @ a) * (b @ b)))


def max_rel(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.abs(got - ref).max() / np.abs(ref).max())


def f32(t: torch.Tensor):
    """Exact host copy (bf16 and fp32 both fit in fp32)."""
    return t.detach().float().cpu().numpy()


def gamma(n: int, u: float = U_MFMA) -> float:
    """Higham's gamma_n = n u / (1 - n u): an n-term dot product computed in
    floating point (products and sums rounded, any order) differs from the
    exact one by at most gamma_n * sum_i |x_i y_i|."""
    return n * u / (1 - n * u)


def selection_equivalent(gpu_sel, ref_sel, ref_pooled_row, t, block_size, tol):
    """True when the GPU's selection equals the oracle's, or differs only by
    swapping blocks whose oracle pooled scores lie within `tol` of each
    other (a near tie under fp32 accumulation).  Also checks validity: own
    block present, ascending, distinct, -1 padding at the end."""
    g = [int(x) for x in gpu_sel]
    r = [int(x) for x in ref_sel]
    if g == r:
        return True
    valid = [x for x in g if x >= 0]
    if valid != sorted(set(valid)) or g[len(valid):] != [-1] * (len(g) - len(valid)):
        return False
    own = t // block_size
    if own not in valid or len(valid) != len([x for x in r if x >= 0]):
        return False
    gv = sorted((ref_pooled_row[j] for j in valid if j != own), reverse=True)
    rv = sorted((ref_pooled_row[j] for j in r if j >= 0 and j != own), reverse=True)
    return all(abs(a - b) <= tol for a, b in zip(gv, rv))


def score_bound(q_idx_row, k_idx_b, t, causal, d_idx, u=U_MFMA):
    """gamma_{d_idx} * max_u sum_i |q_i k_i| over the row's visible keys: how
    far an fp32-accumulated index score, and so a block max of such scores,
    may sit from the exact value."""
    a = np.abs(np.asarray(q_idx_row, dtype=np.float64))
    kk = np.abs(np.asarray(k_idx_b[: t + 1] if causal else k_idx_b, dtype=np.float64))
    return gamma(d_idx, u) * float((kk @ a).max())


def score_bounds(q_idx_b, k_idx_b, causal, d_idx, chunk=256, u=U_MFMA):
    """score_bound of every row of one batch entry at once: q_idx_b [N, H_kv,
    d_idx], k_idx_b [N, d_idx] -> [N, H_kv]."""
    a = np.abs(np.asarray(q_idx_b, dtype=np.float64))
    kk = np.abs(np.asarray(k_idx_b, dtype=np.float64))
    N = a.shape[0]
    out = np.empty(a.shape[:2])
    for t0 in range(0, N, chunk):
        t1 = min(t0 + chunk, N)
        m = np.einsum("thi,ui->thu", a[t0:t1], kk)
        if causal:
            hidden = np.arange(t1 - t0)[:, None] + t0 < np.arange(N)[None, :]    # u > t
            m[np.broadcast_to(hidden[:, None, :], m.shape)] = 0.0
        out[t0:t1] = m.max(axis=2)
    return gamma(d_idx, u) * out


def row_tolerance(q_idx_row, k_idx_b, t, causal, d_idx, u=U_MFMA):
    """Largest gap between two blocks' exact pooled scores that the GPU may
    order the other way: each pooled score may move by score_bound, so twice
    that."""
    return 2.0 * score_bound(q_idx_row, k_idx_b, t, causal, d_idx, u)


def sample_rows(B, N, n, seed, extra=()):
    """Seeded, stratified (b, t) rows: the edges of the selection budget plus
    `extra` positions plus uniform picks."""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 127, 128, 1919, 1920, 2047, 2048, N // 2, N - 129, N - 128, N - 1] + list(extra)
    fixed = sorted({t for t in fixed if 0 <= t < N})
    rows = [(b, t) for b in range(B) for t in fixed]
    while len(rows) < n * B:
        rows.append((int(rng.integers(B)), int(rng.integers(N))))
    return sorted(set(rows))


def _super_span(w: msa_inputs.Workload) -> int:
    nblk = w.N // w.block_size
    sb = 1
    while sb < 64 and ((nblk + sb - 1) // sb + 1) * nblk * 4 * w.B * w.H_kv > (256 << 20):
        sb *= 2
    return sb * w.block_size


def _chunk(w: msa_inputs.Workload, per_q: int, q_cap: int | None = None) -> int:
    span = _super_span(w)
    q = (40 << 30) // per_q
    if q_cap is not None:
        q = min(q, q_cap)
    q -= q % span
    return max(span, min(q, w.N))


def fwd_chunk_queries(w: msa_inputs.Workload) -> int:
    """Queries per forward launch, as the library plans it (for sampling rows
    at chunk seams): partials of at most 40 GiB, and at most 128 MiB of q rows
    per (batch, group) slice of the chunk."""
    esz = 2 if w.dtype == "bf16" else 4
    G = w.H_q // w.H_kv
    return _chunk(w, w.B * w.H_q * w.topk * (w.d * esz + 4), (128 << 20) // (G * w.d * esz))


def bwd_chunk_queries(w: msa_inputs.Workload) -> int:
    """Queries per backward main-kernel launch (bf16 dQ partials of at most
    40 GiB), for sampling rows at its chunk seams."""
    return _chunk(w, w.B * w.H_q * w.topk * w.d * 2)
