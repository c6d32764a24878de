"""Oracle for MiniMax Sparse Attention (MSA) over grouped-query attention.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the test-suite, the smoke
check and the CPU-baseline leg of the benchmark may import this module.  The
library (libmsa) and its Python binding never import, call or link it, and it
imports nothing from them.

A plain, slow, fp64 NumPy statement of what the method computes, written row
by row from the definitions so that a reader can check it against the pages
by eye.  Inputs are upcast to float64 from the exact bits handed to the GPU.

Pages cited (title; section):
  [FMSA] "How Flash-MSA cuts million-token training cost with sparse-k"
  [FA]   "How FlashAttention cuts GPU memory traffic without approximation"
  [MSA]  "How to solve the memory problem with MiniMax Sparse Attention"

Shapes (row-major, as the library takes them):
  q_idx [B, N, H_kv, d_idx]   one index query per GQA group
  k_idx [B, N, d_idx]         one index key per token, shared by all groups
  q     [B, N, H_q, d]        k, v [B, N, H_kv, d]     head h uses group h // G
  block_idx [B, N, H_kv, topk] int64/int32, ascending, -1 padded

Readings taken where the pages leave a step open (each is listed with its
reason in the design notes of the repository):
  * index score = plain dot product of index query and index key; no scale or
    activation is needed for selection ([MSA] "How the indexer works").
  * max-pool over the *visible* tokens of a block only; the diagonal block is
    pooled over u <= t.
  * selection = the query's own block plus the best (k-1) other visible blocks
    ordered by (pooled score descending, block index ascending); output sorted
    ascending and padded with -1 when fewer than k blocks are visible.
  * main-branch scale 1/sqrt(d) unless given; LSE in natural log.
  * KL(pbar || p_px) over the selected support S(t), with pbar the main-branch
    softmax averaged over the group's heads and p_px = softmax(scale_idx * r)
    over the same support; dscore = lam * (p_px - pbar).
  * no KL gradient into q/k/v (detached teacher); no main-loss gradient into
    q_idx/k_idx (top-k has no gradient).

Parity pins live in tests/test_oracle_*.py.  Conventions fixed by the API
rather than by the pages (the KL weight lam and its sum over rows, the default
scale_idx = 1/sqrt(d_idx), the LSE base, the order and padding of block_idx)
are "parity unpinned": the pins check the mathematics, not those choices.
"""

from __future__ import annotations

import math

import numpy as np

NEG_INF = -np.inf


# --------------------------------------------------------------------------
# Small helpers: visibility, blocks, support.
# --------------------------------------------------------------------------

def n_blocks(N: int, block_size: int) -> int:
    """Number of KV blocks of `block_size` tokens covering N tokens."""
    return (N + block_size - 1) // block_size


def visible_keys(t: int, N: int, causal: bool) -> np.ndarray:
    """Keys that query t may attend to: u <= t when causal, all u otherwise
    ([FA] "Architectural compatibility": causal masking)."""
    return np.arange(t + 1 if causal else N)


def block_keys(j: int, N: int, block_size: int) -> np.ndarray:
    """Token positions of KV block j ([FMSA] "Block sparsity mechanism")."""
    return np.arange(j * block_size, min((j + 1) * block_size, N))


def support(sel_row: np.ndarray, t: int, N: int, block_size: int, causal: bool) -> np.ndarray:
    """S(t): the visible keys inside the selected blocks of query t, ascending.

    The main branch runs an exact softmax over exactly these tokens
    ([MSA] "Two-stage process: Index-Branch and Main-Branch")."""
    keys = [block_keys(int(j), N, block_size) for j in sorted(int(x) for x in sel_row if x >= 0)]
    if not keys:
        return np.zeros(0, dtype=np.int64)
    u = np.concatenate(keys)
    if causal:
        u = u[u <= t]
    return u


# --------------------------------------------------------------------------
# A1 + A2 + A3: index scores, block max-pool, top-k with the own block forced.
# --------------------------------------------------------------------------

def index_scores_rows(q_idx_rows: np.ndarray, k_idx_b: np.ndarray, ts: np.ndarray,
                      causal: bool) -> np.ndarray:
    """r[i, u] = q_idx_rows[i] . k_idx_b[u] for the visible u of query ts[i],
    -inf elsewhere ([MSA] "How the indexer works": the index query of the
    group scores every visible token against the shared index key)."""
    q = np.asarray(q_idx_rows, dtype=np.float64)
    k = np.asarray(k_idx_b, dtype=np.float64)
    r = q @ k.T                                   # [rows, N]
    if causal:
        u = np.arange(k.shape[0])[None, :]
        r = np.where(u <= np.asarray(ts)[:, None], r, NEG_INF)
    return r


def block_maxpool_rows(r: np.ndarray, block_size: int) -> np.ndarray:
    """pooled[i, j] = max of r[i, u] over the tokens u of block j (-inf marks
    an invisible block) ([FMSA] "Block sparsity mechanism": KV pairs are chosen
    in blocks by max-pooling the proxy scores)."""
    rows, N = r.shape
    nb = n_blocks(N, block_size)
    padded = np.full((rows, nb * block_size), NEG_INF)
    padded[:, :N] = r
    return padded.reshape(rows, nb, block_size).max(axis=2)


def select_blocks_row(pooled_row: np.ndarray, t: int, block_size: int, topk: int,
                      causal: bool) -> np.ndarray:
    """Block selection for one (query, group) row.

    The query's own block is always kept; the other visible blocks are ranked
    by pooled score, higher first, ties to the lower block index; the best
    topk-1 of them join the own block ([MSA] "How the indexer works"; budget of
    k blocks per query from "Two-stage process").  No softmax is taken: it is
    monotone, so it cannot change the order ([MSA] "Kernel optimizations",
    exp-free top-k).  Output ascending, padded with -1."""
    nb = pooled_row.shape[0]
    own = t // block_size
    last = own if causal else nb - 1
    cands = [j for j in range(last + 1) if j != own]
    # np.lexsort sorts by the last key first: primary -pooled, secondary j.
    cands_arr = np.array(cands, dtype=np.int64)
    if cands_arr.size:
        order = np.lexsort((cands_arr, -pooled_row[cands_arr]))
        chosen = cands_arr[order[: max(topk - 1, 0)]]
    else:
        chosen = cands_arr
    sel = np.sort(np.concatenate([[own], chosen]).astype(np.int64))
    out = np.full(topk, -1, dtype=np.int64)
    out[: sel.size] = sel
    return out


def index_topk(q_idx: np.ndarray, k_idx: np.ndarray, block_size: int, topk: int,
               causal: bool = True, rows=None, want_pooled: bool = False,
               chunk: int = 256):
    """Index branch for every (b, t, g) row (or for `rows`, a list of (b, t)).

    Returns block_idx [B, N, H_kv, topk] (or [len(rows), H_kv, topk]) and, when
    asked, pooled scores of the same leading shape with nblk columns."""
    q_idx = np.asarray(q_idx)
    k_idx = np.asarray(k_idx)
    B, N, d_idx = k_idx.shape
    H_kv = q_idx.shape[-2]
    nb = n_blocks(N, block_size)
    if rows is None:
        bt = [(b, t) for b in range(B) for t in range(N)]
    else:
        bt = [(int(b), int(t)) for b, t in rows]
    # With `rows`, q_idx may be compact: [len(rows), H_kv, d_idx].
    compact = rows is not None and q_idx.ndim == 3
    out = np.full((len(bt), H_kv, topk), -1, dtype=np.int64)
    pooled_out = np.full((len(bt), H_kv, nb), NEG_INF) if want_pooled else None
    for b in sorted({b for b, _ in bt}):
        idx = [i for i, (bb, _) in enumerate(bt) if bb == b]
        for c0 in range(0, len(idx), chunk):
            ii = idx[c0:c0 + chunk]
            ts = np.array([bt[i][1] for i in ii])
            for g in range(H_kv):
                qrows = q_idx[ii, g, :] if compact else q_idx[b, ts, g, :]
                r = index_scores_rows(qrows, k_idx[b], ts, causal)
                pooled = block_maxpool_rows(r, block_size)
                for m, i in enumerate(ii):
                    out[i, g] = select_blocks_row(pooled[m], int(ts[m]), block_size, topk, causal)
                    if want_pooled:
                        pooled_out[i, g] = pooled[m]
    if rows is None:
        out = out.reshape(B, N, H_kv, topk)
        if want_pooled:
            pooled_out = pooled_out.reshape(B, N, H_kv, nb)
    return (out, pooled_out) if want_pooled else out


# --------------------------------------------------------------------------
# FP8 E4M3 index inputs ([MSA] "Kernel optimizations": a lighter indexer
# format).  The index branch is then the same definition over the decoded
# values; only the decoding is new.
# --------------------------------------------------------------------------

def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """Values of OCP FP8 E4M3 codes (the finite form: 1 sign bit, 4 exponent
    bits with bias 7, 3 mantissa bits, no infinities, S.1111.111 is NaN), as
    float64: exponent field 0 is subnormal, m / 8 * 2^-6; otherwise
    (1 + m / 8) * 2^(e - 7)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    out = sign * mag
    return np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, out)


# --------------------------------------------------------------------------
# A5: exact softmax attention over the selected support, with LSE.
# --------------------------------------------------------------------------

def _attend(qg: np.ndarray, kS: np.ndarray, vS: np.ndarray, scale: float):
    """Exact softmax attention of a few query rows over the keys kS:
    O = softmax(scale * q k^T) v, LSE = max + ln(sum exp(s - max))
    ([FA] "Exactness versus approximation": the dense formula;
    "Training and the backward pass": the row log-sum-exp statistic)."""
    s = scale * (qg @ kS.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    ell = e.sum(axis=1, keepdims=True)
    p = e / ell
    return p @ vS, (m + np.log(ell))[:, 0], p


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def sparse_fwd(q, k, v, block_idx, block_size: int, causal: bool = True,
               scale: float | None = None, rows=None):
    """Main branch ([MSA] "Two-stage process"; [FMSA] "Kernel design and
    execution": output plus stored LSE).  Each head h of group g = h // G
    attends over S(t) of (t, g), the support shared by the group's heads
    ([MSA] "Two-stage process": selection is joint for a group's queries).

    Returns O [B,N,H_q,d] and LSE [B,N,H_q] (or [len(rows), ...])."""
    # Arrays keep their (exact) input precision; gathered rows are upcast to
    # fp64 where they are used.  With `rows`, q may be compact
    # [len(rows), H_q, d].
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    block_idx = np.asarray(block_idx)
    B, N, H_kv, d = k.shape
    H_q = q.shape[-2]
    G = H_q // H_kv
    scale = default_scale(d) if scale is None else scale
    bt = [(b, t) for b in range(B) for t in range(N)] if rows is None else [(int(b), int(t)) for b, t in rows]
    compact = rows is not None and q.ndim == 3
    f64 = lambda a: np.asarray(a, dtype=np.float64)
    O = np.zeros((len(bt), H_q, v.shape[3]))
    L = np.zeros((len(bt), H_q))
    for i, (b, t) in enumerate(bt):
        qrow = q[i] if compact else q[b, t]
        for g in range(H_kv):
            S = support(block_idx[b, t, g], t, N, block_size, causal)
            hs = slice(g * G, (g + 1) * G)
            o, lse, _ = _attend(f64(qrow[hs]), f64(k[b, S, g]), f64(v[b, S, g]), scale)
            O[i, hs] = o
            L[i, hs] = lse
    if rows is None:
        return O.reshape(B, N, H_q, -1), L.reshape(B, N, H_q)
    return O, L


def sparse_fwd_recurrence(q, k, v, block_idx, block_size: int, causal: bool = True,
                          scale: float | None = None):
    """The same main branch computed the streaming way: blocks in ascending
    order, each folded into the running (m, l, a) state by the blockwise merge
    recurrence ([FA] "The online softmax trick": new max, rescale factor
    alpha = exp(m - m'), p = exp(s - m'), l' = alpha l + sum p,
    a' = alpha a + p^T V; finally O = a / l).  Used to cross-check the direct
    softmax of sparse_fwd."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, N, H_q, d = q.shape
    H_kv = k.shape[2]
    G = H_q // H_kv
    scale = default_scale(d) if scale is None else scale
    O = np.zeros((B, N, H_q, v.shape[3]))
    L = np.zeros((B, N, H_q))
    for b in range(B):
        for t in range(N):
            for h in range(H_q):
                g = h // G
                m, ell, a = NEG_INF, 0.0, np.zeros(v.shape[3])
                for j in sorted(int(x) for x in block_idx[b, t, g] if x >= 0):
                    u = block_keys(j, N, block_size)
                    if causal:
                        u = u[u <= t]
                    if u.size == 0:
                        continue
                    s = scale * (k[b, u, g] @ q[b, t, h])
                    m_new = max(m, s.max())
                    alpha = math.exp(m - m_new) if m != NEG_INF else 0.0
                    p = np.exp(s - m_new)
                    ell = alpha * ell + p.sum()
                    a = alpha * a + p @ v[b, u, g]
                    m = m_new
                O[b, t, h] = a / ell
                L[b, t, h] = m + math.log(ell)
    return O, L


# --------------------------------------------------------------------------
# A6 + A7: backward of the main branch and the KL index-score gradient.
# --------------------------------------------------------------------------

def sparse_bwd(q, k, v, dO, q_idx, k_idx, block_idx, block_size: int,
               causal: bool = True, scale: float | None = None,
               scale_idx: float | None = None, kl_weight: float = 1.0,
               rows=None, want_dscore: bool = False, o=None):
    """Gradients of the main branch plus the KL-alignment gradient of the index
    branch, all on the selected support.

    Main branch ([FA] "Training and the backward pass"): rebuild P from the
    scores, dV += P^T dO, dP = dO V^T; the softmax Jacobian gives
    dS = P * (dP - D) with D = sum_u P dP, then dQ = scale dS K and
    dK += scale dS^T Q.  dK and dV of a group sum over its G heads.
    When the forward's output `o` is given (as the backward receives it,
    [B,N,H_q,d] or compact per row), D is the row sum of dO * o, the way the
    FlashAttention backward forms it from the stored output; in exact
    arithmetic the two are equal (o = sum_u P v_u, so dO . o = sum_u P dP).

    Index branch ([FMSA] "Removing the KL-divergence bottleneck"; [MSA]
    "Training sparse attention"): teacher pbar = mean over the group's heads of
    the main-branch P (detached: nothing flows back into q/k/v), student
    p_px = softmax(scale_idx * r) over S(t); the gradient of KL(pbar || p_px)
    with respect to the index logit is p_px - pbar, scaled by kl_weight;
    dq_idx = scale_idx sum_u dz_u k_idx_u, dk_idx_u += scale_idx dz_u q_idx.

    Returns a dict with dq, dk, dv, dq_idx, dk_idx, kl (per (b,t,g) row,
    unweighted) and, if asked, dscore [B,N,H_kv,topk,block_size] holding
    kl_weight*(p_px - pbar) at (slot, offset) of key block_idx[slot]*bs+offset,
    zero at masked or padded positions.  With `rows`, only those (b, t) rows
    contribute (dq/dq_idx/kl/dscore are returned for those rows only; dk, dv,
    dk_idx hold those rows' contributions)."""
    # Per-row fp64 upcast as in sparse_fwd; with `rows`, q, dO and q_idx may
    # be compact ([len(rows), ...]).  dk, dv, dk_idx are full-size fp64.
    q, k, v, dO = np.asarray(q), np.asarray(k), np.asarray(v), np.asarray(dO)
    q_idx, k_idx = np.asarray(q_idx), np.asarray(k_idx)
    block_idx = np.asarray(block_idx)
    B, N, H_kv, d = k.shape
    H_q = q.shape[-2]
    G = H_q // H_kv
    topk = block_idx.shape[3]
    d_idx = k_idx.shape[2]
    scale = default_scale(d) if scale is None else scale
    scale_idx = default_scale(d_idx) if scale_idx is None else scale_idx
    bt = [(b, t) for b in range(B) for t in range(N)] if rows is None else [(int(b), int(t)) for b, t in rows]
    compact = rows is not None and q.ndim == 3
    f64 = lambda a: np.asarray(a, dtype=np.float64)
    R = len(bt)
    dq = np.zeros((R, H_q, d))
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    dq_idx = np.zeros((R, H_kv, d_idx))
    dk_idx = np.zeros(k_idx.shape)
    kl = np.zeros((R, H_kv))
    dscore = np.zeros((R, H_kv, topk, block_size)) if want_dscore else None
    for i, (b, t) in enumerate(bt):
        qrow = q[i] if compact else q[b, t]
        dorow = dO[i] if compact else dO[b, t]
        qirow = q_idx[i] if compact else q_idx[b, t]
        orow = None if o is None else (o[i] if compact else o[b, t])
        for g in range(H_kv):
            S = support(block_idx[b, t, g], t, N, block_size, causal)
            hs = slice(g * G, (g + 1) * G)
            Qg, dOg = f64(qrow[hs]), f64(dorow[hs])
            KS, VS = f64(k[b, S, g]), f64(v[b, S, g])
            _, _, P = _attend(Qg, KS, VS, scale)          # [G, |S|]
            dP = dOg @ VS.T
            if orow is None:
                D = (P * dP).sum(axis=1, keepdims=True)
            else:
                D = (dOg * f64(orow[hs])).sum(axis=1, keepdims=True)
            dS = P * (dP - D)
            dq[i, hs] = scale * dS @ KS
            # S holds distinct keys, so fancy-index accumulation is exact.
            dk[b, S, g] += scale * dS.T @ Qg
            dv[b, S, g] += P.T @ dOg
            # KL-alignment on the same support.
            pbar = P.mean(axis=0)
            qi_g, kS_idx = f64(qirow[g]), f64(k_idx[b, S])
            z = scale_idx * (kS_idx @ qi_g)
            z = z - z.max()
            p_px = np.exp(z) / np.exp(z).sum()
            dz = kl_weight * (p_px - pbar)
            dq_idx[i, g] = scale_idx * dz @ kS_idx
            dk_idx[b, S] += scale_idx * np.outer(dz, qi_g)
            nz = pbar > 0
            kl[i, g] = float(np.sum(pbar[nz] * (np.log(pbar[nz]) - np.log(p_px[nz]))))
            if want_dscore:
                for slot in range(topk):
                    j = int(block_idx[b, t, g, slot])
                    if j < 0:
                        continue
                    u = j * block_size + np.arange(block_size)
                    pos = np.minimum(np.searchsorted(S, u), S.size - 1)
                    hit = S[pos] == u
                    dscore[i, g, slot, hit] = dz[pos[hit]]
    out = dict(dk=dk, dv=dv, dk_idx=dk_idx)
    if rows is None:
        out.update(dq=dq.reshape(B, N, H_q, d), dq_idx=dq_idx.reshape(B, N, H_kv, d_idx),
                   kl=kl.reshape(B, N, H_kv))
        if want_dscore:
            out["dscore"] = dscore.reshape(B, N, H_kv, topk, block_size)
    else:
        out.update(dq=dq, dq_idx=dq_idx, kl=kl)
        if want_dscore:
            out["dscore"] = dscore
    return out


# --------------------------------------------------------------------------
# Counting facts used by the measurement and by the pins.
# --------------------------------------------------------------------------

def support_size(t: int, block_size: int, topk: int) -> int:
    """|S(t)| for causal selection with the own block forced and every other
    selected block fully visible: min(k-1, blk(t)) full blocks plus the
    t mod bs + 1 visible tokens of the own block."""
    return min(topk - 1, t // block_size) * block_size + (t % block_size) + 1

