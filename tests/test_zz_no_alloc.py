"""GPU check of msa_sparse_fwd_noalloc (the forward with the library's fixed
device scratch instead of a workspace) against msa_sparse_fwd, through the C
ABI.  Bar: o and lse equal bit for bit, since both run the same kernels on
the same rows and o and lse do not depend on how queries are grouped into
launches.  Calls run back to back on one device and share its scratch: a
large problem whose partials do not fit (several query chunks, the last one
ragged), then a smaller one, then the large one again on fresh inputs with
the device's free memory unchanged across the call."""

import pytest
import torch

import msa_inputs
from tests.gpu_helpers import need_gpu, say

pytestmark = pytest.mark.gpu

# B=1, N=8K, 32/8 heads, d=128, topk 16: about 1.1 GB of partials, so the
# 128 MiB scratch takes the queries in 10 launches (nine of 896, one of 128).
LARGE = msa_inputs.WORKLOADS["fwd-bf16-n8k"]
SMALL = msa_inputs.Workload("noalloc-small", B=2, N=1024, H_q=8, H_kv=2, d=64, d_idx=32, topk=4, seed=91)


def _both(msa, w, seed=None):
    say(f"[noalloc] {w.name} B={w.B} N={w.N} H={w.H_q}/{w.H_kv} d={w.d} topk={w.topk} seed={seed}")
    x = msa_inputs.make_inputs(w, "normal", seed=seed, device="cuda")
    sel = msa.index_topk(x["q_idx"], x["k_idx"], topk=w.topk)
    ref_o, ref_l = msa.sparse_fwd(x["q"], x["k"], x["v"], sel, d_idx=w.d_idx)
    o = torch.full_like(ref_o, float("nan"))
    lse = torch.full_like(ref_l, float("nan"))
    torch.cuda.synchronize()
    return x, sel, ref_o, ref_l, o, lse


def _check(ref_o, ref_l, o, lse):
    assert torch.equal(o, ref_o), f"o differs at {int((o != ref_o).sum())} elements"
    assert torch.equal(lse, ref_l), f"lse differs at {int((lse != ref_l).sum())} elements"


def test_noalloc_forward_matches_the_workspace_forward():
    msa = need_gpu()
    for w, seed in ((LARGE, None), (SMALL, None)):
        x, sel, ref_o, ref_l, o, lse = _both(msa, w, seed)
        got_o, got_l = msa.sparse_fwd_noalloc(x["q"], x["k"], x["v"], sel, o, lse, d_idx=w.d_idx)
        torch.cuda.synchronize()
        assert got_o is o and got_l is lse
        _check(ref_o, ref_l, o, lse)
        say("  equal")

    # The large problem again, on fresh inputs: what the earlier calls left in
    # the scratch does not leak into the result, and the call allocates
    # nothing (free device memory is the same before and after it).
    x, sel, ref_o, ref_l, o, lse = _both(msa, LARGE, seed=LARGE.seed + 1)
    free_before = torch.cuda.mem_get_info()[0]
    msa.sparse_fwd_noalloc(x["q"], x["k"], x["v"], sel, o, lse, d_idx=LARGE.d_idx)
    torch.cuda.synchronize()
    free_after = torch.cuda.mem_get_info()[0]
    _check(ref_o, ref_l, o, lse)
    assert free_after == free_before, (free_before, free_after)
    say("  equal, free memory unchanged")
