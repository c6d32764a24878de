"""The Python binding checks every tensor shape against the others before the
library is loaded or called: the kernels size every buffer from q (and
k / block_idx / q_idx), so a mismatched tensor would be read or written past
its end.  CPU tensors suffice here: the shape check runs first, so a
mismatch raises ValueError naming the tensor, and a consistent set of CPU
tensors gets as far as the device check."""

import pytest
import torch

from block_sparse_attention_branch_amd import binding as bnd

B, N, HQ, HKV, D, DI, K = 2, 256, 8, 2, 64, 32, 4


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def refuse(*a, **kw):
        raise AssertionError("the library must not be reached with invalid shapes")
    monkeypatch.setattr(bnd, "load_library", refuse)


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def fwd_args(**over):
    a = dict(q=bf(B, N, HQ, D), k=bf(B, N, HKV, D), v=bf(B, N, HKV, D),
             block_idx=torch.zeros((B, N, HKV, K), dtype=torch.int32))
    a.update(over)
    return a


def bwd_args(**over):
    a = dict(q=bf(B, N, HQ, D), k=bf(B, N, HKV, D), v=bf(B, N, HKV, D), o=bf(B, N, HQ, D),
             dO=bf(B, N, HQ, D), lse=torch.zeros((B, N, HQ)),
             block_idx=torch.zeros((B, N, HKV, K), dtype=torch.int32),
             q_idx=bf(B, N, HKV, DI), k_idx=bf(B, N, DI))
    a.update(over)
    return a


def test_consistent_shapes_reach_the_device_check():
    with pytest.raises(ValueError, match="device tensor"):
        bnd.index_topk(bf(B, N, HKV, DI), bf(B, N, DI), topk=K)
    with pytest.raises(ValueError, match="device tensor"):
        bnd.sparse_fwd(**fwd_args())
    with pytest.raises(ValueError, match="device tensor"):
        bnd.sparse_bwd(**bwd_args())


@pytest.mark.parametrize("q_idx,k_idx,name", [
    (bf(B, N, HKV, DI), bf(B, N + 128, DI), "k_idx"),      # N differs
    (bf(B, N, HKV, DI), bf(B, N, 2 * DI), "k_idx"),        # d_idx differs
    (bf(B, N, HKV, DI), bf(B + 1, N, DI), "k_idx"),        # batch differs
    (bf(B, N, DI), bf(B, N, DI), "q_idx"),                 # q_idx not 4-D
])
def test_index_topk_shape_mismatch(q_idx, k_idx, name):
    with pytest.raises(ValueError, match=name):
        bnd.index_topk(q_idx, k_idx, topk=K)


@pytest.mark.parametrize("over,name", [
    (dict(k=bf(B, N // 2, HKV, D)), "k"),
    (dict(v=bf(B, N, HKV, 2 * D)), "v"),
    (dict(v=bf(B, N, HKV + 1, D)), "v"),
    (dict(block_idx=torch.zeros((B, N, HKV + 1, K), dtype=torch.int32)), "block_idx"),
    (dict(block_idx=torch.zeros((B, N - 128, HKV, K), dtype=torch.int32)), "block_idx"),
    (dict(block_idx=torch.zeros((B, N, HKV * K), dtype=torch.int32)), "block_idx"),
])
def test_sparse_fwd_shape_mismatch(over, name):
    with pytest.raises(ValueError, match=name):
        bnd.sparse_fwd(**fwd_args(**over))


@pytest.mark.parametrize("over,name", [
    (dict(k=bf(B, N, HKV, 2 * D)), "k"),
    (dict(v=bf(B, N + 128, HKV, D)), "v"),
    (dict(o=bf(B, N, HQ // 2, D)), "o"),
    (dict(dO=bf(B, N, HQ, D // 2)), "dO"),
    (dict(lse=torch.zeros((B, N, HQ + 1))), "lse"),
    (dict(lse=torch.zeros((B, N))), "lse"),
    (dict(block_idx=torch.zeros((B + 1, N, HKV, K), dtype=torch.int32)), "block_idx"),
    (dict(q_idx=bf(B, N, HKV + 1, DI)), "q_idx"),
    (dict(k_idx=bf(B, N, 2 * DI)), "k_idx"),
    (dict(k_idx=bf(B, 2 * N, DI)), "k_idx"),
])
def test_sparse_bwd_shape_mismatch(over, name):
    with pytest.raises(ValueError, match=name):
        bnd.sparse_bwd(**bwd_args(**over))


def test_tensors_on_different_devices_rejected():
    meta_k = torch.empty((B, N, HKV, D), dtype=torch.bfloat16, device="meta")
    with pytest.raises(ValueError, match="is on meta"):
        bnd.sparse_fwd(**fwd_args(k=meta_k))
