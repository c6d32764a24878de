"""C-ABI tests that need no GPU: the library loads, exports every symbol the
header declares, sizes workspaces, and rejects invalid or unsupported
problems before launching anything (every call here fails validation, so no
kernel is ever enqueued)."""

import ctypes
import os
import re

import pytest

from block_sparse_attention_branch_amd import binding as bnd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")

FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
NULL = ctypes.c_void_p(0)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bnd.LIB_PATH):
        pytest.skip("libmsa.so not built")
    return bnd.load_library()


def _declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"MSA_API\s+[\w\s\*]+?\b(msa_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    syms = _declared_symbols()
    for name in ("msa_index_topk", "msa_sparse_fwd", "msa_sparse_bwd", "msa_index_topk_workspace",
                 "msa_sparse_fwd_workspace", "msa_sparse_bwd_workspace", "msa_status_string",
                 "msa_last_error", "msa_version"):
        assert name in syms
    assert set(syms) == set(bnd.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_symbols():
        assert hasattr(lib, name), name
    assert lib.msa_version() >= 1


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4):
        assert lib.msa_status_string(code).decode() not in ("", "unknown status")
    assert lib.msa_status_string(12345).decode() == "unknown status"


def good_dims(**kw):
    base = dict(B=1, N=1024, H_q=8, H_kv=2, d=128, d_idx=64, block_size=128, topk=4, causal=True,
                dtype=bnd.MSA_BF16)
    base.update(kw)
    return bnd.make_dims(**base)


@pytest.mark.parametrize("kw,expect", [
    (dict(B=0), bnd.MSA_ERR_INVALID_ARG),
    (dict(N=-128), bnd.MSA_ERR_INVALID_ARG),
    (dict(topk=0), bnd.MSA_ERR_INVALID_ARG),
    (dict(H_q=6, H_kv=4), bnd.MSA_ERR_INVALID_ARG),
    (dict(dtype=7), bnd.MSA_ERR_INVALID_ARG),
    (dict(block_size=64), bnd.MSA_ERR_UNSUPPORTED),
    (dict(N=1000), bnd.MSA_ERR_UNSUPPORTED),
    (dict(d=96), bnd.MSA_ERR_UNSUPPORTED),
    (dict(d_idx=48), bnd.MSA_ERR_UNSUPPORTED),
    (dict(topk=65), bnd.MSA_ERR_UNSUPPORTED),
    (dict(H_q=6, H_kv=2), bnd.MSA_ERR_UNSUPPORTED),
    (dict(N=128 * (1 << 16)), bnd.MSA_ERR_UNSUPPORTED),
    (dict(B=128, N=1 << 20, H_q=16, H_kv=2), bnd.MSA_ERR_UNSUPPORTED),   # B*N*H_q = 2^31
])
def test_invalid_dims_rejected_by_every_entry_point(lib, kw, expect):
    dims = good_dims(**kw)
    d = ctypes.byref(dims)
    assert lib.msa_index_topk(d, FAKE, FAKE, FAKE, NULL, NULL, 0, NULL) == expect
    assert lib.msa_last_error().decode() != ""
    assert lib.msa_sparse_fwd(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, NULL) == expect
    assert lib.msa_sparse_fwd_noalloc(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL) == expect
    assert lib.msa_sparse_bwd(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1.0, FAKE, FAKE,
                              FAKE, FAKE, FAKE, NULL, NULL, FAKE, 1 << 40, NULL) == expect
    assert lib.msa_index_topk_workspace(d) == 0
    assert lib.msa_sparse_fwd_workspace(d) == 0
    assert lib.msa_sparse_bwd_workspace(d) == 0


def test_null_dims(lib):
    assert lib.msa_index_topk(None, FAKE, FAKE, FAKE, NULL, NULL, 0, NULL) == bnd.MSA_ERR_INVALID_ARG
    assert "dims" in lib.msa_last_error().decode()


def test_required_pointers(lib):
    d = ctypes.byref(good_dims())
    assert lib.msa_index_topk(d, NULL, FAKE, FAKE, NULL, NULL, 0, NULL) == bnd.MSA_ERR_INVALID_ARG
    assert "q_idx" in lib.msa_last_error().decode()
    assert lib.msa_index_topk(d, FAKE, FAKE, NULL, NULL, NULL, 0, NULL) == bnd.MSA_ERR_INVALID_ARG
    assert lib.msa_sparse_fwd(d, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, 1 << 40, NULL) == \
        bnd.MSA_ERR_INVALID_ARG
    assert "lse" in lib.msa_last_error().decode()
    args = [FAKE] * 9
    for missing in range(9):
        a = list(args)
        a[missing] = NULL
        st = lib.msa_sparse_bwd(d, *a, 1.0, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE, 1 << 40, NULL)
        assert st == bnd.MSA_ERR_INVALID_ARG, missing
    st = lib.msa_sparse_bwd(d, *args, float("nan"), FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE,
                            1 << 40, NULL)
    assert st == bnd.MSA_ERR_INVALID_ARG


def test_workspace_too_small(lib):
    dims = good_dims()
    d = ctypes.byref(dims)
    need = lib.msa_sparse_fwd_workspace(d)
    assert need > 0
    st = lib.msa_sparse_fwd(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, NULL)
    assert st == bnd.MSA_ERR_WORKSPACE
    assert str(need) in lib.msa_last_error().decode()
    st = lib.msa_sparse_fwd(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, need, NULL)
    assert st == bnd.MSA_ERR_INVALID_ARG
    bneed = lib.msa_sparse_bwd_workspace(d)
    if bneed > 0:
        st = lib.msa_sparse_bwd(d, *([FAKE] * 9), 1.0, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE,
                                bneed - 1, NULL)
        assert st == bnd.MSA_ERR_WORKSPACE


def test_workspace_sizes_grow_with_problem(lib):
    small = lib.msa_sparse_fwd_workspace(ctypes.byref(good_dims(N=1024)))
    big = lib.msa_sparse_fwd_workspace(ctypes.byref(good_dims(N=8192)))
    assert 0 < small < big
    assert lib.msa_index_topk_workspace(ctypes.byref(good_dims())) == 0


def test_fp32_backward_unsupported(lib):
    d = ctypes.byref(good_dims(dtype=bnd.MSA_F32))
    st = lib.msa_sparse_bwd(d, *([FAKE] * 9), 1.0, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE,
                            1 << 40, NULL)
    assert st == bnd.MSA_ERR_UNSUPPORTED


def test_fp8_only_for_the_index_branch(lib):
    d8 = good_dims(dtype=bnd.MSA_FP8_E4M3)
    st = lib.msa_sparse_fwd(ctypes.byref(d8), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, NULL)
    assert st == bnd.MSA_ERR_UNSUPPORTED
    st = lib.msa_sparse_bwd(ctypes.byref(d8), *([FAKE] * 9), 1.0, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE,
                            1 << 40, NULL)
    assert st == bnd.MSA_ERR_UNSUPPORTED
    assert lib.msa_sparse_fwd_workspace(ctypes.byref(d8)) == 0
    assert lib.msa_sparse_bwd_workspace(ctypes.byref(d8)) == 0
    # The FP8 indexer is built for d_idx = 64; other index dims are refused.
    d32 = good_dims(dtype=bnd.MSA_FP8_E4M3, d_idx=32)
    assert lib.msa_index_topk(ctypes.byref(d32), FAKE, FAKE, FAKE, NULL, NULL, 0, NULL) == bnd.MSA_ERR_UNSUPPORTED
    assert lib.msa_index_topk(ctypes.byref(d8), NULL, FAKE, FAKE, NULL, NULL, 0, NULL) == bnd.MSA_ERR_INVALID_ARG
    bad = good_dims(dtype=7)
    assert lib.msa_index_topk(ctypes.byref(bad), FAKE, FAKE, FAKE, NULL, NULL, 0, NULL) == bnd.MSA_ERR_INVALID_ARG


def test_noalloc_forward_validates_like_the_forward(lib):
    d = ctypes.byref(good_dims())
    for missing in range(6):
        a = [FAKE] * 6
        a[missing] = NULL
        assert lib.msa_sparse_fwd_noalloc(d, *a, NULL) == bnd.MSA_ERR_INVALID_ARG, missing
    d8 = good_dims(dtype=bnd.MSA_FP8_E4M3)
    assert lib.msa_sparse_fwd_noalloc(ctypes.byref(d8), *([FAKE] * 6), NULL) == bnd.MSA_ERR_UNSUPPORTED


def test_noalloc_forward_rejects_problems_beyond_its_scratch(lib):
    # N = 128K with 64/8 heads and topk 16: the block map alone is about
    # 98 MiB and one super-block of partials 34 MiB more, past the 128 MiB
    # the library holds; refused before any HIP call.
    dims = good_dims(N=1 << 17, H_q=64, H_kv=8, topk=16)
    st = lib.msa_sparse_fwd_noalloc(ctypes.byref(dims), *([FAKE] * 6), NULL)
    assert st == bnd.MSA_ERR_UNSUPPORTED
    msg = lib.msa_last_error().decode()
    assert "scratch" in msg and str(128 << 20) in msg
