"""Thin ctypes binding of libmsa (include/msa.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libmsa.so.  PyTorch supplies device memory (outputs and the
workspace are allocated here with torch.empty) and the current stream.  If
the library is missing or a call fails, an exception is raised; there is no
fallback path.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("LIBMSA_PATH", os.path.join(_HERE, "libmsa.so"))

MSA_OK = 0
MSA_ERR_INVALID_ARG = -1
MSA_ERR_UNSUPPORTED = -2
MSA_ERR_WORKSPACE = -3
MSA_ERR_HIP = -4
MSA_F32 = 0
MSA_BF16 = 1
MSA_FP8_E4M3 = 2   # index inputs of msa_index_topk only

EXPORTED = (
    "msa_index_topk_workspace", "msa_index_topk",
    "msa_sparse_fwd_workspace", "msa_sparse_fwd", "msa_sparse_fwd_noalloc",
    "msa_sparse_bwd_workspace", "msa_sparse_bwd",
    "msa_status_string", "msa_last_error", "msa_version",
    "msa_profile_enable", "msa_profile_collect",
)


class MsaDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "N", "H_q", "H_kv", "d", "d_idx", "block_size", "topk", "causal", "dtype")] + \
               [("scale", ctypes.c_float), ("scale_idx", ctypes.c_float)]


class MsaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where} failed with status {status}: {detail}")
        self.status = status


_lib = None


def load_library(path: str | None = None):
    """Load libmsa.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libmsa.so not found at {p}: build it first (__graft_entry__.build())")
    lib = ctypes.CDLL(p)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    dims_p = ctypes.POINTER(MsaDims)
    lib.msa_index_topk_workspace.argtypes = [dims_p]
    lib.msa_index_topk_workspace.restype = sz
    lib.msa_index_topk.argtypes = [dims_p, vp, vp, vp, vp, vp, sz, vp]
    lib.msa_index_topk.restype = i32
    lib.msa_sparse_fwd_workspace.argtypes = [dims_p]
    lib.msa_sparse_fwd_workspace.restype = sz
    lib.msa_sparse_fwd.argtypes = [dims_p, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.msa_sparse_fwd.restype = i32
    lib.msa_sparse_fwd_noalloc.argtypes = [dims_p, vp, vp, vp, vp, vp, vp, vp]
    lib.msa_sparse_fwd_noalloc.restype = i32
    lib.msa_sparse_bwd_workspace.argtypes = [dims_p]
    lib.msa_sparse_bwd_workspace.restype = sz
    lib.msa_sparse_bwd.argtypes = [dims_p, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float,
                                   vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.msa_sparse_bwd.restype = i32
    lib.msa_status_string.argtypes = [i32]
    lib.msa_status_string.restype = ctypes.c_char_p
    lib.msa_last_error.argtypes = []
    lib.msa_last_error.restype = ctypes.c_char_p
    lib.msa_version.argtypes = []
    lib.msa_version.restype = i32
    lib.msa_profile_enable.argtypes = [i32]
    lib.msa_profile_enable.restype = i32
    lib.msa_profile_collect.argtypes = [i32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(i32),
                                        ctypes.POINTER(ctypes.c_double)]
    lib.msa_profile_collect.restype = i32
    if path is None:
        _lib = lib
    return lib


def make_dims(B, N, H_q, H_kv, d, d_idx, block_size=128, topk=16, causal=True, dtype=MSA_BF16,
              scale=0.0, scale_idx=0.0) -> MsaDims:
    return MsaDims(B, N, H_q, H_kv, d, d_idx, block_size, topk, int(bool(causal)), dtype,
                   float(scale or 0.0), float(scale_idx or 0.0))


def _check(lib, status, where):
    if status != MSA_OK:
        raise MsaError(status, where, lib.msa_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MSA_BF16
    if t.dtype == torch.float32:
        return MSA_F32
    if t.dtype == torch.float8_e4m3fn:
        return MSA_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _shapes(spec, **tensors):
    """Check every tensor against its expected shape before anything reaches
    the library: the kernels index each buffer with sizes taken from the
    others, so a mismatch would read or write past an allocation.

    spec: {name: tuple of dimension names or ints}; the first tensor to name
    a dimension fixes its size.  All tensors must also share one device."""
    sizes = {}
    device = None
    for name, want in spec.items():
        t = tensors[name]
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dim() != len(want):
            raise ValueError(f"{name} must have {len(want)} dimensions {tuple(want)}, got shape {tuple(t.shape)}")
        for axis, (dim, n) in enumerate(zip(want, t.shape)):
            if isinstance(dim, int):
                ok = n == dim
                expect = dim
            else:
                expect = sizes.setdefault(dim, n)
                ok = n == expect
            if not ok:
                raise ValueError(f"{name} has shape {tuple(t.shape)}: axis {axis} ({dim}) must be {expect}")
        if device is None:
            device = t.device
        elif t.device != device:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {device}")
    return sizes


def _workspace(nbytes: int, device):
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def index_topk(q_idx: torch.Tensor, k_idx: torch.Tensor, topk: int = 16, block_size: int = 128,
               causal: bool = True, return_pooled: bool = False):
    """block_idx [B,N,H_kv,topk] int32 (and pooled [B,N,H_kv,N/block_size] fp32).
    q_idx, k_idx: bf16, fp32, or float8_e4m3fn (d_idx = 64) for the FP8 indexer."""
    _shapes({"q_idx": ("B", "N", "H_kv", "d_idx"), "k_idx": ("B", "N", "d_idx")}, q_idx=q_idx, k_idx=k_idx)
    _need(q_idx, "q_idx")
    _need(k_idx, "k_idx", q_idx.dtype)
    lib = load_library()
    B, N, H_kv, d_idx = q_idx.shape
    dims = make_dims(B, N, H_kv, H_kv, 64, d_idx, block_size, topk, causal, _dtype_code(q_idx))
    out = torch.empty((B, N, H_kv, topk), dtype=torch.int32, device=q_idx.device)
    pooled = None
    if return_pooled:
        pooled = torch.empty((B, N, H_kv, N // block_size), dtype=torch.float32, device=q_idx.device)
    ws_n = lib.msa_index_topk_workspace(ctypes.byref(dims))
    ws = _workspace(ws_n, q_idx.device)
    st = lib.msa_index_topk(ctypes.byref(dims), _ptr(q_idx), _ptr(k_idx), _ptr(out), _ptr(pooled),
                            _ptr(ws), ws_n, _stream(q_idx.device))
    _check(lib, st, "msa_index_topk")
    return (out, pooled) if return_pooled else out


def sparse_fwd(q, k, v, block_idx, d_idx: int = 64, block_size: int = 128, causal: bool = True,
               scale: float | None = None):
    """o [B,N,H_q,d] (dtype of q) and lse [B,N,H_q] fp32."""
    _shapes({"q": ("B", "N", "H_q", "d"), "k": ("B", "N", "H_kv", "d"), "v": ("B", "N", "H_kv", "d"),
             "block_idx": ("B", "N", "H_kv", "topk")}, q=q, k=k, v=v, block_idx=block_idx)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    _need(block_idx, "block_idx", torch.int32)
    lib = load_library()
    B, N, H_q, d = q.shape
    H_kv = k.shape[2]
    topk = block_idx.shape[3]
    dims = make_dims(B, N, H_q, H_kv, d, d_idx, block_size, topk, causal, _dtype_code(q), scale or 0.0)
    o = torch.empty_like(q)
    lse = torch.empty((B, N, H_q), dtype=torch.float32, device=q.device)
    ws_n = lib.msa_sparse_fwd_workspace(ctypes.byref(dims))
    ws = _workspace(ws_n, q.device)
    st = lib.msa_sparse_fwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(block_idx), _ptr(o),
                            _ptr(lse), _ptr(ws), ws_n, _stream(q.device))
    _check(lib, st, "msa_sparse_fwd")
    return o, lse


def sparse_fwd_noalloc(q, k, v, block_idx, o, lse, d_idx: int = 64, block_size: int = 128,
                       causal: bool = True, scale: float | None = None):
    """msa_sparse_fwd_noalloc: the forward into caller-given o [B,N,H_q,d]
    (dtype of q) and lse [B,N,H_q] fp32, with the library's fixed device
    scratch instead of a workspace.  Nothing is allocated here."""
    _shapes({"q": ("B", "N", "H_q", "d"), "k": ("B", "N", "H_kv", "d"), "v": ("B", "N", "H_kv", "d"),
             "block_idx": ("B", "N", "H_kv", "topk"), "o": ("B", "N", "H_q", "d"), "lse": ("B", "N", "H_q")},
            q=q, k=k, v=v, block_idx=block_idx, o=o, lse=lse)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _need(t, n, q.dtype)
    _need(block_idx, "block_idx", torch.int32)
    _need(lse, "lse", torch.float32)
    lib = load_library()
    B, N, H_q, d = q.shape
    H_kv = k.shape[2]
    topk = block_idx.shape[3]
    dims = make_dims(B, N, H_q, H_kv, d, d_idx, block_size, topk, causal, _dtype_code(q), scale or 0.0)
    with torch.cuda.device(q.device):
        st = lib.msa_sparse_fwd_noalloc(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(block_idx),
                                        _ptr(o), _ptr(lse), _stream(q.device))
    _check(lib, st, "msa_sparse_fwd_noalloc")
    return o, lse


def sparse_bwd(q, k, v, o, dO, lse, block_idx, q_idx, k_idx, kl_weight: float = 1.0,
               block_size: int = 128, causal: bool = True, scale: float | None = None,
               scale_idx: float | None = None, want_dscore: bool = False, want_kl: bool = False):
    """dict with dq, dk, dv (dtype of q), dq_idx, dk_idx (fp32) and optionally
    dscore [B,N,H_kv,topk,block_size] and kl [B,N,H_kv] (fp32)."""
    _shapes({"q": ("B", "N", "H_q", "d"), "k": ("B", "N", "H_kv", "d"), "v": ("B", "N", "H_kv", "d"),
             "o": ("B", "N", "H_q", "d"), "dO": ("B", "N", "H_q", "d"), "lse": ("B", "N", "H_q"),
             "block_idx": ("B", "N", "H_kv", "topk"), "q_idx": ("B", "N", "H_kv", "d_idx"),
             "k_idx": ("B", "N", "d_idx")},
            q=q, k=k, v=v, o=o, dO=dO, lse=lse, block_idx=block_idx, q_idx=q_idx, k_idx=k_idx)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dO, "dO"), (q_idx, "q_idx"), (k_idx, "k_idx")):
        _need(t, n, q.dtype)
    _need(lse, "lse", torch.float32)
    _need(block_idx, "block_idx", torch.int32)
    lib = load_library()
    B, N, H_q, d = q.shape
    H_kv = k.shape[2]
    d_idx = q_idx.shape[3]
    topk = block_idx.shape[3]
    dims = make_dims(B, N, H_q, H_kv, d, d_idx, block_size, topk, causal, _dtype_code(q),
                     scale or 0.0, scale_idx or 0.0)
    dev = q.device
    out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
               dq_idx=torch.empty((B, N, H_kv, d_idx), dtype=torch.float32, device=dev),
               dk_idx=torch.empty((B, N, d_idx), dtype=torch.float32, device=dev))
    out["dscore"] = (torch.empty((B, N, H_kv, topk, block_size), dtype=torch.float32, device=dev)
                     if want_dscore else None)
    out["kl"] = torch.empty((B, N, H_kv), dtype=torch.float32, device=dev) if want_kl else None
    ws_n = lib.msa_sparse_bwd_workspace(ctypes.byref(dims))
    ws = _workspace(ws_n, dev)
    st = lib.msa_sparse_bwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse),
                            _ptr(block_idx), _ptr(q_idx), _ptr(k_idx), float(kl_weight),
                            _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dq_idx"]),
                            _ptr(out["dk_idx"]), _ptr(out["dscore"]), _ptr(out["kl"]), _ptr(ws), ws_n,
                            _stream(dev))
    _check(lib, st, "msa_sparse_bwd")
    return out


def profile_enable(on: bool = True) -> None:
    """Bracket every internal kernel launch with hipEvents (measurement only)."""
    load_library().msa_profile_enable(int(bool(on)))


def profile_collect(max_kernels: int = 64) -> dict:
    """{kernel name: (launches, total ms)} since the previous collect."""
    lib = load_library()
    names = (ctypes.c_char_p * max_kernels)()
    launches = (ctypes.c_int * max_kernels)()
    total = (ctypes.c_double * max_kernels)()
    n = lib.msa_profile_collect(max_kernels, names, launches, total)
    if n < 0:
        raise MsaError(n, "msa_profile_collect", lib.msa_last_error().decode())
    return {names[i].decode(): (launches[i], total[i]) for i in range(n)}
