"""MiniMax Sparse Attention (MSA) over GQA for AMD MI355X (gfx950).

The computation lives in libmsa.so (hand-written HIP kernels behind the C ABI
of include/msa.h); this package only marshals PyTorch tensors into it.
"""

from .binding import (MsaDims, MsaError, index_topk, load_library, make_dims, profile_collect,
                      profile_enable, sparse_bwd, sparse_fwd, sparse_fwd_noalloc, LIB_PATH)

__all__ = ["MsaDims", "MsaError", "index_topk", "load_library", "make_dims", "profile_collect",
           "profile_enable", "sparse_bwd", "sparse_fwd", "sparse_fwd_noalloc", "LIB_PATH"]
