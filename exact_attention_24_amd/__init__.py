"""Exact attention for AMD Instinct MI355X (gfx950).

The computation runs in hand-written HIP kernels behind the C ABI of
``include/fa.h`` (``libfa.so``, built in-tree by ``build.py``); this package is
the thin Python binding over it.  Importing the package does not load the
library; the first call does, and raises if it is not built.
"""

from .binding import (  # noqa: F401
    FA_BF16, FA_F32, FA_FP8_E4M3, FaError, fa_bwd, fa_bwd_noalloc, fa_bwd_workspace_bytes, fa_check_bwd,
    fa_check_fwd, fa_check_kvcache, fa_check_merge, fa_check_varlen_bwd, fa_check_varlen_fwd, fa_fwd,
    fa_fwd_kvcache, fa_kvcache_workspace_bytes, fa_merge, fa_varlen_bwd, fa_varlen_bwd_workspace_bytes,
    fa_varlen_fwd, lib,
)

__all__ = ["fa_fwd", "fa_varlen_fwd", "fa_bwd", "fa_bwd_noalloc", "fa_varlen_bwd", "fa_bwd_workspace_bytes",
           "fa_varlen_bwd_workspace_bytes", "fa_check_fwd", "fa_check_varlen_fwd", "fa_check_bwd",
           "fa_check_varlen_bwd", "fa_merge", "fa_check_merge", "fa_fwd_kvcache", "fa_kvcache_workspace_bytes",
           "fa_check_kvcache", "lib", "FaError"]
