"""Hybrid compressed attention (CSA / HCA) for one layer on MI355X (gfx950).

The work runs in libcsa.so (hand-written HIP kernels behind the C ABI of
include/csa.h); this package holds the in-tree build step and the ctypes
binding with the same entry-point names.
"""
from ._lib import (  # noqa: F401
    ATTEND_NORM_Q, ATTEND_NO_INV_ROPE, FMT_F32, FMT_FP8_BF16, FMT_MXFP4, CsaError,
    attend, compress, hca_attend, index_topk, load, split_main, workspace_bytes,
)
