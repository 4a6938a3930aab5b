"""Exact Euclidean distance transform on AMD Instinct MI355X (gfx950).

The computation lives in ``libedt_mi355x.so`` (hand-written HIP kernels behind
the C ABI of ``include/edt.h``); this package only marshals arguments.

    from exact_euclidean_distance_amd import edt2d, edt3d
    r = edt2d(mask_u8_cuda, return_sqdist=True, return_indices=True)   # (H, W) or (B, H, W)
"""

from ._lib import EDTError, LIB_PATH  # noqa: F401
from .api import (  # noqa: F401
    EDTResult,
    alloc_workspace,
    edt1d,
    edt2d,
    edt,
    edt3d,
    edt_brute,
    chessboard,
    taxicab,
    unravel_indices,
    workspace_size_2d,
    workspace_size_2d_batched,
    workspace_size_3d,
)

__all__ = ["chessboard", "edt", "edt1d", "edt2d", "edt3d", "edt_brute", "taxicab", "unravel_indices", "EDTResult", "EDTError",
           "workspace_size_2d", "workspace_size_2d_batched", "workspace_size_3d",
           "alloc_workspace"]
