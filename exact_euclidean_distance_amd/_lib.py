"""ctypes loader for libedt_mi355x.so (the C ABI declared in include/edt.h).

There is no fallback: if the library is missing the import of a compute entry
point raises, so nothing silently runs anywhere but the HIP kernels.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libedt_mi355x.so")

STATUS = {
    0: "EDT_OK",
    1: "EDT_ERR_INVALID_ARGUMENT",
    2: "EDT_ERR_UNSUPPORTED_SHAPE",
    3: "EDT_ERR_WORKSPACE_TOO_SMALL",
    4: "EDT_ERR_HIP",
}

EXPORTS = (
    "edt2d_workspace_size", "edt2d_u8", "edt3d_workspace_size", "edt3d_u8_batched",
    "edt2d_u8_timed", "edt3d_u8_batched_timed", "edt_status_string", "edt_version",
    "edt2d_batched_workspace_size", "edt2d_u8_batched", "edt2d_u8_batched_timed",
    "edt1d_workspace_size", "edt1d_u8_batched", "edt_unravel_indices",
    "edt_brute_workspace_size", "edt_brute_u8", "edt_brute_metric_u8", "edt3d_u8_batched_idx64",
    "edt2d_taxicab_u8_batched", "edt3d_taxicab_u8_batched",
    "edt2d_chessboard_u8_batched", "edt3d_chessboard_u8_batched",
    "edt2d_u8_batched_noalloc", "edt2d_noalloc_max_workspace",
    "edt_nd_workspace_size", "edt_nd_u8", "edt_unravel_indices_nd",
    "edt2d_proximate_workspace_size", "edt2d_proximate_u8_batched",
    "edt2d_proximate_u8_batched_timed",
)

_lib = None


class EDTError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library (once) and declare the signatures."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m exact_euclidean_distance_amd.build` "
            "(hipcc, gfx950); there is no CPU fallback")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    fp = ctypes.POINTER(ctypes.c_float)
    lib.edt2d_workspace_size.restype = sz
    lib.edt2d_workspace_size.argtypes = [i32, i32]
    lib.edt3d_workspace_size.restype = sz
    lib.edt3d_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.edt2d_u8.restype = ctypes.c_int
    lib.edt2d_u8.argtypes = [vp, i32, i32, fp, vp, vp, vp, vp, sz, vp]
    lib.edt3d_u8_batched.restype = ctypes.c_int
    lib.edt3d_u8_batched.argtypes = [vp, i32, i32, i32, i32, fp, vp, vp, vp, vp, sz, vp]
    lib.edt2d_u8_timed.restype = ctypes.c_int
    lib.edt2d_u8_timed.argtypes = [vp, i32, i32, fp, vp, vp, vp, vp, sz, vp,
                                   fp, ctypes.POINTER(ctypes.c_char_p), i32,
                                   ctypes.POINTER(i32)]
    lib.edt3d_u8_batched_timed.restype = ctypes.c_int
    lib.edt3d_u8_batched_timed.argtypes = [vp, i32, i32, i32, i32, fp, vp, vp, vp, vp, sz, vp,
                                           fp, ctypes.POINTER(ctypes.c_char_p), i32,
                                           ctypes.POINTER(i32)]
    ip = ctypes.POINTER(i32)
    lib.edt2d_batched_workspace_size.restype = sz
    lib.edt2d_batched_workspace_size.argtypes = [i32, i32, i32]
    lib.edt2d_u8_batched.restype = ctypes.c_int
    lib.edt2d_u8_batched.argtypes = [vp, i32, i32, i32, fp, vp, vp, vp, vp, sz, vp]
    lib.edt2d_u8_batched_timed.restype = ctypes.c_int
    lib.edt2d_u8_batched_timed.argtypes = [vp, i32, i32, i32, fp, vp, vp, vp, vp, sz, vp,
                                           fp, ctypes.POINTER(ctypes.c_char_p), i32, ip]
    lib.edt1d_workspace_size.restype = sz
    lib.edt1d_workspace_size.argtypes = [i32, i32]
    lib.edt1d_u8_batched.restype = ctypes.c_int
    lib.edt1d_u8_batched.argtypes = [vp, i32, i32, fp, vp, vp, vp, vp, sz, vp]
    lib.edt_unravel_indices.restype = ctypes.c_int
    lib.edt_unravel_indices.argtypes = [vp, i32, i32, ip, vp, vp]
    lib.edt_brute_workspace_size.restype = sz
    lib.edt_brute_workspace_size.argtypes = [i32, i32, ip]
    lib.edt_brute_u8.restype = ctypes.c_int
    lib.edt_brute_u8.argtypes = [vp, i32, i32, ip, fp, vp, vp, vp, vp, sz, vp]
    lib.edt_brute_metric_u8.restype = ctypes.c_int
    lib.edt_brute_metric_u8.argtypes = [vp, i32, i32, ip, i32, vp, vp, vp, sz, vp]
    lib.edt3d_u8_batched_idx64.restype = ctypes.c_int
    lib.edt3d_u8_batched_idx64.argtypes = [vp, i32, i32, i32, i32, fp, vp, vp, vp, vp, sz, vp]
    lib.edt2d_taxicab_u8_batched.restype = ctypes.c_int
    lib.edt2d_taxicab_u8_batched.argtypes = [vp, i32, i32, i32, vp, vp, vp, sz, vp]
    lib.edt3d_taxicab_u8_batched.restype = ctypes.c_int
    lib.edt3d_taxicab_u8_batched.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, sz, vp]
    lib.edt2d_chessboard_u8_batched.restype = ctypes.c_int
    lib.edt2d_chessboard_u8_batched.argtypes = [vp, i32, i32, i32, vp, vp, vp, sz, vp]
    lib.edt3d_chessboard_u8_batched.restype = ctypes.c_int
    lib.edt3d_chessboard_u8_batched.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, sz, vp]
    lib.edt2d_u8_batched_noalloc.restype = ctypes.c_int
    lib.edt2d_u8_batched_noalloc.argtypes = [vp, i32, i32, i32, fp, vp, vp, vp, vp]
    lib.edt2d_noalloc_max_workspace.restype = sz
    lib.edt2d_noalloc_max_workspace.argtypes = []
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.edt_nd_workspace_size.restype = sz
    lib.edt_nd_workspace_size.argtypes = [i32, i32, i64p, i64p, i32]
    lib.edt_nd_u8.restype = ctypes.c_int
    lib.edt_nd_u8.argtypes = [vp, i32, i32, i64p, i64p, fp, vp, vp, vp, i32, vp, sz, vp]
    lib.edt_unravel_indices_nd.restype = ctypes.c_int
    lib.edt_unravel_indices_nd.argtypes = [vp, i32, ctypes.c_int64, i32, i64p, vp, vp]
    lib.edt2d_proximate_workspace_size.restype = sz
    lib.edt2d_proximate_workspace_size.argtypes = [i32, i32, i32]
    lib.edt2d_proximate_u8_batched.restype = ctypes.c_int
    lib.edt2d_proximate_u8_batched.argtypes = [vp, i32, i32, i32, fp, vp, vp, vp, vp, sz, vp]
    lib.edt2d_proximate_u8_batched_timed.restype = ctypes.c_int
    lib.edt2d_proximate_u8_batched_timed.argtypes = [vp, i32, i32, i32, fp, vp, vp, vp, vp, sz, vp,
                                                     fp, ctypes.POINTER(ctypes.c_char_p), i32, ip]
    lib.edt_status_string.restype = ctypes.c_char_p
    lib.edt_status_string.argtypes = [ctypes.c_int]
    lib.edt_version.restype = ctypes.c_char_p
    lib.edt_version.argtypes = []
    if path == LIB_PATH:
        _lib = lib
    return lib
