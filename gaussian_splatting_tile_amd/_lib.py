"""ctypes declarations for libgs.so (include/gs.h). Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# GS_LIB_PATH names another build of the same sources (the host-sanitized
# one of the CPU tests); the default is the in-tree library.
LIB_PATH = os.environ.get("GS_LIB_PATH") or os.path.join(_HERE, "libgs.so")

GS_OK, GS_ERR_INVALID, GS_ERR_CAPACITY, GS_ERR_OVERFLOW, GS_ERR_HIP = range(5)
GS_TILES_SQUARE, GS_TILES_ELLIPSE = 0, 1
STATUS_NAMES = {0: "GS_OK", 1: "GS_ERR_INVALID", 2: "GS_ERR_CAPACITY", 3: "GS_ERR_OVERFLOW",
                4: "GS_ERR_HIP"}

# Every symbol include/gs.h declares.
EXPORTS = ("gs_constants", "gs_last_error", "gs_version", "gs_preprocess", "gs_preprocess_ex",
           "gs_preprocess_bwd", "gs_bin_and_sort", "gs_bin_and_sort_ex", "gs_bin_and_sort_async_ex",
           "gs_bin_and_sort_async", "gs_tile_ranges", "gs_tile_ranges_async", "gs_composite_fwd",
           "gs_composite_bwd", "gs_composite_fwd_ex", "gs_composite_part_bytes", "gs_composite_bwd_ex", "gs_tile_ranges_ex",
           "gs_preprocess_views", "gs_bin_and_sort_views_async", "gs_appearance_fwd",
           "gs_appearance_bwd", "gs_bin_and_sort_async_noalloc")


class GsCamera(ctypes.Structure):
    _fields_ = [("R", ctypes.c_float * 9), ("t", ctypes.c_float * 3),
                ("campos", ctypes.c_float * 3), ("fx", ctypes.c_float), ("fy", ctypes.c_float),
                ("cx", ctypes.c_float), ("cy", ctypes.c_float), ("width", ctypes.c_int32),
                ("height", ctypes.c_int32)]


class GsError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libgs.so; fails loudly if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m gaussian_splatting_tile_amd.build` (or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I32, I64, U32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
    CAM = ctypes.POINTER(GsCamera)
    lib.gs_constants.restype = None
    lib.gs_constants.argtypes = [P]
    lib.gs_last_error.restype = ctypes.c_char_p
    lib.gs_last_error.argtypes = []
    lib.gs_version.restype = None
    lib.gs_version.argtypes = [P]
    lib.gs_preprocess.restype = ctypes.c_int
    lib.gs_preprocess.argtypes = [CAM, I32, P, P, P, P, P, I32, P, P, P, P, P, P]
    lib.gs_preprocess_ex.restype = ctypes.c_int
    lib.gs_preprocess_ex.argtypes = [CAM, I32, P, P, P, P, P, I32, P, P, P, P, P, U32, P]
    lib.gs_bin_and_sort_ex.restype = ctypes.c_int
    lib.gs_bin_and_sort_ex.argtypes = [CAM, I32, P, P, P, P, P, I64, P, ctypes.POINTER(ctypes.c_size_t),
                                       ctypes.POINTER(ctypes.c_int64), U32, P]
    lib.gs_bin_and_sort_async_ex.restype = ctypes.c_int
    lib.gs_bin_and_sort_async_ex.argtypes = [CAM, I32, P, P, P, P, P, I64, P, ctypes.POINTER(ctypes.c_size_t),
                                             P, U32, P]
    lib.gs_preprocess_bwd.restype = ctypes.c_int
    lib.gs_preprocess_bwd.argtypes = [CAM, I32, P, P, P, P, I32, P, P, P, P, P, P, P, P, P, P, P]
    lib.gs_bin_and_sort.restype = ctypes.c_int
    lib.gs_bin_and_sort.argtypes = [CAM, I32, P, P, P, P, I64, P, ctypes.POINTER(ctypes.c_size_t),
                                    ctypes.POINTER(ctypes.c_int64), P]
    lib.gs_bin_and_sort_async.restype = ctypes.c_int
    lib.gs_bin_and_sort_async.argtypes = [CAM, I32, P, P, P, P, I64, P, ctypes.POINTER(ctypes.c_size_t), P, P]
    lib.gs_tile_ranges.restype = ctypes.c_int
    lib.gs_tile_ranges.argtypes = [CAM, P, I64, P, P, P]
    lib.gs_tile_ranges_async.restype = ctypes.c_int
    lib.gs_tile_ranges_async.argtypes = [CAM, P, P, I64, P, P, P]
    lib.gs_composite_fwd.restype = ctypes.c_int
    lib.gs_composite_fwd.argtypes = [CAM, P, P, P, P, P, P, P, P, P, P, P, P]
    lib.gs_composite_bwd.restype = ctypes.c_int
    lib.gs_composite_bwd.argtypes = [CAM, I32, P, P, P, P, P, P, P, P, P, P, P, P, P, P]
    lib.gs_composite_fwd_ex.restype = ctypes.c_int
    lib.gs_composite_fwd_ex.argtypes = [CAM, I32, P, P, P, P, P, P, P, P, P, P, P, I64, P, P, P, P]
    lib.gs_composite_part_bytes.restype = ctypes.c_size_t
    lib.gs_composite_part_bytes.argtypes = [CAM, I32, I64]
    lib.gs_preprocess_views.restype = ctypes.c_int
    lib.gs_preprocess_views.argtypes = [P, I32, I32, P, P, P, P, P, I32, P, P, P, P, P, U32, P]
    lib.gs_bin_and_sort_async_noalloc.restype = ctypes.c_int
    lib.gs_bin_and_sort_async_noalloc.argtypes = [CAM, I32, P, P, P, P, P, I64, P, U32, P]
    lib.gs_bin_and_sort_views_async.restype = ctypes.c_int
    lib.gs_bin_and_sort_views_async.argtypes = [CAM, I32, I32, P, P, P, P, P, I64, P,
                                                ctypes.POINTER(ctypes.c_size_t), P, U32, P]
    lib.gs_composite_bwd_ex.restype = ctypes.c_int
    lib.gs_composite_bwd_ex.argtypes = [CAM, I32, I32, P, P, P, I64, P, P, P, P, P, P, P, P, P, P, P, P, P]
    lib.gs_tile_ranges_ex.restype = ctypes.c_int
    lib.gs_tile_ranges_ex.argtypes = [CAM, I32, P, I64, P, I64, P, P, P, P]
    lib.gs_appearance_fwd.restype = ctypes.c_int
    lib.gs_appearance_fwd.argtypes = [CAM, I32, P, P, I32, I32, P, P, P]
    lib.gs_appearance_bwd.restype = ctypes.c_int
    lib.gs_appearance_bwd.argtypes = [CAM, I32, P, P, I32, I32, P, P, P, P, P, ctypes.POINTER(ctypes.c_size_t), P]
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != GS_OK:
        msg = load().gs_last_error().decode(errors="replace")
        raise GsError(status, msg)
