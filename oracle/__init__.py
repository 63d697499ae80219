"""Plain CPU oracle for the tile-based Gaussian Splatting rasterizer.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers. The product path
never imports this package.

This module is numpy-level marshalling around ``liboracle.so``, which is
built from ``oracle.cpp`` by :func:`build` (g++, -O2, -ffp-contract=off).
Every arithmetic step lives in ``oracle.cpp``; see its header for the pages
each function follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
# GS_ORACLE_LIB names a prebuilt copy of oracle.cpp (the sanitized build of
# the CPU tests), used as it is; otherwise the in-tree liboracle.so is
# rebuilt whenever oracle.cpp is newer.
_LIB_OVERRIDE = os.environ.get("GS_ORACLE_LIB")
_LIB = _LIB_OVERRIDE or os.path.join(_HERE, "liboracle.so")

TILE = 16


def build(verbose: bool = False) -> str:
    """Compile liboracle.so with the host compiler. Returns its path."""
    cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-o", _LIB + ".tmp", _SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class Camera(ctypes.Structure):
    _fields_ = [("R", ctypes.c_float * 9), ("t", ctypes.c_float * 3),
                ("campos", ctypes.c_float * 3), ("fx", ctypes.c_float),
                ("fy", ctypes.c_float), ("cx", ctypes.c_float), ("cy", ctypes.c_float),
                ("width", ctypes.c_int32), ("height", ctypes.c_int32)]


def make_camera(cam: dict) -> Camera:
    c = Camera()
    c.R[:] = [float(x) for x in np.asarray(cam["R"], np.float32).reshape(9)]
    c.t[:] = [float(x) for x in np.asarray(cam["t"], np.float32).reshape(3)]
    c.campos[:] = [float(x) for x in np.asarray(cam["campos"], np.float32).reshape(3)]
    c.fx, c.fy = float(np.float32(cam["fx"])), float(np.float32(cam["fy"]))
    c.cx, c.cy = float(np.float32(cam["cx"])), float(np.float32(cam["cy"]))
    c.width, c.height = int(cam["width"]), int(cam["height"])
    return c


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not _LIB_OVERRIDE and (not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build()
        _lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        _lib.orc_preprocess.restype = ctypes.c_int
        _lib.orc_preprocess.argtypes = [ctypes.POINTER(Camera), ctypes.c_int32, P, P, P, P, P,
                                        ctypes.c_int32, P, P, P, P, P]
        _lib.orc_preprocess_ex.restype = ctypes.c_int
        _lib.orc_preprocess_ex.argtypes = [ctypes.POINTER(Camera), ctypes.c_int32, P, P, P, P, P,
                                           ctypes.c_int32, P, P, P, P, P, ctypes.c_int32]
        _lib.orc_bin_ex.restype = ctypes.c_int64
        _lib.orc_bin_ex.argtypes = [ctypes.POINTER(Camera), ctypes.c_int32, P, P, P, P, P, ctypes.c_int64,
                                    ctypes.c_int32]
        _lib.orc_ellipse_row_range.restype = None
        _lib.orc_ellipse_row_range.argtypes = [ctypes.c_float] * 6 + [ctypes.c_int32] * 3 + [P]
        _lib.orc_bin.restype = ctypes.c_int64
        _lib.orc_bin.argtypes = [ctypes.POINTER(Camera), ctypes.c_int32, P, P, P, P, ctypes.c_int64]
        _lib.orc_tile_ranges.restype = None
        _lib.orc_tile_ranges.argtypes = [ctypes.POINTER(Camera), P, ctypes.c_int64, P]
        for name in ("orc_composite_fwd_f32", "orc_composite_fwd_f64"):
            getattr(_lib, name).restype = None
            getattr(_lib, name).argtypes = [ctypes.POINTER(Camera)] + [P] * 10
        for name in ("orc_composite_bwd_f32", "orc_composite_bwd_f64"):
            getattr(_lib, name).restype = None
            getattr(_lib, name).argtypes = [ctypes.POINTER(Camera), ctypes.c_int32] + [P] * 12
        _lib.orc_composite_bwd_mass_f32.restype = None
        _lib.orc_composite_bwd_mass_f32.argtypes = [ctypes.POINTER(Camera), ctypes.c_int32] + [P] * 15
        _lib.orc_set_threads.restype = ctypes.c_int
        _lib.orc_set_threads.argtypes = [ctypes.c_int32]
        _lib.orc_constants.restype = None
        _lib.orc_constants.argtypes = [P]
        _lib.orc_sh_basis.restype = None
        _lib.orc_sh_basis.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.c_float, P]
        _lib.orc_tile_span.restype = None
        _lib.orc_tile_span.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                       ctypes.c_int32, ctypes.c_int32, P]
        _lib.orc_exclusive_scan.restype = ctypes.c_uint64
        _lib.orc_exclusive_scan.argtypes = [P, ctypes.c_int64, P]
        _lib.orc_duplicate.restype = ctypes.c_int
        _lib.orc_duplicate.argtypes = [ctypes.POINTER(Camera), ctypes.c_int32, P, P, P, P, P]
        _lib.orc_sort_pairs.restype = None
        _lib.orc_sort_pairs.argtypes = [P, P, ctypes.c_int64]
        _lib.orc_preprocess_bwd.restype = ctypes.c_int
        _lib.orc_preprocess_bwd.argtypes = [ctypes.POINTER(Camera), ctypes.c_int32, P, P, P, P, P,
                                            ctypes.c_int32, P, P, P, P, P, P, P, P, P, P]
        _lib.orc_project_f64.restype = ctypes.c_int
        _lib.orc_project_f64.argtypes = [ctypes.POINTER(Camera), P, P, P, P, ctypes.c_int32, P, P]
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def set_threads(threads: int) -> int:
    """Threads the preprocess and the compositing use (1, the default: the
    canonical single-threaded run). Returns the number set."""
    return int(lib().orc_set_threads(int(threads)))


def tiles_xy(cam: dict):
    return (int(cam["width"]) + TILE - 1) // TILE, (int(cam["height"]) + TILE - 1) // TILE


def constants() -> np.ndarray:
    out = np.zeros(9, np.float32)
    lib().orc_constants(_p(out))
    return out


def sh_basis(d) -> np.ndarray:
    out = np.zeros(16, np.float32)
    lib().orc_sh_basis(float(np.float32(d[0])), float(np.float32(d[1])), float(np.float32(d[2])), _p(out))
    return out


def tile_span(u, v, r, TX, TY):
    out = np.zeros(4, np.int32)
    lib().orc_tile_span(float(np.float32(u)), float(np.float32(v)), float(np.float32(r)),
                        int(TX), int(TY), _p(out))
    return tuple(int(x) for x in out)


def exclusive_scan(counts):
    counts = _c(counts, np.uint32)
    offsets = np.zeros(max(counts.shape[0], 1), np.uint64)
    total = lib().orc_exclusive_scan(_p(counts), counts.shape[0], _p(offsets))
    return offsets[:counts.shape[0]], int(total)


def duplicate(cam: dict, xy_depth, tiles_touched, offsets, total):
    xy_depth = _c(xy_depth, np.float32)
    tiles_touched = _c(tiles_touched, np.uint32)
    offsets = _c(offsets, np.uint64)
    keys = np.zeros(max(total, 1), np.uint64)
    vals = np.zeros(max(total, 1), np.uint32)
    c = make_camera(cam)
    rc = lib().orc_duplicate(ctypes.byref(c), tiles_touched.shape[0], _p(xy_depth), _p(tiles_touched),
                             _p(offsets), _p(keys), _p(vals))
    if rc != 0:
        raise ValueError("orc_duplicate: a tile count disagrees with its span")
    return keys[:total], vals[:total]


def sort_pairs(keys, values):
    keys = np.array(keys, dtype=np.uint64, copy=True)
    values = np.array(values, dtype=np.uint32, copy=True)
    lib().orc_sort_pairs(_p(keys), _p(values), keys.shape[0])
    return keys, values


def preprocess(cam: dict, scene: dict, tile_test: int = 0):
    """Returns dict of xy_depth [n,4], conic_op [n,4], rgb [n,4], tiles_touched [n].
    tile_test: 0 = every tile of the span rectangle, 1 = the ellipse test."""
    n = int(scene["n"])
    means = _c(scene["means"], np.float32)
    scales = _c(scene["scales"], np.float32)
    quats = _c(scene["quats"], np.float32)
    opacity = _c(scene["opacity"], np.float32)
    sh = scene.get("sh")
    sh = None if sh is None else _c(sh, np.float32)
    rgb_in = scene.get("rgb")
    rgb_in = None if rgb_in is None else _c(rgb_in, np.float32)
    deg = int(scene.get("sh_degree", 0))
    out = dict(xy_depth=np.zeros((n, 4), np.float32), conic_op=np.zeros((n, 4), np.float32),
               rgb=np.zeros((n, 4), np.float32), tiles_touched=np.zeros(n, np.uint32))
    c = make_camera(cam)
    rc = lib().orc_preprocess_ex(ctypes.byref(c), n, _p(means), _p(scales), _p(quats), _p(opacity),
                                 _p(sh), deg, _p(rgb_in), _p(out["xy_depth"]), _p(out["conic_op"]),
                                 _p(out["rgb"]), _p(out["tiles_touched"]), int(tile_test))
    if rc != 0:
        raise ValueError("orc_preprocess rejected its arguments")
    return out


def preprocess_bwd(cam: dict, scene: dict, grad_mean2d, grad_conic_op, grad_rgb):
    """Backward of preprocess. Upstream gradients [n,2], [n,4], [n,4] (any
    float type, used as float64). Returns float64 dict grad_means [3,n],
    grad_scales [3,n], grad_quats [4,n], grad_opacity [n], and grad_sh
    [(d+1)^2*3, n] (coefficient-major, as the sh input) or grad_rgb_in [3,n]."""
    n = int(scene["n"])
    means = _c(scene["means"], np.float32)
    scales = _c(scene["scales"], np.float32)
    quats = _c(scene["quats"], np.float32)
    opacity = _c(scene["opacity"], np.float32)
    sh = scene.get("sh")
    sh = None if sh is None else _c(sh, np.float32)
    rgb_in = scene.get("rgb")
    rgb_in = None if rgb_in is None else _c(rgb_in, np.float32)
    deg = int(scene.get("sh_degree", 0))
    gm, gc, gr = (_c(a, np.float64) for a in (grad_mean2d, grad_conic_op, grad_rgb))
    out = dict(grad_means=np.zeros((3, n)), grad_scales=np.zeros((3, n)), grad_quats=np.zeros((4, n)),
               grad_opacity=np.zeros(n))
    if sh is not None:
        out["grad_sh"] = np.zeros((3 * (deg + 1) ** 2, n))
    else:
        out["grad_rgb_in"] = np.zeros((3, n))
    c = make_camera(cam)
    rc = lib().orc_preprocess_bwd(ctypes.byref(c), n, _p(means), _p(scales), _p(quats), _p(opacity),
                                  _p(sh), deg, _p(rgb_in), _p(gm), _p(gc), _p(gr), _p(out["grad_means"]),
                                  _p(out["grad_scales"]), _p(out["grad_quats"]), _p(out["grad_opacity"]),
                                  _p(out.get("grad_sh")), _p(out.get("grad_rgb_in")))
    if rc != 0:
        raise ValueError("orc_preprocess_bwd rejected its arguments")
    return out


def project_f64(cam: dict, mean, scale, quat, sh_coef=None, rgb=None):
    """The projection of one Gaussian in float64. sh_coef: [n_coef, 3] or
    None (then rgb [3]). Returns None when culled, else dict u, v, conic
    (A, B, C), rgb [3], clamp (x, y)."""
    m, s, q = (_c(a, np.float64) for a in (mean, scale, quat))
    shc = None if sh_coef is None else _c(sh_coef, np.float64)
    n_coef = 0 if shc is None else shc.shape[0]
    rgbc = None if rgb is None else _c(rgb, np.float64)
    out = np.zeros(10)
    c = make_camera(cam)
    if not lib().orc_project_f64(ctypes.byref(c), _p(m), _p(s), _p(q), _p(shc), n_coef, _p(rgbc), _p(out)):
        return None
    return dict(u=out[0], v=out[1], conic=out[2:5].copy(), rgb=out[5:8].copy(),
                clamp=(bool(out[8]), bool(out[9])))


def bin_and_sort(cam: dict, xy_depth, tiles_touched, conic_op=None, tile_test: int = 0):
    """Returns (keys u64 [E], point_list u32 [E]). tile_test 1 (the ellipse
    test) needs conic_op."""
    xy_depth = _c(xy_depth, np.float32)
    tiles_touched = _c(tiles_touched, np.uint32)
    conic_op = None if conic_op is None else _c(conic_op, np.float32)
    n = tiles_touched.shape[0]
    c = make_camera(cam)
    E = lib().orc_bin_ex(ctypes.byref(c), n, _p(xy_depth), _p(conic_op), _p(tiles_touched), None, None, 0,
                         int(tile_test))
    if E < 0:
        raise ValueError("orc_bin rejected its arguments")
    keys = np.zeros(max(E, 1), np.uint64)
    vals = np.zeros(max(E, 1), np.uint32)
    E2 = lib().orc_bin_ex(ctypes.byref(c), n, _p(xy_depth), _p(conic_op), _p(tiles_touched), _p(keys),
                          _p(vals), E, int(tile_test))
    assert E2 == E
    return keys[:E], vals[:E]


def tile_ranges(cam: dict, keys):
    keys = _c(keys, np.uint64)
    TX, TY = tiles_xy(cam)
    ranges = np.zeros((TX * TY, 2), np.uint32)
    c = make_camera(cam)
    lib().orc_tile_ranges(ctypes.byref(c), _p(keys), keys.shape[0], _p(ranges))
    return ranges


def composite_fwd(cam: dict, ranges, point_list, xy_depth, conic_op, rgb, bg=(0.0, 0.0, 0.0),
                  dtype=np.float32):
    """Returns dict image [3,H,W], final_T [H,W], n_contrib [H,W], n_examined [H,W]."""
    W, H = int(cam["width"]), int(cam["height"])
    ranges = _c(ranges, np.uint32)
    point_list = _c(point_list, np.uint32)
    xy_depth, conic_op, rgb = (_c(a, dtype) for a in (xy_depth, conic_op, rgb))
    bg = _c(bg, dtype)
    out = dict(image=np.zeros((3, H, W), dtype), final_T=np.zeros((H, W), dtype),
               n_contrib=np.zeros((H, W), np.uint32), n_examined=np.zeros((H, W), np.uint32))
    fn = lib().orc_composite_fwd_f32 if dtype == np.float32 else lib().orc_composite_fwd_f64
    c = make_camera(cam)
    fn(ctypes.byref(c), _p(ranges), _p(point_list), _p(xy_depth), _p(conic_op), _p(rgb), _p(bg),
       _p(out["image"]), _p(out["final_T"]), _p(out["n_contrib"]), _p(out["n_examined"]))
    return out


def composite_bwd(cam: dict, n: int, ranges, point_list, xy_depth, conic_op, rgb, final_T,
                  n_contrib, dL_dimage, bg=(0.0, 0.0, 0.0), dtype=np.float32, mass=False):
    """Returns dict grad_mean2d [n,2], grad_conic_op [n,4], grad_rgb [n,4] (float64).
    With mass (float32 only), also mass_mean2d, mass_conic_op, mass_rgb: per
    element, the sum over pixels of the magnitudes of its terms."""
    ranges = _c(ranges, np.uint32)
    point_list = _c(point_list, np.uint32)
    n_contrib = _c(n_contrib, np.uint32)
    xy_depth, conic_op, rgb, final_T, dL_dimage = (
        _c(a, dtype) for a in (xy_depth, conic_op, rgb, final_T, dL_dimage))
    bg = _c(bg, dtype)
    out = dict(grad_mean2d=np.zeros((n, 2), np.float64), grad_conic_op=np.zeros((n, 4), np.float64),
               grad_rgb=np.zeros((n, 4), np.float64))
    c = make_camera(cam)
    args = [ctypes.byref(c), n, _p(ranges), _p(point_list), _p(xy_depth), _p(conic_op), _p(rgb), _p(bg),
            _p(final_T), _p(n_contrib), _p(dL_dimage), _p(out["grad_mean2d"]), _p(out["grad_conic_op"]),
            _p(out["grad_rgb"])]
    if mass:
        assert dtype == np.float32, "the term magnitudes are taken of the float32 backward"
        for k, w in (("mass_mean2d", 2), ("mass_conic_op", 4), ("mass_rgb", 4)):
            out[k] = np.zeros((n, w), np.float64)
            args.append(_p(out[k]))
        lib().orc_composite_bwd_mass_f32(*args)
        return out
    fn = lib().orc_composite_bwd_f32 if dtype == np.float32 else lib().orc_composite_bwd_f64
    fn(*args)
    return out


def ellipse_row_range(u, v, r, conic, TX, TY, ty):
    """Kept tiles [lo, hi) of row ty under the ellipse test."""
    out = np.zeros(2, np.int32)
    f = lambda x: float(np.float32(x))
    lib().orc_ellipse_row_range(f(u), f(v), f(r), f(conic[0]), f(conic[1]), f(conic[2]), int(TX), int(TY),
                                int(ty), _p(out))
    return int(out[0]), int(out[1])


def render_fwd(cam: dict, scene: dict, bg=(0.0, 0.0, 0.0), tile_test: int = 0):
    """All forward stages; returns a dict with every intermediate."""
    pre = preprocess(cam, scene, tile_test)
    keys, point_list = bin_and_sort(cam, pre["xy_depth"], pre["tiles_touched"], pre["conic_op"], tile_test)
    ranges = tile_ranges(cam, keys)
    fwd = composite_fwd(cam, ranges, point_list, pre["xy_depth"], pre["conic_op"], pre["rgb"], bg)
    out = dict(pre)
    out.update(keys=keys, point_list=point_list, ranges=ranges, **fwd)
    return out
