"""Thin torch binding over the libgs C ABI.

torch supplies device memory and the current HIP stream; every step of the
path runs in libgs's kernels. Function names mirror the C entry points
(gs_preprocess -> preprocess, ...). Inputs must be contiguous float32 /
uint32-compatible tensors on a ROCm device.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np
import torch

from . import _lib
from ._lib import GsError

TILE = 16


def camera(cam: dict) -> _lib.GsCamera:
    """Build the C camera struct from a dict (R [9] row-major world->camera,
    t [3], campos [3], fx, fy, cx, cy, width, height)."""
    c = _lib.GsCamera()
    c.R[:] = [float(x) for x in np.asarray(cam["R"], np.float32).reshape(9)]
    c.t[:] = [float(x) for x in np.asarray(cam["t"], np.float32).reshape(3)]
    c.campos[:] = [float(x) for x in np.asarray(cam["campos"], np.float32).reshape(3)]
    c.fx, c.fy = float(np.float32(cam["fx"])), float(np.float32(cam["fy"]))
    c.cx, c.cy = float(np.float32(cam["cx"])), float(np.float32(cam["cy"]))
    c.width, c.height = int(cam["width"]), int(cam["height"])
    return c


def tiles_xy(cam: dict):
    return (int(cam["width"]) + TILE - 1) // TILE, (int(cam["height"]) + TILE - 1) // TILE


def _cam(cam):
    return cam if isinstance(cam, _lib.GsCamera) else camera(cam)


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def constants():
    out = np.zeros(9, np.float32)
    _lib.load().gs_constants(out.ctypes.data_as(ctypes.c_void_p))
    return out


def version():
    out = np.zeros(3, np.int32)
    _lib.load().gs_version(out.ctypes.data_as(ctypes.c_void_p))
    return tuple(int(x) for x in out)


def preprocess(cam, means, scales, quats, opacity, sh=None, sh_degree=0, rgb_in=None, out=None,
               stream=None, tile_test=0):
    """gs_preprocess_ex. Returns dict xy_depth [n,4], conic_op [n,4], rgb [n,4], tiles_touched [n].
    tile_test: _lib.GS_TILES_SQUARE (0) or _lib.GS_TILES_ELLIPSE (1)."""
    n = int(opacity.shape[0])
    dev = opacity.device
    if out is None:
        out = dict(xy_depth=torch.empty((n, 4), dtype=torch.float32, device=dev),
                   conic_op=torch.empty((n, 4), dtype=torch.float32, device=dev),
                   rgb=torch.empty((n, 4), dtype=torch.float32, device=dev),
                   tiles_touched=torch.empty((n,), dtype=torch.int32, device=dev))
    f32, i32 = torch.float32, torch.int32
    c = _cam(cam)
    _lib.check(_lib.load().gs_preprocess_ex(
        ctypes.byref(c), n, _ptr(means, f32, "means"), _ptr(scales, f32, "scales"),
        _ptr(quats, f32, "quats"), _ptr(opacity, f32, "opacity"), _ptr(sh, f32, "sh"),
        int(sh_degree), _ptr(rgb_in, f32, "rgb_in"), _ptr(out["xy_depth"], f32),
        _ptr(out["conic_op"], f32), _ptr(out["rgb"], f32), _ptr(out["tiles_touched"], i32),
        int(tile_test), _stream(stream)))
    return out


def preprocess_views(cams, means, scales, quats, opacity, sh=None, sh_degree=0, rgb_in=None, out=None,
                     stream=None, tile_test=0):
    """gs_preprocess_views: the records of n Gaussians for every camera of `cams` (one size).
    Returns dict xy_depth [V*n,4], conic_op [V*n,4], rgb [V*n,4], tiles_touched [V*n], camera
    v's records at v*n + g."""
    n = int(opacity.shape[0])
    V = len(cams)
    dev = opacity.device
    if out is None:
        out = dict(xy_depth=torch.empty((V * n, 4), dtype=torch.float32, device=dev),
                   conic_op=torch.empty((V * n, 4), dtype=torch.float32, device=dev),
                   rgb=torch.empty((V * n, 4), dtype=torch.float32, device=dev),
                   tiles_touched=torch.empty((V * n,), dtype=torch.int32, device=dev))
    f32, i32 = torch.float32, torch.int32
    arr = (_lib.GsCamera * V)(*[_cam(c) for c in cams])
    _lib.check(_lib.load().gs_preprocess_views(
        ctypes.cast(arr, ctypes.c_void_p), V, n, _ptr(means, f32, "means"), _ptr(scales, f32, "scales"),
        _ptr(quats, f32, "quats"), _ptr(opacity, f32, "opacity"), _ptr(sh, f32, "sh"),
        int(sh_degree), _ptr(rgb_in, f32, "rgb_in"), _ptr(out["xy_depth"], f32),
        _ptr(out["conic_op"], f32), _ptr(out["rgb"], f32), _ptr(out["tiles_touched"], i32),
        int(tile_test), _stream(stream)))
    return out


def preprocess_bwd(cam, means, scales=None, quats=None, sh=None, sh_degree=0, tiles_touched=None,
                   grad_mean2d=None, grad_conic_op=None, grad_rgb=None, out=None, stream=None):
    """gs_preprocess_bwd. Returns dict grad_means [3,n], grad_scales [3,n], grad_quats [4,n],
    grad_opacity [n], and grad_sh [(d+1)^2,3,n] (when sh is given) or grad_rgb_in [3,n]."""
    n = int(means.shape[1])
    dev = means.device
    f32, i32 = torch.float32, torch.int32
    if out is None:
        out = dict(grad_means=torch.empty((3, n), dtype=f32, device=dev),
                   grad_scales=torch.empty((3, n), dtype=f32, device=dev),
                   grad_quats=torch.empty((4, n), dtype=f32, device=dev),
                   grad_opacity=torch.empty((n,), dtype=f32, device=dev))
        if sh is not None:
            out["grad_sh"] = torch.empty(((sh_degree + 1) ** 2, 3, n), dtype=f32, device=dev)
        else:
            out["grad_rgb_in"] = torch.empty((3, n), dtype=f32, device=dev)
    c = _cam(cam)
    _lib.check(_lib.load().gs_preprocess_bwd(
        ctypes.byref(c), n, _ptr(means, f32, "means"), _ptr(scales, f32, "scales"),
        _ptr(quats, f32, "quats"), _ptr(sh, f32, "sh"), int(sh_degree),
        _ptr(tiles_touched, i32, "tiles_touched"), _ptr(grad_mean2d, f32, "grad_mean2d"),
        _ptr(grad_conic_op, f32, "grad_conic_op"), _ptr(grad_rgb, f32, "grad_rgb"),
        _ptr(out["grad_means"], f32), _ptr(out["grad_scales"], f32), _ptr(out["grad_quats"], f32),
        _ptr(out["grad_opacity"], f32), _ptr(out.get("grad_sh"), f32), _ptr(out.get("grad_rgb_in"), f32),
        _stream(stream)))
    return out


def appearance_params(n_latent: int, n_hidden: int) -> int:
    """Floats in the packed appearance weights: W1 [H][L+3], b1 [H], W2 [3][H], b2 [3]."""
    return n_hidden * (n_latent + 3) + 4 * n_hidden + 3


def appearance_fwd(cam, means, latent, weights, n_hidden, out=None, stream=None):
    """gs_appearance_fwd. latent [L, n]; returns rgb [3, n] (feed it to preprocess as rgb_in)."""
    L, n = int(latent.shape[0]), int(latent.shape[1])
    f32 = torch.float32
    if weights.numel() != appearance_params(L, n_hidden):
        raise ValueError("weights do not match n_latent / n_hidden")
    if out is None:
        out = torch.empty((3, n), dtype=f32, device=latent.device)
    c = _cam(cam)
    _lib.check(_lib.load().gs_appearance_fwd(ctypes.byref(c), n, _ptr(means, f32, "means"),
                                             _ptr(latent, f32, "latent"), L, int(n_hidden),
                                             _ptr(weights, f32, "weights"), _ptr(out, f32), _stream(stream)))
    return out


def appearance_bwd(cam, means, latent, weights, n_hidden, grad_rgb, out=None, scratch=None, stream=None):
    """gs_appearance_bwd. Returns dict grad_latent [L, n], grad_weights (packed as weights)."""
    L, n = int(latent.shape[0]), int(latent.shape[1])
    f32 = torch.float32
    dev = latent.device
    if out is None:
        out = dict(grad_latent=torch.empty((L, n), dtype=f32, device=dev),
                   grad_weights=torch.empty_like(weights))
    c = _cam(cam)
    lib = _lib.load()
    need = ctypes.c_size_t(0)
    _lib.check(lib.gs_appearance_bwd(ctypes.byref(c), n, None, None, L, int(n_hidden), None, None, None, None,
                                     None, ctypes.byref(need), None))
    if scratch is None or scratch.numel() < need.value:
        scratch = torch.empty((max(int(need.value), 4),), dtype=torch.uint8, device=dev)
    have = ctypes.c_size_t(scratch.numel())
    _lib.check(lib.gs_appearance_bwd(ctypes.byref(c), n, _ptr(means, f32, "means"), _ptr(latent, f32, "latent"), L,
                                     int(n_hidden), _ptr(weights, f32, "weights"), _ptr(grad_rgb, f32, "grad_rgb"),
                                     _ptr(out["grad_latent"], f32), _ptr(out["grad_weights"], f32),
                                     _ptr(scratch), ctypes.byref(have), _stream(stream)))
    return out


class BinBuffers:
    """Entry buffers (keys, point_list, scratch, the device entry count)
    reused across frames; grown on demand when a frame needs more entries
    than the capacity."""

    def __init__(self, device, capacity: int = 1 << 20):
        self.device = device
        self.capacity = 0
        self.keys = self.point_list = self.scratch = None
        self.n_entries_dev = torch.zeros((1,), dtype=torch.int64, device=device)
        self._need = {}
        self._ensure(int(capacity))

    def _ensure(self, capacity: int):
        if capacity > self.capacity:
            self.capacity = capacity
            self.keys = torch.empty((capacity,), dtype=torch.int64, device=self.device)
            self.point_list = torch.empty((capacity,), dtype=torch.int32, device=self.device)
            self.scratch = None
            self._need = {}

    def scratch_for(self, c, n: int):
        need = self._need.get(n)
        if need is None:
            q = ctypes.c_size_t(0)
            _lib.check(_lib.load().gs_bin_and_sort(ctypes.byref(c), n, None, None, None, None,
                                                   self.capacity, None, ctypes.byref(q), None, None))
            need = self._need[n] = int(q.value)
        if self.scratch is None or self.scratch.numel() < need:
            self.scratch = torch.empty((max(need, 256),), dtype=torch.uint8, device=self.device)
        return self.scratch

    def entries(self) -> int:
        """E of the last asynchronous binning (waits for the stream). E >
        capacity means the frame rendered nothing and must be redone after
        _ensure(E)."""
        return int(self.n_entries_dev.item())


def bin_and_sort(cam, xy_depth, tiles_touched, buffers: BinBuffers | None = None, stream=None,
                 conic_op=None, tile_test=0):
    """gs_bin_and_sort_ex. Returns (keys int64 [E] (uint64 bits), point_list int32 [E], E).
    The ellipse tile test (tile_test=1) needs conic_op.

    Grows the buffers and retries once if the entry count exceeds capacity.
    """
    c = _cam(cam)
    n = int(tiles_touched.shape[0])
    if buffers is None:
        buffers = BinBuffers(xy_depth.device, capacity=max(1024, 16 * n))
    lib = _lib.load()
    for attempt in range(2):
        scratch = buffers.scratch_for(c, n)
        nbytes = ctypes.c_size_t(scratch.numel())
        n_entries = ctypes.c_int64(0)
        st = lib.gs_bin_and_sort_ex(ctypes.byref(c), n, _ptr(xy_depth, torch.float32, "xy_depth"),
                                    _ptr(conic_op, torch.float32, "conic_op"),
                                    _ptr(tiles_touched, torch.int32, "tiles_touched"),
                                    _ptr(buffers.keys), _ptr(buffers.point_list), buffers.capacity,
                                    _ptr(scratch), ctypes.byref(nbytes), ctypes.byref(n_entries),
                                    int(tile_test), _stream(stream))
        if st == _lib.GS_ERR_CAPACITY and attempt == 0:
            buffers._ensure(int(n_entries.value * 5 // 4 + 1024))
            continue
        _lib.check(st)
        E = int(n_entries.value)
        return buffers.keys[:E], buffers.point_list[:E], E
    raise AssertionError("unreachable")


def bin_and_sort_async(cam, xy_depth, tiles_touched, buffers: BinBuffers, stream=None, conic_op=None,
                       tile_test=0):
    """gs_bin_and_sort_async_ex: never waits. Returns (keys int64 [capacity], point_list int32
    [capacity]); E lands in buffers.n_entries_dev (read it with buffers.entries())."""
    c = _cam(cam)
    n = int(tiles_touched.shape[0])
    scratch = buffers.scratch_for(c, n)
    nbytes = ctypes.c_size_t(scratch.numel())
    _lib.check(_lib.load().gs_bin_and_sort_async_ex(
        ctypes.byref(c), n, _ptr(xy_depth, torch.float32, "xy_depth"), _ptr(conic_op, torch.float32, "conic_op"),
        _ptr(tiles_touched, torch.int32, "tiles_touched"), _ptr(buffers.keys), _ptr(buffers.point_list),
        buffers.capacity, _ptr(scratch), ctypes.byref(nbytes), _ptr(buffers.n_entries_dev), int(tile_test),
        _stream(stream)))
    return buffers.keys, buffers.point_list


def bin_and_sort_async_noalloc(cam, xy_depth, tiles_touched, keys, point_list, n_entries_dev, stream=None,
                               conic_op=None, tile_test=0):
    """gs_bin_and_sort_async_noalloc: as bin_and_sort_async, into the caller's keys (int64
    [capacity]) and point_list (int32 [capacity]), with the library's fixed workspace instead
    of a scratch buffer. E lands in n_entries_dev (int64 [1]). Calls that overlap on one GPU
    race on that workspace."""
    c = _cam(cam)
    n = int(tiles_touched.shape[0])
    capacity = int(keys.numel())
    if point_list.numel() != capacity:
        raise ValueError("keys and point_list must have the same length")
    _lib.check(_lib.load().gs_bin_and_sort_async_noalloc(
        ctypes.byref(c), n, _ptr(xy_depth, torch.float32, "xy_depth"), _ptr(conic_op, torch.float32, "conic_op"),
        _ptr(tiles_touched, torch.int32, "tiles_touched"), _ptr(keys, torch.int64, "keys"),
        _ptr(point_list, torch.int32, "point_list"), capacity, _ptr(n_entries_dev, torch.int64, "n_entries_dev"),
        int(tile_test), _stream(stream)))
    return keys, point_list


def _check_chunks(chunks, cam, capacity, n_views=1):
    need = chunk_words(cam, capacity, n_views)
    if chunks.dtype != torch.int32 or chunks.numel() < need:
        raise ValueError(f"chunks must be int32 with at least {need} elements")


def bin_and_sort_views_async(cam, n_views: int, xy_depth, tiles_touched, buffers: BinBuffers, stream=None,
                             conic_op=None, tile_test=0):
    """gs_bin_and_sort_views_async: one binning of a stack of n_views views of cam's size
    (records from preprocess_views). Returns (keys, point_list), both [capacity]; E lands in
    buffers.n_entries_dev."""
    c = _cam(cam)
    n_all = int(tiles_touched.shape[0])
    if n_all % n_views:
        raise ValueError("the records must hold n_views equal views")
    scratch = buffers.scratch_for(c, n_all)
    nbytes = ctypes.c_size_t(scratch.numel())
    _lib.check(_lib.load().gs_bin_and_sort_views_async(
        ctypes.byref(c), int(n_views), n_all // n_views, _ptr(xy_depth, torch.float32, "xy_depth"),
        _ptr(conic_op, torch.float32, "conic_op"), _ptr(tiles_touched, torch.int32, "tiles_touched"),
        _ptr(buffers.keys), _ptr(buffers.point_list), buffers.capacity, _ptr(scratch), ctypes.byref(nbytes),
        _ptr(buffers.n_entries_dev), int(tile_test), _stream(stream)))
    return buffers.keys, buffers.point_list


def tile_ranges_async(cam, buffers: BinBuffers, out=None, order=None, stream=None, chunks=None, n_views=1):
    """gs_tile_ranges_async over the last asynchronous binning into buffers.
    `order` (int32 [TX*TY]) receives the heaviest-first tile schedule if given;
    `chunks` (int32 [chunk_words(cam, buffers.capacity)]) the chunk schedule of
    the chunked backward (gs_tile_ranges_ex); n_views > 1: the tiles of a view
    stack (bin_and_sort_views_async)."""
    c = _cam(cam)
    if out is None:
        TX, TY = tiles_xy(dict(width=c.width, height=c.height))
        out = torch.empty((TX * TY * n_views, 2), dtype=torch.int32, device=buffers.keys.device)
    if chunks is not None or n_views != 1:
        if chunks is not None:
            _check_chunks(chunks, cam, buffers.capacity, n_views)
        _lib.check(_lib.load().gs_tile_ranges_ex(ctypes.byref(c), int(n_views), _ptr(buffers.keys), 0,
                                                 _ptr(buffers.n_entries_dev), buffers.capacity,
                                                 _ptr(out, torch.int32), _ptr(order, torch.int32, "order"),
                                                 _ptr(chunks, torch.int32, "chunks"), _stream(stream)))
        return out
    _lib.check(_lib.load().gs_tile_ranges_async(ctypes.byref(c), _ptr(buffers.keys), _ptr(buffers.n_entries_dev),
                                                buffers.capacity, _ptr(out, torch.int32),
                                                _ptr(order, torch.int32, "order"), _stream(stream)))
    return out


def tile_ranges(cam, keys, n_entries: int, out=None, order=None, stream=None, chunks=None):
    """gs_tile_ranges. Returns ranges int32 [TX*TY, 2] (uint32 values); `order`
    (int32 [TX*TY]) receives the heaviest-first tile schedule if given; `chunks`
    (int32 [chunk_words(cam, len(keys))]) the chunk schedule of the chunked
    backward (gs_tile_ranges_ex)."""
    TX, TY = tiles_xy(cam if isinstance(cam, dict) else
                      dict(width=cam.width, height=cam.height))
    if out is None:
        out = torch.empty((TX * TY, 2), dtype=torch.int32, device=keys.device)
    c = _cam(cam)
    if chunks is not None:
        _check_chunks(chunks, cam, keys.numel())
        _lib.check(_lib.load().gs_tile_ranges_ex(ctypes.byref(c), 1, _ptr(keys, torch.int64, "keys"), int(n_entries),
                                                 None, int(keys.numel()), _ptr(out, torch.int32),
                                                 _ptr(order, torch.int32, "order"),
                                                 _ptr(chunks, torch.int32, "chunks"), _stream(stream)))
        return out
    _lib.check(_lib.load().gs_tile_ranges(ctypes.byref(c), _ptr(keys, torch.int64, "keys"),
                                          int(n_entries), _ptr(out, torch.int32),
                                          _ptr(order, torch.int32, "order"), _stream(stream)))
    return out


# Below this many tiles a frame cannot fill the GPU's workgroup slots with
# whole lists, and the forward composites the chunk schedule instead.
SCHEDULED_FORWARD_MAX_TILES = 2048


def scheduled_forward(cam) -> bool:
    """Whether Rasterizer and ViewBatch composite the forward by the chunk
    schedule for this camera (small tile grids: few, long lists)."""
    TX, TY = tiles_xy(cam if isinstance(cam, dict) else dict(width=cam.width, height=cam.height))
    return TX * TY < SCHEDULED_FORWARD_MAX_TILES


def ckpt_rows(capacity: int) -> int:
    """Rows of the checkpoint buffer gs_composite_fwd_ex needs for `capacity` entries."""
    return (int(capacity) + 255) // 256 * 256


def chunk_words(cam, capacity: int, n_views: int = 1) -> int:
    """Length of the chunk schedule gs_tile_ranges_ex writes for `capacity` entries."""
    TX, TY = tiles_xy(cam if isinstance(cam, dict) else dict(width=cam.width, height=cam.height))
    return 4 + 4 * (TX * TY * n_views + (int(capacity) + 255) // 256)


def part_bytes(cam, capacity: int, n_views: int = 1) -> int:
    """Bytes of the workspace the scheduled forward (composite_fwd with chunks) needs."""
    c = _cam(cam)
    return int(_lib.load().gs_composite_part_bytes(ctypes.byref(c), int(n_views), int(capacity)))


def composite_fwd(cam, ranges, point_list, xy_depth, conic_op, rgb, bg=(0.0, 0.0, 0.0),
                  with_examined=False, out=None, order=None, stream=None, ckpt=None, capacity=None,
                  chunks=None, part=None, n_views=1):
    """gs_composite_fwd, or gs_composite_fwd_ex when `ckpt` (float32 [ckpt_rows(capacity), 4]) or
    `chunks` is given: ckpt then receives the per-pixel state at every 256-entry boundary, for
    composite_bwd's chunked walk; with the schedule `chunks` (from tile_ranges) the lists are
    composited as its work items, long ones in 256-entry chunks, in the workspace `part`
    (uint8 [part_bytes(cam, capacity)]; allocated here if not given). capacity defaults to
    point_list's length. Returns dict image [3,H,W], final_T [H,W], n_contrib [H,W] (int32), and
    n_examined [H,W] when requested."""
    W, H = (cam["width"], cam["height"]) if isinstance(cam, dict) else (cam.width, cam.height)
    dev = xy_depth.device
    if out is None:
        lead = (n_views,) if n_views != 1 else ()
        out = dict(image=torch.empty(lead + (3, H, W), dtype=torch.float32, device=dev),
                   final_T=torch.empty(lead + (H, W), dtype=torch.float32, device=dev),
                   n_contrib=torch.empty(lead + (H, W), dtype=torch.int32, device=dev))
        if with_examined:
            out["n_examined"] = torch.empty(lead + (H, W), dtype=torch.int32, device=dev)
    bgc = (ctypes.c_float * 3)(*[float(x) for x in bg])
    c = _cam(cam)
    if ckpt is not None or chunks is not None or n_views != 1:
        nk = int(point_list.numel() if capacity is None else capacity)
        if ckpt is not None and (ckpt.dtype != torch.float32 or ckpt.numel() < 4 * ckpt_rows(nk)):
            raise ValueError(f"ckpt must be float32 with at least {ckpt_rows(nk)} rows of 4")
        if chunks is not None:
            _check_chunks(chunks, cam, nk, n_views)
            need = part_bytes(cam, nk, n_views)
            if part is None:
                part = torch.empty((need,), dtype=torch.uint8, device=xy_depth.device)
            elif part.numel() * part.element_size() < need:
                raise ValueError(f"part must hold at least {need} bytes")
        _lib.check(_lib.load().gs_composite_fwd_ex(
            ctypes.byref(c), int(n_views), _ptr(ranges, torch.int32, "ranges"),
            _ptr(point_list, torch.int32, "point_list"),
            _ptr(xy_depth, torch.float32), _ptr(conic_op, torch.float32), _ptr(rgb, torch.float32),
            ctypes.cast(bgc, ctypes.c_void_p), _ptr(out["image"]), _ptr(out["final_T"]),
            _ptr(out["n_contrib"]), _ptr(out.get("n_examined")), _ptr(order, torch.int32, "order"), nk,
            _ptr(ckpt, torch.float32, "ckpt"), _ptr(chunks, torch.int32, "chunks"),
            _ptr(part if chunks is not None else None, None, "part"), _stream(stream)))
        return out
    _lib.check(_lib.load().gs_composite_fwd(
        ctypes.byref(c), _ptr(ranges, torch.int32, "ranges"), _ptr(point_list, torch.int32, "point_list"),
        _ptr(xy_depth, torch.float32), _ptr(conic_op, torch.float32), _ptr(rgb, torch.float32),
        ctypes.cast(bgc, ctypes.c_void_p), _ptr(out["image"]), _ptr(out["final_T"]),
        _ptr(out["n_contrib"]), _ptr(out.get("n_examined")), _ptr(order, torch.int32, "order"),
        _stream(stream)))
    return out


def composite_bwd(cam, n, ranges, point_list, xy_depth, conic_op, rgb, final_T, n_contrib,
                  dL_dimage, bg=(0.0, 0.0, 0.0), out=None, order=None, stream=None, chunks=None, image=None,
                  ckpt=None, capacity=None, n_views=1):
    """gs_composite_bwd, or gs_composite_bwd_ex (one workgroup per 256-entry chunk of a list)
    when `chunks` is given, with the `image` and `ckpt` of the same frame's
    composite_fwd(ckpt=..., capacity=...) and that capacity (default: point_list's length).
    Returns dict grad_mean2d [n,2], grad_conic_op [n,4], grad_rgb [n,4]."""
    dev = xy_depth.device
    if out is None:
        out = dict(grad_mean2d=torch.empty((n, 2), dtype=torch.float32, device=dev),
                   grad_conic_op=torch.empty((n, 4), dtype=torch.float32, device=dev),
                   grad_rgb=torch.empty((n, 4), dtype=torch.float32, device=dev))
    bgc = (ctypes.c_float * 3)(*[float(x) for x in bg])
    c = _cam(cam)
    if n_views != 1 and chunks is None:
        raise ValueError("the backward of a view stack takes the schedule (chunks)")
    if chunks is not None:
        if ckpt is None or image is None:
            raise ValueError("the chunked backward needs the forward's image and ckpt")
        cap = int(point_list.numel() if capacity is None else capacity)
        _check_chunks(chunks, cam, cap, n_views)
        if ckpt.dtype != torch.float32 or ckpt.numel() < 4 * ckpt_rows(cap):
            raise ValueError(f"ckpt must be float32 with at least {ckpt_rows(cap)} rows of 4")
        _lib.check(_lib.load().gs_composite_bwd_ex(
            ctypes.byref(c), int(n_views), int(n), _ptr(ranges, torch.int32, "ranges"),
            _ptr(point_list, torch.int32, "point_list"), _ptr(chunks, torch.int32, "chunks"), cap,
            _ptr(xy_depth, torch.float32), _ptr(conic_op, torch.float32), _ptr(rgb, torch.float32),
            ctypes.cast(bgc, ctypes.c_void_p), _ptr(image, torch.float32, "image"),
            _ptr(final_T, torch.float32, "final_T"), _ptr(n_contrib, torch.int32, "n_contrib"),
            _ptr(ckpt, torch.float32, "ckpt"), _ptr(dL_dimage, torch.float32, "dL_dimage"),
            _ptr(out["grad_mean2d"]), _ptr(out["grad_conic_op"]), _ptr(out["grad_rgb"]), _stream(stream)))
        return out
    _lib.check(_lib.load().gs_composite_bwd(
        ctypes.byref(c), int(n), _ptr(ranges, torch.int32, "ranges"),
        _ptr(point_list, torch.int32, "point_list"), _ptr(xy_depth, torch.float32),
        _ptr(conic_op, torch.float32), _ptr(rgb, torch.float32), ctypes.cast(bgc, ctypes.c_void_p),
        _ptr(final_T, torch.float32, "final_T"), _ptr(n_contrib, torch.int32, "n_contrib"),
        _ptr(dL_dimage, torch.float32, "dL_dimage"), _ptr(out["grad_mean2d"]),
        _ptr(out["grad_conic_op"]), _ptr(out["grad_rgb"]), _ptr(order, torch.int32, "order"),
        _stream(stream)))
    return out


@dataclass
class Scene:
    """Device-resident Gaussian parameters in the C-ABI layouts."""
    means: torch.Tensor
    scales: torch.Tensor
    quats: torch.Tensor
    opacity: torch.Tensor
    sh: torch.Tensor | None = None
    sh_degree: int = 0
    rgb: torch.Tensor | None = None

    @property
    def n(self) -> int:
        return int(self.opacity.shape[0])

    @staticmethod
    def from_numpy(d: dict, device="cuda") -> "Scene":
        t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)
        return Scene(t(d["means"]), t(d["scales"]), t(d["quats"]), t(d["opacity"]), t(d.get("sh")),
                     int(d.get("sh_degree", 0)), t(d.get("rgb")))


class Rasterizer:
    """Runs the whole path for one camera at a time, reusing its buffers."""

    def __init__(self, device="cuda", capacity: int = 1 << 20, tile_test: int = 0):
        self.device = torch.device(device)
        self.bins = BinBuffers(self.device, capacity)
        self.tile_test = int(tile_test)

    def forward(self, cam: dict, scene: Scene, bg=(0.0, 0.0, 0.0), with_examined=False,
                checkpoints=True, scheduled=None):
        """Render one view. With checkpoints (the default) the forward keeps the
        per-pixel state at every 256-entry boundary, and backward() then walks
        long lists in 256-entry chunks in parallel; without, backward() walks
        each list whole. With scheduled, the forward too composites the work
        items of the chunk schedule (long lists in chunks); by default it does
        when the tile grid alone is small (see scheduled_forward)."""
        c = camera(cam)
        pre = preprocess(c, scene.means, scene.scales, scene.quats, scene.opacity, scene.sh,
                         scene.sh_degree, scene.rgb, tile_test=self.tile_test)
        keys, point_list, E = bin_and_sort(c, pre["xy_depth"], pre["tiles_touched"], self.bins,
                                           conic_op=pre["conic_op"], tile_test=self.tile_test)
        TX, TY = tiles_xy(cam)
        order = torch.empty((TX * TY,), dtype=torch.int32, device=self.device)
        if scheduled is None:
            # the schedule cuts lists only when they average more than a chunk
            # (E known here); otherwise its items are the tiles themselves
            scheduled = scheduled_forward(cam) and E > 256 * TX * TY
        chunks = (torch.empty((chunk_words(cam, E),), dtype=torch.int32, device=self.device)
                  if checkpoints or scheduled else None)
        ranges = tile_ranges(cam, keys, E, order=order, chunks=chunks)
        ckpt = torch.empty((ckpt_rows(E), 4), dtype=torch.float32, device=self.device) if checkpoints else None
        fwd = composite_fwd(cam, ranges, point_list, pre["xy_depth"], pre["conic_op"], pre["rgb"], bg,
                            with_examined=with_examined, order=order, ckpt=ckpt, capacity=E,
                            chunks=chunks if scheduled else None)
        if checkpoints:
            fwd.update(ckpt=ckpt, chunks=chunks)
        out = dict(pre)
        out.update(keys=keys, point_list=point_list, n_entries=E, ranges=ranges, tile_order=order, **fwd)
        return out

    def backward(self, cam: dict, scene: Scene, fwd: dict, dL_dimage, bg=(0.0, 0.0, 0.0),
                 to_parameters=False):
        """Gradients of the splat records (grad_mean2d, grad_conic_op, grad_rgb); with
        to_parameters, also those of the Gaussians' parameters (gs_preprocess_bwd)."""
        ch = fwd.get("chunks")
        g = composite_bwd(cam, scene.n, fwd["ranges"], fwd["point_list"], fwd["xy_depth"],
                          fwd["conic_op"], fwd["rgb"], fwd["final_T"], fwd["n_contrib"], dL_dimage, bg,
                          order=fwd.get("tile_order"), chunks=ch, image=fwd["image"] if ch is not None else None,
                          ckpt=fwd.get("ckpt"), capacity=fwd["n_entries"])
        if to_parameters:
            g.update(preprocess_bwd(cam, scene.means, scene.scales, scene.quats, scene.sh, scene.sh_degree,
                                    fwd["tiles_touched"], g["grad_mean2d"], g["grad_conic_op"], g["grad_rgb"]))
        return g


class ViewBatch:
    """Forward and backward of one scene seen from a fixed list of cameras,
    enqueued with no host synchronisation (asynchronous binning keeps each
    view's entry count on the device), so the whole batch can be recorded
    once as a HIP graph and replayed.

    Each view owns its buffers, sized for `capacity` entries. A view whose
    entry count exceeds the capacity renders the background; `entries()`
    reads every view's count after a run (one wait per batch, not per frame)
    and `check()` raises if any view overflowed.

    loss_grad(view, image, out): writes dL/dI of that view into `out`
    ([3, H, W] float32) from its rendered image; it is enqueued on the same
    stream between the forward and the backward, so it must not allocate or
    synchronise if the batch is to be captured.
    """

    def __init__(self, cams, scene: "Scene", capacity: int, device="cuda", bg=(0.0, 0.0, 0.0),
                 tile_order=True, streams: int = 1, tile_test: int = 0, chunked: bool = True,
                 scheduled=None):
        self.device = torch.device(device)
        self.scene = scene
        self.bg = bg
        self.tile_test = int(tile_test)
        self.views = []
        # views are spread round-robin over `streams` streams (default
        # priority), so small frames that cannot fill the GPU alone overlap
        self.streams = [torch.cuda.Stream(device=self.device) for _ in range(streams)] if streams > 1 else []
        n = scene.n
        f32, i32 = torch.float32, torch.int32
        for cam in cams:
            c = camera(cam)
            W, H = int(cam["width"]), int(cam["height"])
            TX, TY = tiles_xy(cam)
            bins = BinBuffers(self.device, capacity)
            bins.scratch_for(c, n)
            v = dict(
                cam=cam, c=c, bins=bins,
                pre=dict(xy_depth=torch.empty((n, 4), dtype=f32, device=self.device),
                         conic_op=torch.empty((n, 4), dtype=f32, device=self.device),
                         rgb=torch.empty((n, 4), dtype=f32, device=self.device),
                         tiles_touched=torch.empty((n,), dtype=i32, device=self.device)),
                ranges=torch.empty((TX * TY, 2), dtype=i32, device=self.device),
                order=torch.empty((TX * TY,), dtype=i32, device=self.device) if tile_order else None,
                fwd=dict(image=torch.empty((3, H, W), dtype=f32, device=self.device),
                         final_T=torch.empty((H, W), dtype=f32, device=self.device),
                         n_contrib=torch.empty((H, W), dtype=i32, device=self.device)),
                # forward state at 256-entry boundaries and the chunk schedule, for the chunked backward
                ckpt=torch.empty((ckpt_rows(capacity), 4), dtype=f32, device=self.device) if chunked else None,
                chunks=torch.empty((chunk_words(cam, capacity),), dtype=i32, device=self.device) if chunked else None,
                part=(torch.empty((part_bytes(cam, capacity),), dtype=torch.uint8, device=self.device)
                      if chunked and (scheduled_forward(cam) if scheduled is None else scheduled) else None),
                dL_dimage=torch.zeros((3, H, W), dtype=f32, device=self.device),
                grads=dict(grad_mean2d=torch.empty((n, 2), dtype=f32, device=self.device),
                           grad_conic_op=torch.empty((n, 4), dtype=f32, device=self.device),
                           grad_rgb=torch.empty((n, 4), dtype=f32, device=self.device)))
            self.views.append(v)
        self.graph = None

    def enqueue(self, loss_grad=None):
        """Enqueue every view on the current stream (forked over the batch's
        streams and joined back when it has several): preprocess, binning,
        ranges, forward, loss_grad (if given), backward. Nothing waits on the
        host."""
        main = torch.cuda.current_stream(self.device)
        if self.streams:
            fork = torch.cuda.Event()
            fork.record(main)
            for s in self.streams:
                s.wait_event(fork)
        for i, v in enumerate(self.views):
            s = self.streams[i % len(self.streams)] if self.streams else main
            with torch.cuda.stream(s):
                self._enqueue_view(i, v, loss_grad)
        for s in self.streams:
            join = torch.cuda.Event()
            join.record(s)
            main.wait_event(join)

    def _enqueue_view(self, i, v, loss_grad):
        sc = self.scene
        c, pre, bins = v["c"], v["pre"], v["bins"]
        preprocess(c, sc.means, sc.scales, sc.quats, sc.opacity, sc.sh, sc.sh_degree, sc.rgb, out=pre,
                   tile_test=self.tile_test)
        keys, pl = bin_and_sort_async(c, pre["xy_depth"], pre["tiles_touched"], bins, conic_op=pre["conic_op"],
                                      tile_test=self.tile_test)
        tile_ranges_async(c, bins, out=v["ranges"], order=v["order"], chunks=v["chunks"])
        composite_fwd(c, v["ranges"], pl, pre["xy_depth"], pre["conic_op"], pre["rgb"], self.bg,
                      out=v["fwd"], order=v["order"], ckpt=v["ckpt"], capacity=bins.capacity,
                      chunks=v["chunks"] if v["part"] is not None else None, part=v["part"])
        if loss_grad is not None:
            loss_grad(i, v["fwd"]["image"], v["dL_dimage"])
        composite_bwd(c, sc.n, v["ranges"], pl, pre["xy_depth"], pre["conic_op"], pre["rgb"],
                      v["fwd"]["final_T"], v["fwd"]["n_contrib"], v["dL_dimage"], self.bg,
                      out=v["grads"], order=v["order"], chunks=v["chunks"], image=v["fwd"]["image"],
                      ckpt=v["ckpt"], capacity=bins.capacity)

    def capture(self, loss_grad=None, warmup: int = 1):
        """Record enqueue(loss_grad) as one HIP graph (after `warmup` eager runs
        on a side stream, as graph capture requires)."""
        s = torch.cuda.Stream(device=self.device)
        s.wait_stream(torch.cuda.current_stream(self.device))
        with torch.cuda.stream(s):
            for _ in range(warmup):
                self.enqueue(loss_grad)
        torch.cuda.current_stream(self.device).wait_stream(s)
        torch.cuda.synchronize(self.device)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.enqueue(loss_grad)
        return self.graph

    def replay(self):
        if self.graph is None:
            raise RuntimeError("ViewBatch.replay: capture() first")
        self.graph.replay()

    def entries(self):
        """Entry count of every view after the last run (waits for the stream)."""
        return [v["bins"].entries() for v in self.views]

    def check(self):
        E = self.entries()
        over = [(i, e) for i, e in enumerate(E) if e > self.views[i]["bins"].capacity]
        if over:
            raise GsError(_lib.GS_ERR_CAPACITY, f"views over capacity (view, entries): {over}")
        return E


class _StackGroup:
    """The buffers and launch sequence of one stack of views (see ViewStack)."""

    def __init__(self, cams, scene, capacity, device, tile_test, scheduled, fwd, dL, grads, first):
        self.cams, self.scene, self.tile_test, self.first = cams, scene, tile_test, first
        V = self.V = len(cams)
        self.c = camera(cams[0])  # the size of one view
        n = scene.n
        TX, TY = tiles_xy(cams[0])
        f32, i32, dev = torch.float32, torch.int32, device
        self.bins = BinBuffers(dev, capacity)
        self.bins.scratch_for(self.c, V * n)
        self.pre = dict(xy_depth=torch.empty((V * n, 4), dtype=f32, device=dev),
                        conic_op=torch.empty((V * n, 4), dtype=f32, device=dev),
                        rgb=torch.empty((V * n, 4), dtype=f32, device=dev),
                        tiles_touched=torch.empty((V * n,), dtype=i32, device=dev))
        self.ranges = torch.empty((V * TX * TY, 2), dtype=i32, device=dev)
        self.order = torch.empty((V * TX * TY,), dtype=i32, device=dev)
        self.chunks = torch.empty((chunk_words(self.c, capacity, V),), dtype=i32, device=dev)
        self.ckpt = torch.empty((ckpt_rows(capacity), 4), dtype=f32, device=dev)
        # the scheduled forward when the stacked grid is small (few, long lists)
        if scheduled is None:
            scheduled = V * TX * TY < SCHEDULED_FORWARD_MAX_TILES
        self.part = (torch.empty((part_bytes(self.c, capacity, V),), dtype=torch.uint8, device=dev)
                     if scheduled else None)
        sl = slice(first, first + V)
        self.fwd = {k: t[sl] for k, t in fwd.items()}
        self.dL_dimage = dL[sl]
        self.grads = {k: t[first * n:(first + V) * n] for k, t in grads.items()}

    def enqueue(self, bg, loss_grad):
        sc, V, c = self.scene, self.V, self.c
        preprocess_views(self.cams, sc.means, sc.scales, sc.quats, sc.opacity, sc.sh, sc.sh_degree, sc.rgb,
                         out=self.pre, tile_test=self.tile_test)
        keys, pl = bin_and_sort_views_async(c, V, self.pre["xy_depth"], self.pre["tiles_touched"], self.bins,
                                            conic_op=self.pre["conic_op"], tile_test=self.tile_test)
        tile_ranges_async(c, self.bins, out=self.ranges, order=self.order, chunks=self.chunks, n_views=V)
        composite_fwd(c, self.ranges, pl, self.pre["xy_depth"], self.pre["conic_op"], self.pre["rgb"], bg,
                      out=self.fwd, order=self.order, ckpt=self.ckpt, capacity=self.bins.capacity,
                      chunks=self.chunks if self.part is not None else None, part=self.part, n_views=V)
        if loss_grad is not None:
            loss_grad(self.first, self.fwd["image"], self.dL_dimage)
        composite_bwd(c, V * sc.n, self.ranges, pl, self.pre["xy_depth"], self.pre["conic_op"], self.pre["rgb"],
                      self.fwd["final_T"], self.fwd["n_contrib"], self.dL_dimage, bg, out=self.grads,
                      chunks=self.chunks, image=self.fwd["image"], ckpt=self.ckpt, capacity=self.bins.capacity,
                      n_views=V)


class ViewStack:
    """A batch of views of one size composited as stacked frames: in a stack,
    view v is the band of tile rows [v TY, v TY + TY) of one tile grid, so
    each stage (one preprocess for all its cameras, one binning, one ranges
    call, one forward, one backward) is a single launch sequence over the
    stack instead of one per view. With streams > 1 the batch is cut into
    that many stacks, each on its own stream (the stages of one fill the
    gaps between those of another). Images are [V, 3, H, W], per-pixel
    buffers [V, H, W], splat records' gradients [V*n, ...] (view v's at
    v*n + g). No host synchronisation; `check()` reports an overflow of a
    stack's `capacity` entries (that stack then renders the background).

    loss_grad(first, image, out): writes dL/dI of views first, first + 1,
    ... (out and image are [k, 3, H, W] slices of the batch) from their
    images; enqueued between each stack's forward and backward.
    """

    def __init__(self, cams, scene: "Scene", capacity: int, device="cuda", bg=(0.0, 0.0, 0.0),
                 tile_test: int = 0, scheduled=None, streams: int = 1):
        self.device = torch.device(device)
        self.scene, self.bg = scene, bg
        cams = list(cams)
        self.V = V = len(cams)
        W, H = int(cams[0]["width"]), int(cams[0]["height"])
        if any(int(c["width"]) != W or int(c["height"]) != H for c in cams):
            raise ValueError("a view stack needs cameras of one size")
        S = max(1, min(int(streams), V))
        n, f32, i32, dev = scene.n, torch.float32, torch.int32, self.device
        self.fwd = dict(image=torch.empty((V, 3, H, W), dtype=f32, device=dev),
                        final_T=torch.empty((V, H, W), dtype=f32, device=dev),
                        n_contrib=torch.empty((V, H, W), dtype=i32, device=dev))
        self.dL_dimage = torch.zeros((V, 3, H, W), dtype=f32, device=dev)
        self.grads = dict(grad_mean2d=torch.empty((V * n, 2), dtype=f32, device=dev),
                          grad_conic_op=torch.empty((V * n, 4), dtype=f32, device=dev),
                          grad_rgb=torch.empty((V * n, 4), dtype=f32, device=dev))
        bounds = [round(i * V / S) for i in range(S + 1)]
        self.groups = [_StackGroup(cams[bounds[i]:bounds[i + 1]], scene, capacity, dev, int(tile_test), scheduled,
                                   self.fwd, self.dL_dimage, self.grads, bounds[i]) for i in range(S)]
        # default-priority streams for every stack but the first, which runs on the caller's
        self.streams = [torch.cuda.Stream(device=dev) for _ in range(S - 1)]
        self.graph = None

    def enqueue(self, loss_grad=None):
        """Enqueue the batch on the current stream (forked over the stacks' streams and
        joined back): per stack preprocess, binning, ranges and schedule, forward,
        loss_grad (if given), backward. Nothing waits on the host."""
        main = torch.cuda.current_stream(self.device)
        if self.streams:
            fork = torch.cuda.Event()
            fork.record(main)
            for s in self.streams:
                s.wait_event(fork)
        for i, grp in enumerate(self.groups):
            with torch.cuda.stream(self.streams[i - 1] if i else main):
                grp.enqueue(self.bg, loss_grad)
        for s in self.streams:
            join = torch.cuda.Event()
            join.record(s)
            main.wait_event(join)

    def capture(self, loss_grad=None, warmup: int = 1):
        """Record enqueue(loss_grad) as one HIP graph (after `warmup` eager runs on a side
        stream, as graph capture requires)."""
        s = torch.cuda.Stream(device=self.device)
        s.wait_stream(torch.cuda.current_stream(self.device))
        with torch.cuda.stream(s):
            for _ in range(warmup):
                self.enqueue(loss_grad)
        torch.cuda.current_stream(self.device).wait_stream(s)
        torch.cuda.synchronize(self.device)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.enqueue(loss_grad)
        return self.graph

    def replay(self):
        if self.graph is None:
            raise RuntimeError("ViewStack.replay: capture() first")
        self.graph.replay()

    def entries(self):
        """Entries of each stack after the last run (waits for the stream)."""
        return [g.bins.entries() for g in self.groups]

    def check(self):
        E = self.entries()
        over = [(i, e) for i, (e, g) in enumerate(zip(E, self.groups)) if e > g.bins.capacity]
        if over:
            raise GsError(_lib.GS_ERR_CAPACITY, f"stacks over capacity (stack, entries): {over}")
        return E
