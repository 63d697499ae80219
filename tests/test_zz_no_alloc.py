"""gs_bin_and_sort_async_noalloc (the binning call that allocates nothing,
its workspace a fixed array inside the library) against
gs_bin_and_sort_async_ex with a caller-owned workspace, both called through
the C ABI on the same preprocessed splats: the entry count, the sorted keys
and the point list must be identical bit for bit. Two calls in a row, the
second on a smaller scene (and with the ellipse tile test), so the second
starts on a workspace that still holds the first call's contents; an
oversized request is refused before anything is enqueued."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def _splats(name, tile_test):
    import torch
    import gaussian_splatting_tile_amd as gs
    scene, cam, _ = synth.config_scene(name)
    sc = gs.Scene.from_numpy(scene)
    pre = gs.preprocess(cam, sc.means, sc.scales, sc.quats, sc.opacity, sc.sh, sc.sh_degree, sc.rgb,
                        tile_test=tile_test)
    torch.cuda.synchronize()
    return cam, pre


def _bin(cam, pre, capacity, tile_test, noalloc, fill):
    """One binning through the C ABI; returns (E, keys[:E], values[:E])."""
    import torch
    import gaussian_splatting_tile_amd as gs
    from gaussian_splatting_tile_amd import _lib
    lib = _lib.load()
    dev = pre["xy_depth"].device
    c = gs.camera(cam)
    n = int(pre["tiles_touched"].shape[0])
    keys = torch.full((capacity,), fill, dtype=torch.int64, device=dev)
    vals = torch.full((capacity,), fill & 0x7FFFFFFF, dtype=torch.int32, device=dev)
    n_dev = torch.full((1,), -1, dtype=torch.int64, device=dev)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    if noalloc:
        rc = lib.gs_bin_and_sort_async_noalloc(ctypes.byref(c), n, P(pre["xy_depth"]), P(pre["conic_op"]),
                                               P(pre["tiles_touched"]), P(keys), P(vals), capacity, P(n_dev),
                                               tile_test, st)
    else:
        nbytes = ctypes.c_size_t(0)
        assert lib.gs_bin_and_sort_async_ex(ctypes.byref(c), n, None, None, None, None, None, capacity, None,
                                            ctypes.byref(nbytes), None, tile_test, None) == 0
        ws = torch.empty((nbytes.value,), dtype=torch.uint8, device=dev)
        rc = lib.gs_bin_and_sort_async_ex(ctypes.byref(c), n, P(pre["xy_depth"]), P(pre["conic_op"]),
                                          P(pre["tiles_touched"]), P(keys), P(vals), capacity, P(ws),
                                          ctypes.byref(nbytes), P(n_dev), tile_test, st)
    assert rc == 0, (rc, lib.gs_last_error())
    torch.cuda.synchronize()
    E = int(n_dev.item())
    assert 0 < E <= capacity, (E, capacity)
    return E, keys[:E].cpu().numpy().view(np.uint64), vals[:E].cpu().numpy().view(np.uint32)


def _same(cam, pre, capacity, tile_test, what):
    E0, k0, v0 = _bin(cam, pre, capacity, tile_test, noalloc=False, fill=0x5A5A5A5A5A5A5A5A)
    E1, k1, v1 = _bin(cam, pre, capacity, tile_test, noalloc=True, fill=0x3C3C3C3C3C3C3C3C)
    say(f"[noalloc] {what}: E {E0} / {E1}")
    assert E1 == E0, (what, E0, E1)
    assert np.array_equal(k1, k0), f"{what}: keys differ at {np.nonzero(k1 != k0)[0][:5]}"
    assert np.array_equal(v1, v0), f"{what}: point lists differ at {np.nonzero(v1 != v0)[0][:5]}"


def test_noalloc_binning_matches_the_workspace_call():
    import torch
    assert torch.cuda.is_available()
    # first call: the 160k-Gaussian scene at 720 x 720, square spans
    cam1, pre1 = _splats("cfg1", 0)
    _same(cam1, pre1, 1_000_000, 0, "cfg1 160k 720x720 square")
    # second call, smaller: 1,000 Gaussians at 64 x 64, ellipse tile test
    cam0, pre0 = _splats("cfg0", 1)
    _same(cam0, pre0, 4096, 1, "cfg0 1k 64x64 ellipse")


def test_noalloc_binning_refuses_an_oversized_workspace():
    import torch
    import gaussian_splatting_tile_amd as gs
    from gaussian_splatting_tile_amd import _lib
    lib = _lib.load()
    cam, pre = _splats("cfg0", 0)
    dev = pre["xy_depth"].device
    keys = torch.zeros((8,), dtype=torch.int64, device=dev)
    vals = torch.zeros((8,), dtype=torch.int32, device=dev)
    n_dev = torch.full((1,), -7, dtype=torch.int64, device=dev)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    c = gs.camera(cam)
    # a capacity whose workspace exceeds the fixed array: refused, nothing enqueued
    rc = lib.gs_bin_and_sort_async_noalloc(ctypes.byref(c), 1000, P(pre["xy_depth"]), None,
                                           P(pre["tiles_touched"]), P(keys), P(vals), 1 << 30, P(n_dev), 0,
                                           None)
    assert rc == _lib.GS_ERR_INVALID
    assert b"workspace" in lib.gs_last_error()
    torch.cuda.synchronize()
    assert int(n_dev.item()) == -7
