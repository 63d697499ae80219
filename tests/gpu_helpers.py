"""Shared helpers for the GPU parity tests: run the HIP path through the
binding and the oracle on the same seeded inputs, and compare to the bar.

Bar (per stage):
  * bit-exact: every preprocess output, tile counts, keys, sorted order,
    tile ranges and the entry count;
  * n_contrib equal on >= 99.9% of pixels;
  * image and 1 - final_T within 1e-4 absolute on pixels whose n_contrib
    matches;
  * gradients per group: max|gpu - oracle| / max|oracle| <= 1e-3.
"""
from __future__ import annotations

import numpy as np

IMAGE_ATOL = 1e-4
NCONTRIB_FRAC = 0.999
GRAD_REL = 1e-3


def to_np(t):
    return t.detach().cpu().numpy()


def gpu_forward(cam, scene_np, bg=(0.0, 0.0, 0.0), capacity=1 << 16, rast=None, scheduled=None):
    """Rasterizer.forward; scheduled None leaves the choice of the scheduled
    (chunked) forward to the Rasterizer (small tile grids)."""
    import gaussian_splatting_tile_amd as gs
    import torch
    sc = gs.Scene.from_numpy(scene_np)
    r = rast or gs.Rasterizer(capacity=capacity)
    out = r.forward(cam, sc, bg=bg, with_examined=True, scheduled=scheduled)
    torch.cuda.synchronize()
    res = {k: to_np(v) for k, v in out.items() if hasattr(v, "detach") and k not in ("ckpt", "chunks")}
    res["n_entries"] = out["n_entries"]
    res["keys"] = res["keys"].view(np.uint64)
    for k in ("point_list", "ranges", "tiles_touched", "n_contrib", "n_examined"):
        res[k] = res[k].view(np.uint32)
    return res, out, sc, r


def gpu_backward(cam, sc, out, dLdI, bg=(0.0, 0.0, 0.0), final_T=None, n_contrib=None, chunked=False):
    """gs_composite_bwd on the forward's state (or the given final_T and
    n_contrib); with chunked, gs_composite_bwd_ex on the forward's checkpoints."""
    import gaussian_splatting_tile_amd as gs
    import torch
    dev = out["xy_depth"].device
    if chunked:
        assert final_T is None and n_contrib is None, "chunks start from the forward's own state"
    fT = out["final_T"] if final_T is None else torch.from_numpy(np.ascontiguousarray(final_T)).to(dev)
    nc = out["n_contrib"] if n_contrib is None else torch.from_numpy(
        np.ascontiguousarray(n_contrib).view(np.int32)).to(dev)
    g = torch.from_numpy(np.ascontiguousarray(dLdI, np.float32)).to(dev)
    grads = gs.composite_bwd(cam, sc.n, out["ranges"], out["point_list"], out["xy_depth"], out["conic_op"],
                             out["rgb"], fT, nc, g, bg, chunks=out["chunks"] if chunked else None,
                             image=out["image"] if chunked else None, ckpt=out["ckpt"] if chunked else None,
                             capacity=out["n_entries"])
    torch.cuda.synchronize()
    return {k: to_np(v).astype(np.float64) for k, v in grads.items()}


def oracle_forward(orc, cam, scene_np, bg=(0.0, 0.0, 0.0)):
    return orc.render_fwd(cam, scene_np, bg=bg)


def oracle_backward(orc, cam, scene_np, ofwd, dLdI, bg=(0.0, 0.0, 0.0)):
    return orc.composite_bwd(cam, scene_np["n"], ofwd["ranges"], ofwd["point_list"], ofwd["xy_depth"],
                             ofwd["conic_op"], ofwd["rgb"], ofwd["final_T"], ofwd["n_contrib"],
                             dLdI.astype(np.float32), bg=bg)


def assert_bits_equal(a, b, what):
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    if a.dtype.kind == "f":
        a = a.view(np.uint32 if a.dtype.itemsize == 4 else np.uint64)
        b = b.view(a.dtype)
    bad = np.nonzero(a.reshape(-1) != b.reshape(-1))[0]
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at flat index {bad[:5].tolist()}"


def assert_preprocess_equal(g, o):
    for k in ("xy_depth", "conic_op", "rgb", "tiles_touched"):
        assert_bits_equal(g[k], o[k], k)


def assert_binning_equal(g, o):
    assert g["n_entries"] == o["keys"].shape[0], (g["n_entries"], o["keys"].shape[0])
    assert_bits_equal(g["keys"], o["keys"], "keys")
    assert_bits_equal(g["point_list"], o["point_list"], "point_list")
    assert_bits_equal(g["ranges"], o["ranges"], "ranges")


def compare_forward(g, o):
    """Returns a report dict; asserts the tolerance bar."""
    same = g["n_contrib"] == o["n_contrib"]
    frac = float(same.mean())
    err_img = np.abs(g["image"] - o["image"])[:, same]
    err_T = np.abs(g["final_T"] - o["final_T"])[same]
    rep = dict(ncontrib_match=frac, n_mismatch=int((~same).sum()),
               max_img_err=float(err_img.max()) if err_img.size else 0.0,
               max_T_err=float(err_T.max()) if err_T.size else 0.0,
               max_img_err_mismatched=float(np.abs(g["image"] - o["image"])[:, ~same].max()) if (~same).any() else 0.0)
    assert frac >= NCONTRIB_FRAC, rep
    assert rep["max_img_err"] <= IMAGE_ATOL, rep
    assert rep["max_T_err"] <= IMAGE_ATOL, rep
    return rep


def compare_gradients(g, o, rel=GRAD_REL):
    rep = {}
    for key, cols, name in (("grad_mean2d", slice(0, 2), "mean2d"), ("grad_conic_op", slice(0, 3), "conic"),
                            ("grad_conic_op", slice(3, 4), "opacity"), ("grad_rgb", slice(0, 3), "rgb")):
        ref = o[key][:, cols]
        got = g[key][:, cols]
        scale = np.abs(ref).max()
        err = np.abs(got - ref).max()
        rep[name] = (float(err), float(scale))
        assert err <= rel * max(scale, 1e-30), (name, err, scale, rep)
    assert not g["grad_rgb"][:, 3].any()
    return rep
