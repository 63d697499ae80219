"""Shared helpers for the GPU parity tests: run the HIP path through the
binding and the oracle on the same seeded inputs, and compare to the bar.

Bar (per stage):
  * bit-exact: every preprocess output, tile counts, keys, sorted order,
    tile ranges and the entry count;
  * n_contrib equal on >= 99.9% of pixels;
  * image and 1 - final_T within 1e-4 absolute on pixels whose n_contrib
    matches;
  * on pixels whose n_contrib differs (a stop decision at T ~ 1e-4 taken on
    the other side of the threshold after float32 rounding of T), image
    within 1e-4 (1 + max|c| + max|bg|) and final_T within 2e-4: one side
    composited at most what is left behind T < ~1e-4 (colour at most
    T max|c|, background T max|bg|) and the other did not; and at most
    MISMATCH_PER_TILE such pixels in any one 16 x 16 tile;
  * gradients per group: max|gpu - oracle| / max|oracle| <= 1e-3, and per
    element |gpu - oracle| <= 1e-3 max(|oracle|, 1e-2 max|oracle|): every
    element at least 1% of its group's largest is held to 1e-3 of itself.
    Smaller ones are held to 1e-5 of the group's largest: a stop decision
    at T ~ 1e-4 taken on the other side of the threshold, or a chunk that
    restarts from its checkpoint, moves an element by an amount of order
    1e-4 times a term, whatever the element's size.
"""
from __future__ import annotations

import numpy as np

IMAGE_ATOL = 1e-4
NCONTRIB_FRAC = 0.999
GRAD_REL = 1e-3
T_STOP = 1e-4
MISMATCH_PER_TILE = 4
GRAD_ELEMENT_FLOOR = 1e-2


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
                             dLdI.astype(np.float32), bg=bg, mass=True)


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


def compare_forward(g, o, bg=(0.0, 0.0, 0.0)):
    """Returns a report dict; asserts the tolerance bar (see the module
    docstring), including a bound on pixels whose n_contrib differs."""
    same = g["n_contrib"] == o["n_contrib"]
    frac = float(same.mean())
    d_img = np.abs(g["image"].astype(np.float64) - o["image"])
    d_T = np.abs(g["final_T"].astype(np.float64) - o["final_T"])
    err_img = d_img[:, same]
    err_T = d_T[same]
    rgb = np.asarray(o["rgb"], np.float64)
    cmax = float(np.abs(rgb[:, :3]).max()) if rgb.size else 0.0
    bgmax = float(max(abs(float(b)) for b in bg))
    mis_img_bound = IMAGE_ATOL * (1.0 + cmax + bgmax)
    mis_T_bound = 2.0 * T_STOP
    H, W = g["final_T"].shape
    ys, xs = np.nonzero(~same)
    per_tile = np.bincount((ys // 16) * ((W + 15) // 16) + xs // 16) if ys.size else np.zeros(1, np.int64)
    rep = dict(ncontrib_match=frac, n_mismatch=int((~same).sum()),
               max_img_err=float(err_img.max()) if err_img.size else 0.0,
               max_T_err=float(err_T.max()) if err_T.size else 0.0,
               max_img_err_mismatched=float(d_img[:, ~same].max()) if (~same).any() else 0.0,
               max_T_err_mismatched=float(d_T[~same].max()) if (~same).any() else 0.0,
               max_mismatch_per_tile=int(per_tile.max()),
               mismatch_img_bound=mis_img_bound)
    assert frac >= NCONTRIB_FRAC, rep
    assert rep["max_img_err"] <= IMAGE_ATOL, rep
    assert rep["max_T_err"] <= IMAGE_ATOL, rep
    assert rep["max_img_err_mismatched"] <= mis_img_bound, rep
    assert rep["max_T_err_mismatched"] <= mis_T_bound, rep
    assert rep["max_mismatch_per_tile"] <= MISMATCH_PER_TILE, rep
    _report("fwd", rep)
    return rep


def _report(kind, rep):
    """Appends a parity report line to $GS_PARITY_REPORT when it is set."""
    import json
    import os
    path = os.environ.get("GS_PARITY_REPORT")
    if path:
        test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
        with open(path, "a") as f:
            f.write(json.dumps(dict(kind=kind, test=test, **rep)) + "\n")


GROUPS = (("grad_mean2d", slice(0, 2), "mean2d"), ("grad_conic_op", slice(0, 3), "conic"),
          ("grad_conic_op", slice(3, 4), "opacity"), ("grad_rgb", slice(0, 3), "rgb"))


def compare_gradients(g, o, rel=GRAD_REL):
    rep = {}
    stats = {}
    for key, cols, name in GROUPS:
        ref = o[key][:, cols]
        got = g[key][:, cols]
        scale = np.abs(ref).max()
        d = np.abs(got - ref)
        err = d.max()
        rep[name] = (float(err), float(scale))
        # per element: the error against the element itself, with floors
        # relative to the group maximum and (if the oracle gave it) to the
        # element's own term magnitudes
        st = {}
        aref = np.abs(ref)
        for f in (1e-1, 1e-2, 1e-3, 1e-4):
            st[f"gmax_{f:g}"] = float((d / np.maximum(aref, f * max(scale, 1e-30))).max()) if d.size else 0.0
        mkey = key.replace("grad_", "mass_")
        if mkey in o:
            m = o[mkey][:, cols]
            for f in (1e-1, 1e-2, 1e-3):
                st[f"mass_{f:g}"] = float((d / np.maximum(np.maximum(aref, f * m), 1e-30)).max()) if d.size else 0.0
        stats[name] = st
        assert err <= rel * max(scale, 1e-30), (name, err, scale, rep)
        per_el = st[f"gmax_{GRAD_ELEMENT_FLOOR:g}"]
        assert per_el <= rel, (name, "per element", per_el, rep)
    assert not g["grad_rgb"][:, 3].any()
    _report("grad", dict(groups=rep, per_element=stats))
    return rep
