"""Pins for the oracle's backward compositing.

The fp64 backward is checked against central finite differences of the fp64
forward (loss L = sum(dL/dI * image)) on tiny scenes where no skip, clamp or
termination decision changes within +-h; the fp32 backward against the fp64
one; and two special cases in closed form.
"""
import math

import numpy as np
import pytest

import synth

PARAMS = ["u", "v", "A", "B", "C", "o", "r", "g", "b"]


def tiny_case(orc, seed, n=6, W=32, H=32, op_hi=0.95):
    cam = synth.look_at_camera((0.05, 0.1, -4.0), (0.0, 0.0, 0.0), W, H, 36.0, 36.0, W / 2, H / 2)
    scene = synth.random_scene(n, seed, cam, scale_lo=0.1, scale_hi=0.35, op_lo=0.3, op_hi=op_hi,
                               spread=0.7, depth_lo=2.0, depth_hi=5.0)
    pre = orc.preprocess(cam, scene)
    keys, pl = orc.bin_and_sort(cam, pre["xy_depth"], pre["tiles_touched"])
    ranges = orc.tile_ranges(cam, keys)
    dLdI = synth.upstream_gradient(seed + 100, W, H).astype(np.float64)
    return cam, n, pre, pl, ranges, dLdI


def fwd64(orc, cam, pre, pl, ranges, xy, co, rgb, bg=(0.0, 0.0, 0.0)):
    return orc.composite_fwd(cam, ranges, pl, xy, co, rgb, bg, dtype=np.float64)


def loss(out, dLdI):
    return float((out["image"] * dLdI).sum())


def param_view(xy, co, rgb, name):
    return {"u": (xy, 0), "v": (xy, 1), "A": (co, 0), "B": (co, 1), "C": (co, 2), "o": (co, 3),
            "r": (rgb, 0), "g": (rgb, 1), "b": (rgb, 2)}[name]


def grad_of(g, name, i):
    return {"u": g["grad_mean2d"][i, 0], "v": g["grad_mean2d"][i, 1], "A": g["grad_conic_op"][i, 0],
            "B": g["grad_conic_op"][i, 1], "C": g["grad_conic_op"][i, 2], "o": g["grad_conic_op"][i, 3],
            "r": g["grad_rgb"][i, 0], "g": g["grad_rgb"][i, 1], "b": g["grad_rgb"][i, 2]}[name]


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_fp64_backward_matches_finite_differences(orc, seed):
    cam, n, pre, pl, ranges, dLdI = tiny_case(orc, seed)
    xy = pre["xy_depth"].astype(np.float64)
    co = pre["conic_op"].astype(np.float64)
    rgb = pre["rgb"].astype(np.float64)
    base = fwd64(orc, cam, pre, pl, ranges, xy, co, rgb)
    assert base["n_contrib"].sum() > 0
    g = orc.composite_bwd(cam, n, ranges, pl, xy, co, rgb, base["final_T"], base["n_contrib"], dLdI,
                          dtype=np.float64)
    checked = 0
    for i in range(n):
        if pre["tiles_touched"][i] == 0:
            continue
        for name in PARAMS:
            arr, k = param_view(xy, co, rgb, name)
            x0 = arr[i, k]
            ests = []
            for h in (1e-6 * max(1.0, abs(x0)), 0.25e-6 * max(1.0, abs(x0))):
                arr[i, k] = x0 + h
                fp = fwd64(orc, cam, pre, pl, ranges, xy, co, rgb)
                arr[i, k] = x0 - h
                fm = fwd64(orc, cam, pre, pl, ranges, xy, co, rgb)
                arr[i, k] = x0
                same = ((fp["n_contrib"] == base["n_contrib"]).all()
                        and (fm["n_contrib"] == base["n_contrib"]).all())
                ests.append((loss(fp, dLdI) - loss(fm, dLdI)) / (2 * h) if same else None)
            if None in ests or abs(ests[0] - ests[1]) > 1e-4 * max(1.0, abs(ests[0])):
                continue  # a decision flips within +-h; not a smooth point
            want = ests[1]
            got = grad_of(g, name, i)
            assert abs(got - want) <= 1e-5 * max(1.0, abs(want)), (i, name, got, want)
            checked += 1
    assert checked >= 20


@pytest.mark.parametrize("seed", [4, 5])
def test_fp32_backward_close_to_fp64(orc, seed):
    cam, n, pre, pl, ranges, dLdI = tiny_case(orc, seed, n=8)
    f32 = orc.composite_fwd(cam, ranges, pl, pre["xy_depth"], pre["conic_op"], pre["rgb"])
    f64 = orc.composite_fwd(cam, ranges, pl, pre["xy_depth"], pre["conic_op"], pre["rgb"], dtype=np.float64)
    assert (f32["n_contrib"] == f64["n_contrib"]).all()
    g32 = orc.composite_bwd(cam, n, ranges, pl, pre["xy_depth"], pre["conic_op"], pre["rgb"],
                            f32["final_T"], f32["n_contrib"], dLdI.astype(np.float32))
    g64 = orc.composite_bwd(cam, n, ranges, pl, pre["xy_depth"], pre["conic_op"], pre["rgb"],
                            f64["final_T"], f64["n_contrib"], dLdI, dtype=np.float64)
    for key in ("grad_mean2d", "grad_conic_op", "grad_rgb"):
        ref = g64[key]
        assert np.abs(g32[key] - ref).max() <= 1e-5 * max(1e-12, np.abs(ref).max())


def test_single_gaussian_colour_gradient(orc):
    """One splat, T = 1 in front of it: dL/dc = sum_pixels alpha_p g_p."""
    cam = synth.look_at_camera((0.0, 0.0, -4.0), (0.0, 0.0, 0.0), 32, 32, 32.0, 32.0, 16.0, 16.0)
    xy = np.array([[15.3, 16.6, 4.0, 9.0]], np.float64)
    co = np.array([[0.2, 0.05, 0.15, 0.8]], np.float64)
    rgb = np.array([[0.3, 0.6, 0.9, 0.0]], np.float64)
    tt = np.array([4], np.uint32)
    keys, pl = orc.bin_and_sort(cam, xy.astype(np.float32), tt)
    ranges = orc.tile_ranges(cam, keys)
    f = orc.composite_fwd(cam, ranges, pl, xy, co, rgb, dtype=np.float64)
    dLdI = synth.upstream_gradient(9, 32, 32).astype(np.float64)
    g = orc.composite_bwd(cam, 1, ranges, pl, xy, co, rgb, f["final_T"], f["n_contrib"], dLdI,
                          dtype=np.float64)
    ys, xs = np.mgrid[0:32, 0:32]
    dx, dy = xs - 15.3, ys - 16.6
    alpha = np.minimum(0.99, 0.8 * np.exp(-0.5 * (0.2 * dx * dx + 0.15 * dy * dy) - 0.05 * dx * dy))
    alpha = np.where(alpha >= 1 / 255, alpha, 0.0)
    for ch in range(3):
        np.testing.assert_allclose(g["grad_rgb"][0, ch], (alpha * dLdI[ch]).sum(), rtol=1e-12)


def test_saturated_splat_has_no_geometry_gradient(orc):
    """At the centre pixel o G = 1 > 0.99: that pixel sends nothing to o, the
    conic or the mean; its colour gradient is 0.99 g (T = 1 in front)."""
    cam = synth.look_at_camera((0.0, 0.0, -4.0), (0.0, 0.0, 0.0), 32, 32, 32.0, 32.0, 16.0, 16.0)
    xy = np.array([[16.0, 16.0, 4.0, 4.0]], np.float64)
    co = np.array([[1.0, 0.0, 1.0, 1.0]], np.float64)
    rgb = np.array([[0.3, 0.6, 0.9, 0.0]], np.float64)
    keys, pl = orc.bin_and_sort(cam, xy.astype(np.float32), np.array([4], np.uint32))
    ranges = orc.tile_ranges(cam, keys)
    f = orc.composite_fwd(cam, ranges, pl, xy, co, rgb, dtype=np.float64)
    dLdI = np.zeros((3, 32, 32))
    dLdI[:, 16, 16] = [1.0, -2.0, 0.5]
    g = orc.composite_bwd(cam, 1, ranges, pl, xy, co, rgb, f["final_T"], f["n_contrib"], dLdI,
                          dtype=np.float64)
    assert not g["grad_conic_op"].any() and not g["grad_mean2d"].any()
    amax = float(np.float32(0.99))  # the clamp constant is the fp32 0.99 in both precisions
    np.testing.assert_allclose(g["grad_rgb"][0, :3], [amax, -2 * amax, 0.5 * amax], rtol=1e-12)
    # a neighbouring pixel is unsaturated and does send gradient to o
    dLdI2 = np.zeros((3, 32, 32))
    dLdI2[:, 16, 17] = 1.0
    g2 = orc.composite_bwd(cam, 1, ranges, pl, xy, co, rgb, f["final_T"], f["n_contrib"], dLdI2,
                           dtype=np.float64)
    G = math.exp(-0.5)
    np.testing.assert_allclose(g2["grad_conic_op"][0, 3], G * (0.3 + 0.6 + 0.9), rtol=1e-12)
