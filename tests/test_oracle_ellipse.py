"""Pins for the oracle's ellipse tile test (zenn 2.3.4: of the span's tiles,
keep those the splat's ellipse may overlap; reading: the region where the
splat can reach alpha >= 1/255, with the opacity-independent threshold
11.1 > 2 ln 255 plus a rounding bound).

What the reading fixes, checked here against the square-span method and
brute force rather than against the formula itself:
  * the image, final_T and every gradient are bit-identical to the
    square-span method (a dropped tile holds no pixel the splat changes);
  * each tile's list is a subsequence of its square-span list, and every
    dropped (splat, tile) pair has alpha < 1/255 at all 256 pixels;
  * the kept set contains every (splat, tile) pair with a pixel inside the
    exact ellipse Q <= 2 ln 255 and is at most a few percent larger;
  * rows keep contiguous runs inside the span; E = sum of tiles_touched.
"""
import numpy as np
import pytest

import synth

LN255x2 = 2.0 * np.log(255.0)


def _scene(seed, W=257, H=129, n=2500, deg=None):
    cam = synth.look_at_camera((0.2, -0.1, -4.0), (0.0, 0.0, 0.0), W, H, 150.0, 160.0)
    scene = synth.random_scene(n, seed, cam, sh_degree=deg, scale_lo=0.005, scale_hi=0.25, op_lo=0.02,
                               op_hi=0.99, spread=1.3, depth_lo=1.0, depth_hi=7.0)
    return cam, scene


def _both(orc, cam, scene, bg=(0.0, 0.0, 0.0)):
    a = orc.render_fwd(cam, scene, bg=bg, tile_test=0)
    b = orc.render_fwd(cam, scene, bg=bg, tile_test=1)
    return a, b


CASES = [("cfg0", None), ("rand", 0), ("rand", 1), ("rand", 2)]


def _case(name, seed):
    if name == "cfg0":
        scene, cam, _ = synth.config_scene("cfg0")
        return cam, scene
    return _scene(seed, deg=seed if seed < 4 else None)


@pytest.mark.parametrize("name,seed", CASES)
def test_image_and_gradients_unchanged(orc, name, seed):
    cam, scene = _case(name, seed)
    bg = (0.2, 0.5, 0.9)
    a, b = _both(orc, cam, scene, bg)
    assert b["keys"].size < a["keys"].size  # the test drops entries
    for k in ("image", "final_T"):
        assert a[k].tobytes() == b[k].tobytes(), k
    # the preprocess records of the Gaussians both keep are the same
    keep = b["tiles_touched"] > 0
    assert np.array_equal(a["xy_depth"][keep], b["xy_depth"][keep])
    # dropped Gaussians: nothing kept means no pixel reaches 1/255
    assert ((a["tiles_touched"] > 0) | ~keep).all()
    dL = synth.upstream_gradient(5 + (seed or 0), cam["width"], cam["height"])
    n = scene["n"]
    ga = orc.composite_bwd(cam, n, a["ranges"], a["point_list"], a["xy_depth"], a["conic_op"], a["rgb"],
                           a["final_T"], a["n_contrib"], dL, bg)
    gb = orc.composite_bwd(cam, n, b["ranges"], b["point_list"], b["xy_depth"], b["conic_op"], b["rgb"],
                           b["final_T"], b["n_contrib"], dL, bg)
    for k in ga:
        assert np.array_equal(ga[k], gb[k]), k


def _pairs(o):
    """(tile, gaussian) pairs of a binned frame, as a set."""
    t = (o["keys"] >> np.uint64(32)).astype(np.int64)
    return set(zip(t.tolist(), o["point_list"].astype(np.int64).tolist()))


@pytest.mark.parametrize("name,seed", CASES[:3])
def test_lists_are_subsequences_and_dropped_pairs_are_invisible(orc, name, seed):
    cam, scene = _case(name, seed)
    a, b = _both(orc, cam, scene)
    W, H = cam["width"], cam["height"]
    TX = (W + 15) // 16
    # subsequence per tile
    for t in range(a["ranges"].shape[0]):
        la = a["point_list"][a["ranges"][t, 0]:a["ranges"][t, 1]]
        lb = b["point_list"][b["ranges"][t, 0]:b["ranges"][t, 1]]
        it = iter(la.tolist())
        assert all(g in it for g in lb.tolist()), t
    dropped = _pairs(a) - _pairs(b)
    assert dropped
    xy, co = a["xy_depth"], a["conic_op"]
    ys, xs = np.mgrid[0:16, 0:16]
    for t, g in dropped:
        tx, ty = t % TX, t // TX
        dx = (xs + 16 * tx).astype(np.float32) - xy[g, 0]
        dy = (ys + 16 * ty).astype(np.float32) - xy[g, 1]
        A, B, C, o = (np.float32(v) for v in co[g])
        power = np.float32(-0.5) * ((A * dx) * dx + (C * dy) * dy) - (B * dx) * dy
        alpha = np.minimum(np.float32(0.99), o * np.exp(power.astype(np.float64)).astype(np.float32))
        inside = ((xs + 16 * tx) < W) & ((ys + 16 * ty) < H)
        assert (alpha[inside] < np.float32(1.0 / 255.0)).all(), (t, g)


def test_kept_set_is_tight(orc):
    """Kept pairs contain every pair with a pixel inside the exact ellipse
    Q <= 2 ln 255 and exceed that set by only a few percent."""
    cam, scene = _scene(7, n=4000)
    a, b = _both(orc, cam, scene)
    W, H = cam["width"], cam["height"]
    TX = (W + 15) // 16
    xy, co = a["xy_depth"].astype(np.float64), a["conic_op"].astype(np.float64)
    ys, xs = np.mgrid[0:16, 0:16]
    exact = set()
    for t, g in _pairs(a):
        tx, ty = t % TX, t // TX
        dx = xs + 16 * tx - xy[g, 0]
        dy = ys + 16 * ty - xy[g, 1]
        A, B, C = co[g, :3]
        q = A * dx * dx + 2 * B * dx * dy + C * dy * dy
        if (q <= LN255x2).any():
            exact.add((t, g))
    kept = _pairs(b)
    assert exact <= kept
    assert len(kept) <= 1.08 * len(exact), (len(kept), len(exact))


def test_row_ranges_are_runs_inside_the_span(orc):
    rng = np.random.default_rng(3)
    TX, TY = 20, 12
    for _ in range(3000):
        u, v = rng.uniform(-40, 360), rng.uniform(-40, 230)
        a_, c_ = rng.uniform(0.3, 400.0, 2)
        b_ = rng.uniform(-1, 1) * np.sqrt(a_ * c_) * 0.999
        det = a_ * c_ - b_ * b_
        conic = (c_ / det, -b_ / det, a_ / det)
        mid = 0.5 * (a_ + c_)
        r = np.ceil(3 * np.sqrt(mid + np.sqrt(max(mid * mid - det, 0.1))))
        x0, x1, y0, y1 = orc.tile_span(u, v, r, TX, TY)
        for ty in range(y0, y1):
            lo, hi = orc.ellipse_row_range(u, v, r, conic, TX, TY, ty)
            assert hi <= lo or (x0 <= lo < hi <= x1)


def test_counts_match_entries(orc):
    cam, scene = _scene(11)
    pre = orc.preprocess(cam, scene, tile_test=1)
    keys, pl = orc.bin_and_sort(cam, pre["xy_depth"], pre["tiles_touched"], pre["conic_op"], 1)
    assert keys.size == int(pre["tiles_touched"].sum())
    with pytest.raises(ValueError):
        orc.bin_and_sort(cam, pre["xy_depth"], pre["tiles_touched"], None, 1)
