"""Pins for the oracle's forward compositing.

Expected values: closed forms for one and two Gaussians, the termination
edge, the 1 - final_T = sum(alpha_i T_i) identity, and an independent
brute-force per-pixel compositor (numpy, written here) that sorts all splats
by depth and keeps those whose tile span holds the pixel's tile.
"""
import math

import numpy as np
import pytest

import synth


def cam0():
    return synth.look_at_camera((0.0, 0.0, -4.0), (0.0, 0.0, 0.0), 64, 64, 64.0, 64.0, 32.0, 32.0)


def render(orc, cam, splats, bg=(0.0, 0.0, 0.0), dtype=np.float32):
    """splats: list of (u, v, z, r, A, B, C, o, (r, g, b)); bins and composites."""
    n = len(splats)
    xy = np.array([[s[0], s[1], s[2], s[3]] for s in splats], np.float32).reshape(n, 4)
    co = np.array([[s[4], s[5], s[6], s[7]] for s in splats], np.float32).reshape(n, 4)
    rgb = np.array([list(s[8]) + [0.0] for s in splats], np.float32).reshape(n, 4)
    TX, TY = orc.tiles_xy(cam)
    tt = np.array([(lambda sp: (sp[1] - sp[0]) * (sp[3] - sp[2]))(orc.tile_span(s[0], s[1], s[3], TX, TY))
                   for s in splats], np.uint32)
    keys, pl = orc.bin_and_sort(cam, xy, tt)
    ranges = orc.tile_ranges(cam, keys)
    out = orc.composite_fwd(cam, ranges, pl, xy, co, rgb, bg, dtype=dtype)
    out.update(ranges=ranges, point_list=pl, xy=xy, co=co, rgb=rgb)
    return out


def test_single_gaussian_closed_form(orc):
    """Isotropic splat at (32, 32), a = 0.94, o = 0.9: alpha = 0.9 exp(-|d|^2 / (2a))."""
    cam = cam0()
    a = 0.94
    out = render(orc, cam, [(32.0, 32.0, 4.0, 4.0, 1 / a, 0.0, 1 / a, 0.9, (1.0, 0.5, 0.25))])
    for (x, y), d2 in [((32, 32), 0), ((33, 32), 1), ((33, 33), 2), ((34, 32), 4), ((35, 32), 9), ((32, 29), 9)]:
        alpha = min(0.99, 0.9 * math.exp(-d2 / (2 * a)))
        assert alpha >= 1 / 255
        np.testing.assert_allclose(out["image"][:, y, x], np.array([1.0, 0.5, 0.25]) * alpha, rtol=2e-6)
        np.testing.assert_allclose(out["final_T"][y, x], 1 - alpha, rtol=2e-6)
        assert out["n_contrib"][y, x] == 1
    # the page-style alpha table for |d|^2 = 0, 1, 2, 4, 9
    got = [float(out["image"][0, y, x]) for (x, y) in [(32, 32), (33, 32), (33, 33), (34, 32), (35, 32)]]
    np.testing.assert_allclose(got, [0.9 * math.exp(-d / (2 * a)) for d in (0, 1, 2, 4, 9)], rtol=2e-6)
    # below the alpha floor: skipped, examined but not a contributor
    assert out["n_contrib"][32, 37] == 0 and out["image"][0, 32, 37] == 0 and out["final_T"][32, 37] == 1
    assert out["n_examined"][32, 37] == 1
    # outside the tile span (tiles 1..2 in x and y): never examined
    assert out["n_examined"][5, 5] == 0 and out["final_T"][5, 5] == 1


def test_saturation_clamp(orc):
    cam = cam0()
    out = render(orc, cam, [(32.0, 32.0, 4.0, 4.0, 1.0, 0.0, 1.0, 1.0, (1.0, 1.0, 1.0))])
    np.testing.assert_allclose(out["final_T"][32, 32], 1 - np.float32(0.99), rtol=1e-7)


def test_two_coincident_gaussians_order(orc):
    cam = cam0()
    base = (32.0, 32.0)
    s1 = base + (2.0, 4.0, 1.0, 0.0, 1.0, 0.6, (1.0, 0.0, 0.0))
    s2 = base + (3.0, 4.0, 1.0, 0.0, 1.0, 0.5, (0.0, 1.0, 0.0))
    out = render(orc, cam, [s1, s2])
    x, y = 33, 32
    g = math.exp(-0.5)
    a1, a2 = 0.6 * g, 0.5 * g
    np.testing.assert_allclose(out["image"][:, y, x], [a1, a2 * (1 - a1), 0.0], rtol=3e-6, atol=1e-7)
    np.testing.assert_allclose(out["final_T"][y, x], (1 - a1) * (1 - a2), rtol=3e-6)
    # swapping depths swaps the roles
    s1b = s1[:2] + (3.0,) + s1[3:]
    s2b = s2[:2] + (2.0,) + s2[3:]
    out2 = render(orc, cam, [s1b, s2b])
    np.testing.assert_allclose(out2["image"][:, y, x], [a1 * (1 - a2), a2, 0.0], rtol=3e-6, atol=1e-7)
    # equal depth: index order decides (stable sort)
    s2c = s2[:2] + (2.0,) + s2[3:]
    out3 = render(orc, cam, [s1, s2c])
    np.testing.assert_allclose(out3["image"][:, y, x], [a1, a2 * (1 - a1), 0.0], rtol=3e-6, atol=1e-7)


def test_termination_edge(orc):
    """Two saturated splats leave T = (1 - 0.99f)^2 < 1e-4 in fp32: the pixel
    stops after the second (composited, then tested), the third is unseen."""
    cam = cam0()
    sat = [(32.0, 32.0, z, 4.0, 1.0, 0.0, 1.0, 1.0, (0.5, 0.5, 0.5)) for z in (1.0, 2.0)]
    third = (32.0, 32.0, 3.0, 4.0, 1.0, 0.0, 1.0, 1.0, (1.0, 0.0, 0.0))
    out = render(orc, cam, sat + [third])
    T = (np.float32(1) - np.float32(0.99)) ** 2
    assert T < np.float32(1e-4)
    assert out["n_contrib"][32, 32] == 2 and out["n_examined"][32, 32] == 2
    assert out["final_T"][32, 32] == np.float32(T)
    assert out["image"][0, 32, 32] == out["image"][1, 32, 32]  # no red from the third


def test_alpha_sum_identity(orc):
    """With white splats and black background the image is sum(alpha_i T_i) = 1 - final_T."""
    scene, cam, _ = synth.config_scene("cfg0")
    scene = dict(scene)
    scene["rgb"] = np.ones_like(scene["rgb"])
    out = orc.render_fwd(cam, scene)
    for ch in range(3):
        np.testing.assert_allclose(out["image"][ch], 1.0 - out["final_T"], atol=2e-6)


def test_background(orc):
    scene, cam, _ = synth.config_scene("cfg0")
    bg = (0.25, 0.5, 1.0)
    a = orc.render_fwd(cam, scene)
    b = orc.render_fwd(cam, scene, bg=bg)
    for ch in range(3):
        np.testing.assert_allclose(b["image"][ch], a["image"][ch] + a["final_T"] * bg[ch], atol=1e-6)
    np.testing.assert_array_equal(a["n_contrib"], b["n_contrib"])


def brute_force(cam, xy, co, rgb, bg=(0.0, 0.0, 0.0)):
    """Per pixel: every splat whose tile span holds the pixel's tile, sorted by
    (depth, index), composited front to back (float32 numpy arithmetic)."""
    W, H = cam["width"], cam["height"]
    f = np.float32
    order = np.lexsort((np.arange(len(xy)), xy[:, 2]))
    img = np.zeros((3, H, W), np.float32)
    Tm = np.ones((H, W), np.float32)
    nc = np.zeros((H, W), np.int64)
    for y in range(H):
        for x in range(W):
            tx, ty = x // 16, y // 16
            T, C, last, j = f(1), np.zeros(3, np.float32), 0, 0
            for g in order:
                u, v, z, r = xy[g]
                if r == 0:
                    continue
                if not (tx * 16 <= u + r and (tx + 1) * 16 > u - r and ty * 16 <= v + r and (ty + 1) * 16 > v - r):
                    continue
                j += 1
                dx, dy = f(x) - u, f(y) - v
                A, B, Cc, o = co[g]
                power = f(-0.5) * ((A * dx) * dx + (Cc * dy) * dy) - (B * dx) * dy
                alpha = min(f(0.99), o * np.exp(power, dtype=np.float32))
                if alpha < f(1.0) / f(255.0):
                    continue
                C = C + rgb[g, :3] * (alpha * T)
                T = T * (f(1) - alpha)
                last = j
                if T < f(1e-4):
                    break
            img[:, y, x] = C + T * np.asarray(bg, np.float32)
            Tm[y, x] = T
            nc[y, x] = last
    return img, Tm, nc


@pytest.mark.parametrize("seed", [0, 1])
def test_matches_brute_force(orc, seed):
    cam = synth.look_at_camera((0.1, -0.2, -4.0), (0.0, 0.0, 0.0), 40, 36, 40.0, 40.0, 20.0, 18.0)
    scene = synth.random_scene(60, seed, cam, scale_lo=0.02, scale_hi=0.25, op_lo=0.2, op_hi=1.0)
    out = orc.render_fwd(cam, scene, bg=(0.1, 0.2, 0.3))
    img, T, nc = brute_force(cam, out["xy_depth"], out["conic_op"], out["rgb"], bg=(0.1, 0.2, 0.3))
    assert (out["n_contrib"] == nc).mean() >= 0.99
    same = out["n_contrib"] == nc
    np.testing.assert_allclose(out["image"][:, same], img[:, same], atol=2e-6)
    np.testing.assert_allclose(out["final_T"][same], T[same], atol=2e-6)


def test_threaded_oracle_matches_single_threaded(orc):
    """The oracle's multi-threaded run (used to time it on all host cores)
    gives the single-threaded preprocess, binning and forward outputs bit for
    bit (independent Gaussians and pixel rows), and the backward to double
    rounding (per-thread partial sums added in thread order)."""
    import synth
    cam = synth.look_at_camera((0.3, -0.2, -4.0), (0.0, 0.0, 0.0), 257, 129, 150.0, 150.0)
    scene = synth.random_scene(3000, 17, cam, sh_degree=2, spread=1.3)
    dLdI = synth.upstream_gradient(9, 257, 129)
    bg = (0.1, 0.2, 0.3)
    outs = {}
    try:
        for threads in (1, 5):
            assert orc.set_threads(threads) == threads
            f = orc.render_fwd(cam, scene, bg=bg)
            b = orc.composite_bwd(cam, scene["n"], f["ranges"], f["point_list"], f["xy_depth"], f["conic_op"],
                                  f["rgb"], f["final_T"], f["n_contrib"], dLdI, bg=bg, mass=True)
            outs[threads] = (f, b)
    finally:
        orc.set_threads(1)
    (f1, b1), (f5, b5) = outs[1], outs[5]
    assert f1["keys"].size > 10000
    for k in ("xy_depth", "conic_op", "rgb", "tiles_touched", "keys", "point_list", "ranges", "image", "final_T",
              "n_contrib", "n_examined"):
        assert np.array_equal(np.asarray(f1[k]).view(np.uint8), np.asarray(f5[k]).view(np.uint8)), k
    for k in b1:
        ref = b1[k]
        assert np.abs(b5[k] - ref).max() <= 1e-12 * max(np.abs(ref).max(), 1e-300), k


def test_alpha_is_the_rounded_double_exponential(orc):
    """Reading R31 of the compositing exponential: G is exp of the float32
    power evaluated in double and rounded once to float32. One splat over a
    16 x 16 tile, 200 random conics and opacities (at the 1/255 floor,
    ordinary, and saturating at 0.99): every pixel's final T is 1 - alpha
    bit for bit, or 1 where alpha is below the floor. A float32 exponential
    (numpy's) differs from this on about 3% of the pixels."""
    import math
    f = np.float32
    cam = synth.look_at_camera((0, 0, -4), (0, 0, 0), 16, 16, 16.0, 16.0)
    rng = np.random.default_rng(3)
    ys, xs = np.mgrid[0:16, 0:16]
    differs_f32 = 0
    for _ in range(200):
        u, v = rng.uniform(-2.0, 18.0, 2).astype(np.float32)
        A, C = np.exp(rng.uniform(np.log(0.01), np.log(3.0), 2)).astype(np.float32)
        B = f(rng.uniform(-0.9, 0.9) * math.sqrt(float(A) * float(C)))
        o = f(rng.choice([rng.uniform(0.003, 0.01), rng.uniform(0.05, 0.99), 1.0]))
        out = orc.composite_fwd(cam, np.array([[0, 1]], np.uint32), np.array([0], np.uint32),
                                np.array([[u, v, 5.0, 20.0]], np.float32), np.array([[A, B, C, o]], np.float32),
                                np.array([[0.5, 0.5, 0.5, 0.0]], np.float32))
        dx = (xs.astype(np.float32) - u).astype(np.float32)
        dy = (ys.astype(np.float32) - v).astype(np.float32)
        power = (f(-0.5) * ((A * dx) * dx + (C * dy) * dy) - (B * dx) * dy).astype(np.float32)
        G = np.array([np.float32(math.exp(float(p))) for p in power.ravel()], np.float32).reshape(16, 16)
        alpha = np.minimum(f(0.99), o * G).astype(np.float32)
        expect = np.where(alpha < f(1) / f(255), f(1), f(1) - alpha).astype(np.float32)
        np.testing.assert_array_equal(out["final_T"].view(np.uint32), expect.view(np.uint32))
        a32 = np.minimum(f(0.99), o * np.exp(power)).astype(np.float32)
        t32 = np.where(a32 < f(1) / f(255), f(1), f(1) - a32).astype(np.float32)
        differs_f32 += int((t32.view(np.uint32) != expect.view(np.uint32)).sum())
    assert differs_f32 > 100  # the pin tells the two readings apart
