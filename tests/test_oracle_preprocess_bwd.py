"""Pins for the oracle's projection + SH backward (orc_preprocess_bwd).

The analytic backward is checked against central finite differences of the
float64 projection (orc_project_f64, the preprocess widened to double) for
every input of every visible Gaussian, with the frustum-clamp branch taken
on both sides of its boundary; against closed forms for an on-axis
isotropic Gaussian and for the SH coefficients; and against invariants the
mathematics fixes (the quaternion gradient is orthogonal to q, vanishes for
isotropic scales and scales as 1/k under q -> kq).
"""
import numpy as np
import pytest

import synth


def _case(seed, sh_degree, n=24, spread=1.6, W=64, H=48):
    cam = synth.look_at_camera((0.3, -0.2, -4.0), (0.0, 0.1, 0.0), W, H, 40.0, 44.0, W / 2 + 1.5,
                               H / 2 - 2.0)
    scene = synth.random_scene(n, seed, cam, sh_degree=sh_degree, scale_lo=0.05, scale_hi=0.4,
                               spread=spread, depth_lo=1.5, depth_hi=6.0)
    return cam, scene


def _upstream(seed, n):
    rng = np.random.default_rng(seed + 7)
    return rng.normal(size=(n, 2)), rng.normal(size=(n, 4)), rng.normal(size=(n, 4))


def _gaussian(scene, i):
    m = scene["means"][:, i].astype(np.float64)
    s = scene["scales"][:, i].astype(np.float64)
    q = scene["quats"][:, i].astype(np.float64)
    if scene.get("sh") is not None:
        k = (scene["sh_degree"] + 1) ** 2
        shc = np.asarray(scene["sh"]).reshape(-1, 3, scene["n"])[:k, :, i].astype(np.float64)
        return m, s, q, shc, None
    return m, s, q, None, scene["rgb"][:, i].astype(np.float64)


def _loss(orc, cam, m, s, q, shc, rgb, gm, gc, gr):
    p = orc.project_f64(cam, m, s, q, shc, rgb)
    if p is None:
        return None, None
    L = gm[0] * p["u"] + gm[1] * p["v"] + gc[0] * p["conic"][0] + gc[1] * p["conic"][1] \
        + gc[2] * p["conic"][2] + float(np.dot(gr[:3], p["rgb"]))
    return L, p["clamp"]


def _fd(orc, cam, args, which, j, gm, gc, gr, clamp):
    """Central difference with one Richardson step: (4 D(h/2) - D(h)) / 3,
    h = 1e-4 max(1, |x|) (truncation O(h^4), rounding ~ eps |L| / h)."""
    x = [a.copy() if a is not None else None for a in args]
    base = x[which].flat[j]
    h = 1e-4 * max(1.0, abs(base))
    d = []
    for step in (h, h / 2):
        vals = []
        for sign in (1, -1):
            x[which].flat[j] = base + sign * step
            L, c = _loss(orc, cam, *x, gm, gc, gr)
            if L is None or c != clamp:
                return None  # a decision flips within +-h: not a point to difference at
            vals.append(L)
        d.append((vals[0] - vals[1]) / (2 * step))
    return (4 * d[1] - d[0]) / 3


@pytest.mark.parametrize("seed,sh_degree", [(0, None), (1, 0), (2, 1), (3, 2), (4, 3), (5, 3)])
def test_backward_matches_finite_differences(orc, seed, sh_degree):
    cam, scene = _case(seed, sh_degree)
    n = scene["n"]
    gm, gc, gr = _upstream(seed, n)
    pre = orc.preprocess(cam, scene)
    g = orc.preprocess_bwd(cam, scene, gm, gc, gr)
    checked, clamped = 0, 0
    for i in range(n):
        if pre["tiles_touched"][i] == 0:
            continue
        args = list(_gaussian(scene, i))
        _, clamp = _loss(orc, cam, *args, gm[i], gc[i], gr[i])
        clamped += int(clamp[0] or clamp[1])
        groups = [("grad_means", 0, 3), ("grad_scales", 1, 3), ("grad_quats", 2, 4)]
        if args[3] is not None:
            groups.append(("grad_sh", 3, args[3].size))
        else:
            groups.append(("grad_rgb_in", 4, 3))
        for key, which, count in groups:
            fd = np.array([_fd(orc, cam, args, which, j, gm[i], gc[i], gr[i], clamp) for j in range(count)],
                          dtype=object)
            if any(v is None for v in fd):
                continue
            fd = fd.astype(np.float64)
            an = g[key][:, i]
            scale = max(np.abs(fd).max(), 1e-12)
            assert np.abs(an - fd).max() <= 1e-7 * scale + 1e-9, (key, i, an, fd)
            checked += 1
        assert g["grad_opacity"][i] == gc[i, 3]
    assert checked >= 20
    if seed >= 4:
        assert clamped >= 1, "the frustum-clamp branch was not exercised"


def test_clamp_branch_both_axes(orc):
    """Gaussians beyond 1.3x the half-width on either axis (centre off
    screen, footprint on screen): gradients still match finite differences."""
    W, H = 64, 48
    cam = synth.look_at_camera((0.0, 0.0, -4.0), (0.0, 0.0, 0.0), W, H, 40.0, 40.0)
    z = 2.0
    pts = []
    for rx, ry in [(1.36, 0.2), (-1.4, -0.1), (0.1, 1.38), (-0.2, -1.45), (1.35, 1.33)]:
        x = rx * (W / 2) / 40.0 * z
        y = ry * (H / 2) / 40.0 * z
        pts.append((x, y, z - 4.0 + 4.0))
    n = len(pts)
    rng = np.random.default_rng(11)
    means = np.array(pts, np.float64).T  # camera at -4 z looking +z: world z = p_cam z - 4
    means[2] -= 4.0
    scene = synth.scenes._pack(means.T, np.full((n, 3), 0.45), rng.normal(size=(n, 4)),
                               np.full(n, 0.8), rgb=rng.uniform(size=(n, 3)))
    gm, gc, gr = _upstream(3, n)
    pre = orc.preprocess(cam, scene)
    g = orc.preprocess_bwd(cam, scene, gm, gc, gr)
    hit = 0
    for i in range(n):
        assert pre["tiles_touched"][i] > 0
        args = list(_gaussian(scene, i))
        _, clamp = _loss(orc, cam, *args, gm[i], gc[i], gr[i])
        assert clamp[0] or clamp[1]
        for key, which, count in [("grad_means", 0, 3), ("grad_scales", 1, 3), ("grad_quats", 2, 4)]:
            fd = np.array([_fd(orc, cam, args, which, j, gm[i], gc[i], gr[i], clamp) for j in range(count)])
            scale = max(np.abs(fd).max(), 1e-12)
            assert np.abs(g[key][:, i] - fd).max() <= 1e-7 * scale + 1e-9, (key, i)
            hit += 1
    assert hit == 3 * n


def test_on_axis_isotropic_closed_form(orc):
    """Identity rotation, scale s on every axis, centre on the optical axis at
    depth z (W = I): a = c = (f s / z)^2 + 0.3, b = 0, so A = 1/a, C = 1/c and
      dL/ds_x = -gA / a^2 * 2 s f^2 / z^2,  dL/ds_y = -gC / c^2 * 2 s f^2 / z^2,
      dL/ds_z = 0;
    and with only dL/du: dL/dmean = (gu f / z, 0, 0)."""
    f, z, s = 64.0, 4.0, 0.05
    cam = dict(R=np.eye(3, dtype=np.float32).reshape(9), t=np.zeros(3, np.float32),
               campos=np.zeros(3, np.float32), fx=np.float32(f), fy=np.float32(f), cx=np.float32(32),
               cy=np.float32(32), width=64, height=64)
    scene = synth.scenes._pack(np.array([[0.0, 0.0, z]]), np.full((1, 3), s), np.array([[1.0, 0, 0, 0]]),
                               np.array([0.7]), rgb=np.array([[0.2, 0.4, 0.6]]))
    a = (f * s / z) ** 2 + 0.3
    gA, gC = 0.7, -1.3
    g = orc.preprocess_bwd(cam, scene, np.zeros((1, 2)), np.array([[gA, 0.0, gC, 0.0]]), np.zeros((1, 4)))
    k = 2 * s * f * f / (z * z)
    exp = np.array([-gA / a ** 2 * k, -gC / a ** 2 * k, 0.0])
    np.testing.assert_allclose(g["grad_scales"][:, 0], exp, rtol=1e-6, atol=1e-9)
    np.testing.assert_allclose(g["grad_quats"][:, 0], 0.0, atol=1e-9)
    gu = 0.9
    g = orc.preprocess_bwd(cam, scene, np.array([[gu, 0.0]]), np.zeros((1, 4)), np.zeros((1, 4)))
    np.testing.assert_allclose(g["grad_means"][:, 0], [gu * f / z, 0.0, 0.0], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(g["grad_scales"][:, 0], 0.0, atol=1e-12)


@pytest.mark.parametrize("deg", [0, 1, 2, 3])
def test_sh_coefficient_gradient_is_basis_times_colour_gradient(orc, deg):
    """dL/dsh[k][ch] = dL/dcolour_ch * Y_k(dir), with Y the basis pinned in
    test_oracle_sh; at degree 0 the colour sends nothing to the mean."""
    cam, scene = _case(21, deg)
    n = scene["n"]
    gm0 = np.zeros((n, 2))
    gc0 = np.zeros((n, 4))
    gr = np.random.default_rng(5).normal(size=(n, 4))
    pre = orc.preprocess(cam, scene)
    g = orc.preprocess_bwd(cam, scene, gm0, gc0, gr)
    k = (deg + 1) ** 2
    seen = 0
    for i in range(n):
        if pre["tiles_touched"][i] == 0:
            assert not g["grad_sh"][:, i].any()
            continue
        d = scene["means"][:, i].astype(np.float64) - np.asarray(cam["campos"], np.float64)
        d /= np.linalg.norm(d)
        Y = orc.sh_basis(d)[:k].astype(np.float64)
        exp = (Y[:, None] * gr[i, :3][None, :]).reshape(-1)
        np.testing.assert_allclose(g["grad_sh"][:, i], exp, rtol=2e-6, atol=1e-9)
        if deg == 0:
            np.testing.assert_allclose(g["grad_means"][:, i], 0.0, atol=1e-12)
        seen += 1
    assert seen > 5


def test_quaternion_gradient_invariants(orc):
    cam, scene = _case(31, None, n=40)
    n = scene["n"]
    gm, gc, gr = _upstream(31, n)
    pre = orc.preprocess(cam, scene)
    vis = pre["tiles_touched"] > 0
    assert vis.sum() > 10
    g = orc.preprocess_bwd(cam, scene, gm, gc, gr)
    q = scene["quats"].astype(np.float64)
    # orthogonal to q: the forward depends on q only through q / |q|
    dot = (g["grad_quats"] * q).sum(0)
    assert np.abs(dot[vis]).max() <= 1e-9 * np.abs(g["grad_quats"]).max()
    # q -> 4 q (exact in float32): the gradient scales by 1/4
    s2 = dict(scene)
    s2["quats"] = (scene["quats"] * 4).astype(np.float32)
    g2 = orc.preprocess_bwd(cam, s2, gm, gc, gr)
    np.testing.assert_allclose(g2["grad_quats"], g["grad_quats"] / 4, rtol=1e-9, atol=1e-12)
    for key in ("grad_means", "grad_scales"):
        np.testing.assert_allclose(g2[key], g[key], rtol=1e-9, atol=1e-12)
    # isotropic scales: Sigma does not depend on the rotation
    s3 = dict(scene)
    s3["scales"] = np.repeat(scene["scales"][:1], 3, axis=0)
    g3 = orc.preprocess_bwd(cam, s3, gm, gc, gr)
    assert np.abs(g3["grad_quats"]).max() <= 1e-9 * max(1.0, np.abs(g3["grad_scales"]).max())


def test_culled_gaussians_get_zero_gradients(orc):
    W, H = 32, 32
    cam = synth.look_at_camera((0.0, 0.0, -4.0), (0.0, 0.0, 0.0), W, H, 30.0, 30.0)
    means = np.array([[0.0, 0.0, -4.5],     # behind the camera
                      [0.0, 0.0, -3.96],    # in front of it but nearer than z = 0.05
                      [40.0, 0.0, 0.0],     # far off screen
                      [0.0, 0.0, 0.0]])     # visible
    n = 4
    quats = np.array([[1.0, 0, 0, 0]] * 3 + [[0.0, 0, 0, 0]])  # the visible one has q = 0: culled
    scene = synth.scenes._pack(means, np.full((n, 3), 0.1), quats, np.full(n, 0.5),
                               rgb=np.full((n, 3), 0.5))
    gm, gc, gr = _upstream(1, n)
    pre = orc.preprocess(cam, scene)
    assert not pre["tiles_touched"].any()
    g = orc.preprocess_bwd(cam, scene, gm, gc, gr)
    for key, v in g.items():
        assert not v.any(), key
