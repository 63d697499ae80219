"""Pins for the oracle's preprocess (projection, conic, radius, tile span, cull).

Every expected value here comes from a closed form written in float64, from
a library routine (scipy's quaternion rotation), or from a brute-force
predicate - never from the oracle itself.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.spatial.transform import Rotation

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def scene_of(means, scales, quats, opacity=None, rgb=None):
    means = np.asarray(means, np.float64).reshape(-1, 3)
    n = means.shape[0]
    scales = np.broadcast_to(np.asarray(scales, np.float64), (n, 3))
    quats = np.broadcast_to(np.asarray(quats, np.float64), (n, 4))
    opacity = np.full(n, 0.5) if opacity is None else np.broadcast_to(np.asarray(opacity, np.float64), (n,))
    rgb = np.ones((n, 3)) if rgb is None else np.broadcast_to(np.asarray(rgb, np.float64), (n, 3))
    return dict(n=n, means=np.ascontiguousarray(means.T, np.float32),
                scales=np.ascontiguousarray(scales.T, np.float32),
                quats=np.ascontiguousarray(quats.T, np.float32),
                opacity=np.ascontiguousarray(opacity, np.float32),
                rgb=np.ascontiguousarray(rgb.T, np.float32), sh=None, sh_degree=0)


def cam0():
    return synth.look_at_camera((0.0, 0.0, -4.0), (0.0, 0.0, 0.0), 64, 64, 64.0, 64.0, 32.0, 32.0)


def identity_cam(W=64, H=64, f=64.0):
    return dict(R=np.eye(3, dtype=np.float32).reshape(9), t=np.zeros(3, np.float32),
                campos=np.zeros(3, np.float32), fx=np.float32(f), fy=np.float32(f),
                cx=np.float32(W / 2), cy=np.float32(H / 2), width=W, height=H)


def closed_form_cov2d(cam, mean, cov3d, clamp=True):
    """Sigma_2d = J W Sigma W^T J^T + 0.3 I in float64 (the pages' EWA formula)."""
    R = np.asarray(cam["R"], np.float64).reshape(3, 3)
    pc = R @ np.asarray(mean, np.float64) + np.asarray(cam["t"], np.float64)
    x, y, z = pc
    fx, fy = float(cam["fx"]), float(cam["fy"])
    if clamp:
        limx = 1.3 * 0.5 * cam["width"] / fx
        limy = 1.3 * 0.5 * cam["height"] / fy
        x = min(limx, max(-limx, x / z)) * z
        y = min(limy, max(-limy, y / z)) * z
    J = np.array([[fx / z, 0.0, -fx * x / z ** 2], [0.0, fy / z, -fy * y / z ** 2]])
    T = J @ R
    return T @ cov3d @ T.T + 0.3 * np.eye(2), pc


def conic_of(cov):
    return np.linalg.inv(cov)


def radius_of(cov):
    a, b, c = cov[0, 0], cov[0, 1], cov[1, 1]
    det = a * c - b * b
    mid = 0.5 * (a + c)
    lam = mid + math.sqrt(max(mid * mid - det, 0.1))
    return 3.0 * math.sqrt(lam)


def test_constants_match_pages(orc):
    g = json.load(open(os.path.join(GOLDEN, "learn_gs_constants.json")))
    c = orc.constants()
    expect = [g["TILE"], g["DILATION"], g["Z_NEAR"], g["FRUSTUM_CLAMP"], g["DISC_FLOOR"], g["SIGMA"],
              g["ALPHA_MIN"], g["ALPHA_MAX"], g["T_STOP"]]
    np.testing.assert_array_equal(c, np.asarray(expect, np.float32))


def test_on_axis_isotropic_closed_form(orc):
    """f s / z = 0.8 -> a = c = 0.8^2 + 0.3, b = 0; radius 3 sqrt(a + sqrt(0.1)) ceiled."""
    cam = cam0()
    s = 0.05
    out = orc.preprocess(cam, scene_of([0, 0, 0], [s, s, s], [1, 0, 0, 0]))
    a = (64.0 * s / 4.0) ** 2 + 0.3
    u, v, z, r = out["xy_depth"][0]
    A, B, C, o = out["conic_op"][0]
    assert (u, v, z) == (32.0, 32.0, 4.0)
    np.testing.assert_allclose([A, B, C], [1 / a, 0.0, 1 / a], rtol=1e-6, atol=1e-7)
    assert r == math.ceil(3.0 * math.sqrt(a + math.sqrt(0.1))) == 4
    # span: floor((32-4)/16)=1 .. floor((32+4)/16)+1=3 in both axes -> 2x2 tiles
    assert out["tiles_touched"][0] == 4
    assert o == np.float32(0.5)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_off_axis_isotropic_closed_form(orc, seed):
    """Isotropic Sigma = s^2 I gives Sigma_2d = s^2 J J^T + 0.3 I for any rotation."""
    rng = np.random.default_rng(seed)
    cam = synth.view_camera(seed + 10, 4.0, 96, 80, 90.0, 70.0)
    n = 64
    R = np.asarray(cam["R"], np.float64).reshape(3, 3)
    pc = np.stack([rng.uniform(-0.4, 0.4, n), rng.uniform(-0.4, 0.4, n), np.ones(n)], 1)
    pc *= rng.uniform(1.0, 6.0, (n, 1))
    means = (pc - np.asarray(cam["t"], np.float64)) @ R  # R^T (p_c - t)
    s = rng.uniform(0.01, 0.2, n)
    quats = rng.standard_normal((n, 4))
    scene = scene_of(means, np.repeat(s[:, None], 3, 1), quats)
    out = orc.preprocess(cam, scene)
    checked = 0
    for i in range(n):
        m64 = scene["means"][:, i].astype(np.float64)
        s64 = float(scene["scales"][0, i])
        cov, pcc = closed_form_cov2d(cam, m64, s64 * s64 * np.eye(3))
        if out["tiles_touched"][i] == 0:
            continue
        conic = conic_of(cov)
        A, B, C, _ = out["conic_op"][i]
        scale = max(abs(conic[0, 0]), abs(conic[1, 1]))
        np.testing.assert_allclose([A, B, C], [conic[0, 0], conic[0, 1], conic[1, 1]],
                                   atol=3e-5 * scale)
        u, v, z, r = out["xy_depth"][i]
        np.testing.assert_allclose([u, v, z], [cam["fx"] * pcc[0] / pcc[2] + cam["cx"],
                                               cam["fy"] * pcc[1] / pcc[2] + cam["cy"], pcc[2]],
                                   rtol=1e-5, atol=1e-4)
        rr = radius_of(cov)
        if abs(rr - round(rr)) > 1e-3:
            assert r == math.ceil(rr)
        checked += 1
    assert checked > n // 2


@pytest.mark.parametrize("seed", [3, 4])
def test_anisotropic_matches_library_rotation(orc, seed):
    """Sigma = R(q) S^2 R(q)^T with R(q) from scipy (scalar-last quaternions)."""
    rng = np.random.default_rng(seed)
    cam = synth.view_camera(seed + 20, 4.0, 128, 128, 120.0)
    n = 64
    scene = synth.random_scene(n, seed, cam, scale_lo=0.02, scale_hi=0.2, spread=0.8)
    out = orc.preprocess(cam, scene)
    for i in range(n):
        if out["tiles_touched"][i] == 0:
            continue
        q = scene["quats"][:, i].astype(np.float64)
        Rq = Rotation.from_quat([q[1], q[2], q[3], q[0]]).as_matrix()
        S = np.diag(scene["scales"][:, i].astype(np.float64))
        cov3 = Rq @ S @ S @ Rq.T
        cov, _ = closed_form_cov2d(cam, scene["means"][:, i].astype(np.float64), cov3)
        conic = conic_of(cov)
        A, B, C, _ = out["conic_op"][i]
        scale = max(abs(conic[0, 0]), abs(conic[1, 1]))
        np.testing.assert_allclose([A, B, C], [conic[0, 0], conic[0, 1], conic[1, 1]],
                                   atol=1e-4 * scale)


def test_frustum_clamp_branch(orc):
    """Far off-axis centre: J is built from x/z clamped to 1.3 * W/(2 fx)."""
    cam = identity_cam(64, 64, 64.0)
    lim = 1.3 * 32.0 / 64.0
    for (xz, yz) in [(0.8, 0.0), (-0.9, 0.1), (0.1, 0.75), (0.7, -0.72)]:
        z = 4.0
        mean = np.array([xz * z, yz * z, z])
        s = 0.8
        scene = scene_of(mean, [s, 0.5 * s, 0.7 * s], [0.9, 0.1, -0.3, 0.2])
        out = orc.preprocess(cam, scene)
        assert out["tiles_touched"][0] > 0
        q = scene["quats"][:, 0].astype(np.float64)
        Rq = Rotation.from_quat([q[1], q[2], q[3], q[0]]).as_matrix()
        S = np.diag(scene["scales"][:, 0].astype(np.float64))
        cov3 = Rq @ S @ S @ Rq.T
        cov_c, _ = closed_form_cov2d(cam, scene["means"][:, 0].astype(np.float64), cov3, clamp=True)
        cov_u, _ = closed_form_cov2d(cam, scene["means"][:, 0].astype(np.float64), cov3, clamp=False)
        A, B, C, _ = out["conic_op"][0]
        got = np.array([A, B, C])
        want_c = conic_of(cov_c)[[0, 0, 1], [0, 1, 1]]
        want_u = conic_of(cov_u)[[0, 0, 1], [0, 1, 1]]
        np.testing.assert_allclose(got, want_c, atol=1e-5 * np.abs(want_c).max())
        assert np.abs(got - want_u).max() > 1e-2 * np.abs(want_u).max()
        assert abs(xz) > lim or abs(yz) > lim


def test_quaternion_scale_invariance(orc):
    cam = cam0()
    rng = np.random.default_rng(7)
    q = rng.standard_normal(4)
    base = orc.preprocess(cam, scene_of([0.1, -0.2, 0.3], [0.05, 0.1, 0.02], q))
    for k in (1e-3, 0.5, 3.0, 1e3):
        o = orc.preprocess(cam, scene_of([0.1, -0.2, 0.3], [0.05, 0.1, 0.02], k * q))
        np.testing.assert_allclose(o["conic_op"][0], base["conic_op"][0], rtol=2e-6)
        assert o["xy_depth"][0][3] == base["xy_depth"][0][3]


def test_isotropic_independent_of_rotation(orc):
    cam = cam0()
    rng = np.random.default_rng(8)
    base = orc.preprocess(cam, scene_of([0.2, 0.1, -0.1], [0.07] * 3, [1, 0, 0, 0]))
    for _ in range(10):
        o = orc.preprocess(cam, scene_of([0.2, 0.1, -0.1], [0.07] * 3, rng.standard_normal(4)))
        np.testing.assert_allclose(o["conic_op"][0], base["conic_op"][0], rtol=2e-6, atol=1e-7)


def test_near_plane_boundary(orc):
    """z must be strictly greater than 0.05 (the notebook's Pc[:, 2] > Z_NEAR)."""
    cam = identity_cam()
    z0 = np.float32(0.05)
    z1 = np.nextafter(z0, np.float32(1.0))
    out = orc.preprocess(cam, scene_of([[0, 0, z0], [0, 0, z1], [0, 0, -1.0]], [0.001] * 3, [1, 0, 0, 0]))
    assert out["tiles_touched"][0] == 0 and out["tiles_touched"][1] > 0 and out["tiles_touched"][2] == 0
    assert out["xy_depth"][1][2] == z1
    assert not out["xy_depth"][0].any() and not out["conic_op"][0].any() and not out["rgb"][0].any()


def test_degenerate_and_non_finite_are_culled(orc):
    cam = cam0()
    nan, inf = float("nan"), float("inf")
    means = [[nan, 0, 0], [0, 0, 0], [0, 0, 0], [0, 0, 0], [0, 0, 0], [inf, 0, 0], [0, 0, 0]]
    scales = [[0.05] * 3, [0.05] * 3, [inf, 0.05, 0.05], [0.05] * 3, [nan, 0.05, 0.05], [0.05] * 3, [0.05] * 3]
    quats = [[1, 0, 0, 0], [0, 0, 0, 0], [1, 0, 0, 0], [1, 0, 0, 0], [1, 0, 0, 0], [1, 0, 0, 0], [1, 0, 0, 0]]
    opac = [0.5, 0.5, 0.5, nan, 0.5, 0.5, 0.5]
    out = orc.preprocess(cam, scene_of(means, scales, quats, opac))
    assert list(out["tiles_touched"]) == [0, 0, 0, 0, 0, 0, 4]
    for k in ("xy_depth", "conic_op", "rgb"):
        assert not out[k][:6].any()


def test_off_screen_culled(orc):
    cam = cam0()
    # world x maps to -u here (camera looks down +z from z = -4): x = +3 -> u = 32 - 48
    out = orc.preprocess(cam, scene_of([[3.0, 0, 0], [0, 3.0, 0], [0.3, 0, 0]], [0.01] * 3, [1, 0, 0, 0]))
    assert out["tiles_touched"][0] == 0 and out["tiles_touched"][1] == 0
    assert out["tiles_touched"][2] > 0


def test_tile_span_equals_brute_force_overlap(orc):
    """learn-gs claim 2: spans cover exactly the tiles the 2r square touches."""
    rng = np.random.default_rng(11)
    uv = rng.uniform(0, 1, (300, 2)) * 80 - 8  # includes off-screen centres
    r = rng.integers(1, 30, 300).astype(np.float32)
    TX = TY = 4
    for i in range(300):
        u, v = np.float32(uv[i, 0]), np.float32(uv[i, 1])
        x0, x1, y0, y1 = orc.tile_span(u, v, r[i], TX, TY)
        for tx in range(TX):
            for ty in range(TY):
                overlap = (tx * 16 <= u + r[i] and (tx + 1) * 16 > u - r[i]
                           and ty * 16 <= v + r[i] and (ty + 1) * 16 > v - r[i])
                listed = (x0 <= tx < x1) and (y0 <= ty < y1)
                assert overlap == listed, (i, tx, ty)


def test_tiles_touched_is_span_area_and_listed(orc):
    cam = synth.config_scene("cfg0")[1]
    scene = synth.config_scene("cfg0")[0]
    out = orc.preprocess(cam, scene)
    TX, TY = orc.tiles_xy(cam)
    for g in range(0, scene["n"], 7):
        u, v, z, r = out["xy_depth"][g]
        if out["tiles_touched"][g] == 0:
            assert r == 0
            continue
        brute = sum(1 for tx in range(TX) for ty in range(TY)
                    if tx * 16 <= u + r and (tx + 1) * 16 > u - r and ty * 16 <= v + r and (ty + 1) * 16 > v - r)
        assert brute == out["tiles_touched"][g]
