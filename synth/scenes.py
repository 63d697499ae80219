"""Procedural scenes and cameras, drawn with numpy's PCG64 from fixed seeds.

The five workloads mirror the shapes of the scenes the pages measure on:

* ``cfg0`` - 1,000 Gaussians on a jittered unit sphere, 64x64, precomputed RGB.
* ``cfg1`` - the 160,000-Gaussian procedural gallery scene (60% sphere shell
  coloured by its normal, 20% three-turn helix, 20% checkered plane), SH
  degree 3, 720x720 ("rigel" README, the gallery scene and timing table).
* ``cfg2`` - the ``cfg1`` scene at 1920x1080, fx = fy = 1100, plus an
  upstream gradient dL/dI ~ N(0, 1).
* ``cfg3`` - 1,000,000 Gaussians, dense overdraw: 80% in a thick shell
  r in [0.9, 1.0], 20% uniform in a cube of side 6, 1920x1080.
* ``cfg4`` - 300,000 Gaussians drawn like ``cfg3``, 16 views at 400x400 on a
  radius-4 sphere, with a second scene as the L1 target.

Layouts: means/scales [3][N], quats [4][N] (w, x, y, z), opacity [N],
sh [(d+1)^2][3][N] (coefficient-major, then channel), rgb [3][N].
Cameras: dict(R row-major world->camera, t, campos, fx, fy, cx, cy, width,
height) with p_cam = R p + t, +z forward, image y down.
"""
from __future__ import annotations

import numpy as np

# Y_0 = 1 / (2 sqrt(pi)); used only to turn a scene colour into a DC
# coefficient when drawing inputs.
_Y0 = 0.28209479177387814

CONFIGS = ("cfg0", "cfg1", "cfg2", "cfg3", "cfg4")


def look_at_camera(eye, target, width, height, fx, fy, cx=None, cy=None, up=(0.0, 1.0, 0.0)):
    """Pinhole camera at ``eye`` looking at ``target``; image x right, y down."""
    eye = np.asarray(eye, np.float64)
    target = np.asarray(target, np.float64)
    up = np.asarray(up, np.float64)
    f = target - eye
    f = f / np.linalg.norm(f)
    if abs(float(np.dot(f, up / np.linalg.norm(up)))) > 0.999:
        up = np.array([0.0, 0.0, 1.0])
    x = np.cross(f, up)
    x = x / np.linalg.norm(x)
    y = np.cross(f, x)
    R = np.stack([x, y, f]).astype(np.float32)
    t = (-(R.astype(np.float64) @ eye)).astype(np.float32)
    return dict(R=R.reshape(9), t=t, campos=eye.astype(np.float32),
                fx=np.float32(fx), fy=np.float32(fy),
                cx=np.float32(width / 2.0 if cx is None else cx),
                cy=np.float32(height / 2.0 if cy is None else cy),
                width=int(width), height=int(height))


def view_camera(seed, radius, width, height, fx, fy=None):
    """Camera at a random direction (seeded) on a sphere, looking at the origin."""
    rng = np.random.default_rng(seed)
    d = rng.standard_normal(3)
    d = d / np.linalg.norm(d)
    return look_at_camera(radius * d, (0.0, 0.0, 0.0), width, height, fx, fx if fy is None else fy)


def _unit(rng, n):
    d = rng.standard_normal((n, 3))
    return d / np.linalg.norm(d, axis=1, keepdims=True)


def _log_uniform(rng, lo, hi, shape):
    return np.exp(rng.uniform(np.log(lo), np.log(hi), shape))


def _quats(rng, n):
    q = rng.standard_normal((n, 4))
    return q / np.linalg.norm(q, axis=1, keepdims=True)


def _pack(means, scales, quats, opacity, sh=None, sh_degree=0, rgb=None):
    out = dict(n=int(means.shape[0]),
               means=np.ascontiguousarray(means.T, np.float32),
               scales=np.ascontiguousarray(scales.T, np.float32),
               quats=np.ascontiguousarray(quats.T, np.float32),
               opacity=np.ascontiguousarray(opacity, np.float32),
               sh=None, rgb=None, sh_degree=int(sh_degree))
    if sh is not None:
        out["sh"] = np.ascontiguousarray(sh, np.float32)
    if rgb is not None:
        out["rgb"] = np.ascontiguousarray(rgb.T, np.float32)
    return out


def shell_scene(n, seed, scale_lo=0.005, scale_hi=0.05, op_lo=0.1, op_hi=0.99):
    """Jittered unit-sphere shell with precomputed RGB (the 1k/64x64 case)."""
    rng = np.random.default_rng(seed)
    d = _unit(rng, n)
    means = d + rng.normal(0.0, 0.02, (n, 3))
    scales = _log_uniform(rng, scale_lo, scale_hi, (n, 3))
    quats = _quats(rng, n)
    opacity = rng.uniform(op_lo, op_hi, n)
    rgb = rng.uniform(0.0, 1.0, (n, 3))
    return _pack(means, scales, quats, opacity, rgb=rgb)


def gallery_scene(n, seed):
    """Sphere shell coloured by normal (60%), three-turn helix (20%),
    checkered 4x4 plane at y = -1.2 (20%); SH degree 3."""
    rng = np.random.default_rng(seed)
    n_shell = int(round(0.6 * n))
    n_helix = int(round(0.2 * n))
    n_plane = n - n_shell - n_helix
    d = _unit(rng, n_shell)
    shell = d + rng.normal(0.0, 0.02, (n_shell, 3))
    shell_col = 0.5 * (d + 1.0)
    t = rng.uniform(0.0, 1.0, n_helix)
    helix = np.stack([0.6 * np.cos(6 * np.pi * t), -1.0 + 2.0 * t, 0.6 * np.sin(6 * np.pi * t)], 1)
    helix = helix + rng.normal(0.0, 0.02, (n_helix, 3))
    helix_col = np.stack([t, 1.0 - t, np.full_like(t, 0.5)], 1)
    px = rng.uniform(-2.0, 2.0, n_plane)
    pz = rng.uniform(-2.0, 2.0, n_plane)
    plane = np.stack([px, np.full_like(px, -1.2), pz], 1)
    check = (np.floor(px / 0.5) + np.floor(pz / 0.5)).astype(np.int64) % 2
    plane_col = np.repeat(np.where(check == 0, 0.9, 0.1)[:, None], 3, 1)
    means = np.concatenate([shell, helix, plane])
    colour = np.concatenate([shell_col, helix_col, plane_col])
    scales = _log_uniform(rng, 0.003, 0.03, (n, 3))
    quats = _quats(rng, n)
    opacity = rng.uniform(0.3, 0.99, n)
    sh = rng.normal(0.0, 0.05, (16, 3, n))
    sh[0] = (colour / _Y0).T
    return _pack(means, scales, quats, opacity, sh=sh, sh_degree=3)


def dense_scene(n, seed):
    """Thick shell r ~ U(0.9, 1.0) (80%) plus a uniform cube of side 6 (20%);
    SH degree 3 with DC ~ U(0, 1) and the rest ~ N(0, 0.1)."""
    rng = np.random.default_rng(seed)
    n_shell = int(round(0.8 * n))
    n_cube = n - n_shell
    d = _unit(rng, n_shell)
    r = rng.uniform(0.9, 1.0, n_shell)
    shell = d * r[:, None]
    cube = rng.uniform(-3.0, 3.0, (n_cube, 3))
    means = np.concatenate([shell, cube])
    scales = _log_uniform(rng, 0.002, 0.02, (n, 3))
    quats = _quats(rng, n)
    opacity = rng.uniform(0.05, 0.9, n)
    sh = rng.normal(0.0, 0.1, (16, 3, n))
    sh[0] = rng.uniform(0.0, 1.0, (3, n))
    return _pack(means, scales, quats, opacity, sh=sh, sh_degree=3)


def random_scene(n, seed, cam, sh_degree=None, scale_lo=0.01, scale_hi=0.3, op_lo=0.05, op_hi=0.99,
                 depth_lo=1.0, depth_hi=6.0, spread=1.2, unit_quats=False):
    """Small random scene in front of ``cam`` (for edge-case and FD tests).

    Means are placed along rays through the image (``spread`` times the
    frame, so some land off-screen) at depths U(depth_lo, depth_hi).
    Quaternions are left unnormalised unless ``unit_quats``.
    """
    rng = np.random.default_rng(seed)
    W, H = cam["width"], cam["height"]
    R = np.asarray(cam["R"], np.float64).reshape(3, 3)
    eye = np.asarray(cam["campos"], np.float64)
    px = rng.uniform(-0.5 * spread, 0.5 * spread, n) * W + cam["cx"]
    py = rng.uniform(-0.5 * spread, 0.5 * spread, n) * H + cam["cy"]
    z = rng.uniform(depth_lo, depth_hi, n)
    pc = np.stack([(px - cam["cx"]) / cam["fx"] * z, (py - cam["cy"]) / cam["fy"] * z, z], 1)
    means = pc @ R + eye  # R is orthonormal: world = R^T p_cam + eye
    scales = _log_uniform(rng, scale_lo, scale_hi, (n, 3))
    q = rng.standard_normal((n, 4))
    if unit_quats:
        q = q / np.linalg.norm(q, axis=1, keepdims=True)
    else:
        q = q * rng.uniform(0.5, 2.0, (n, 1))
    opacity = rng.uniform(op_lo, op_hi, n)
    if sh_degree is None:
        rgb = rng.uniform(0.0, 1.0, (n, 3))
        return _pack(means, scales, q, opacity, rgb=rgb)
    k = (sh_degree + 1) ** 2
    sh = rng.normal(0.0, 0.2, (k, 3, n))
    sh[0] = rng.uniform(0.0, 1.0, (3, n)) / _Y0
    return _pack(means, scales, q, opacity, sh=sh, sh_degree=sh_degree)


def upstream_gradient(seed, width, height):
    """dL/dI ~ N(0, 1) per channel, planar [3][H][W] float32."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((3, height, width)).astype(np.float32)


def config_scene(name: str, view: int = 0):
    """(scene, camera, dL_dimage or None) for one of the five workloads.

    For ``cfg4`` the returned gradient is None (it is an L1 residual against
    ``config_scene('cfg4_ref', view)``, which the caller renders).
    """
    if name == "cfg0":
        cam = look_at_camera((0.0, 0.0, -4.0), (0.0, 0.0, 0.0), 64, 64, 64.0, 64.0, 32.0, 32.0)
        return shell_scene(1000, 1000), cam, None
    if name == "cfg1":
        cam = view_camera(2001, 4.0, 720, 720, 720.0)
        return gallery_scene(160_000, 1001), cam, None
    if name == "cfg2":
        cam = view_camera(2001, 4.0, 1920, 1080, 1100.0)
        return gallery_scene(160_000, 1001), cam, upstream_gradient(3002, 1920, 1080)
    if name == "cfg3":
        cam = view_camera(2003, 4.0, 1920, 1080, 1100.0)
        return dense_scene(1_000_000, 1003), cam, upstream_gradient(3003, 1920, 1080)
    if name == "cfg4":
        cam = view_camera(4000 + view, 4.0, 400, 400, 400.0)
        return dense_scene(300_000, 1004), cam, None
    if name == "cfg4_ref":
        cam = view_camera(4000 + view, 4.0, 400, 400, 400.0)
        return dense_scene(300_000, 1504), cam, None
    raise KeyError(name)
