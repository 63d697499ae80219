"""Pins for the oracle's spherical-harmonic colour (degrees 0..3).

The basis is checked against scipy's complex spherical harmonics (a library
routine), by quadrature orthonormality, and by parity; the colour layout is
checked through preprocess with one-hot coefficients.
"""
import numpy as np
import pytest
from scipy import special

import synth


def real_sh_scipy(l, m, d):
    """Real SH in the (Condon-Shortley phased) convention the page's table
    uses: sqrt(2) Im Y_l^|m| for m < 0, Y_l^0, sqrt(2) Re Y_l^m for m > 0."""
    x, y, z = d
    theta = np.arccos(np.clip(z, -1, 1))  # polar
    phi = np.arctan2(y, x)                # azimuth
    Y = special.sph_harm_y(l, abs(m), theta, phi)
    if m < 0:
        return np.sqrt(2.0) * Y.imag
    if m > 0:
        return np.sqrt(2.0) * Y.real
    return Y.real


def basis_index(l, m):
    return l * l + l + m


def random_dirs(n, seed):
    rng = np.random.default_rng(seed)
    d = rng.standard_normal((n, 3))
    return d / np.linalg.norm(d, axis=1, keepdims=True)


def test_basis_matches_scipy(orc):
    for d in random_dirs(200, 0):
        d32 = d.astype(np.float32)
        got = orc.sh_basis(d32)
        for l in range(4):
            for m in range(-l, l + 1):
                want = real_sh_scipy(l, m, d32.astype(np.float64))
                assert abs(got[basis_index(l, m)] - want) < 2e-6 * max(1.0, abs(want)), (l, m, d)


def test_basis_orthonormal_by_quadrature(orc):
    """Integral of Y_i Y_j over the sphere is delta_ij (Gauss-Legendre x uniform phi)."""
    nt, nphi = 24, 48
    ct, wt = np.polynomial.legendre.leggauss(nt)
    phis = (np.arange(nphi) + 0.5) * 2 * np.pi / nphi
    G = np.zeros((16, 16))
    for c, w in zip(ct, wt):
        s = np.sqrt(1 - c * c)
        for p in phis:
            Y = orc.sh_basis(np.array([s * np.cos(p), s * np.sin(p), c])).astype(np.float64)
            G += w * (2 * np.pi / nphi) * np.outer(Y, Y)
    np.testing.assert_allclose(G, np.eye(16), atol=5e-6)


def test_basis_parity(orc):
    for d in random_dirs(50, 1):
        a = orc.sh_basis(d)
        b = orc.sh_basis(-d)
        for l in range(4):
            for m in range(-l, l + 1):
                k = basis_index(l, m)
                assert abs(b[k] - (-1) ** l * a[k]) < 1e-6


@pytest.mark.parametrize("degree", [0, 1, 2, 3])
def test_colour_layout_one_hot(orc, degree):
    """Coefficient k of channel ch (sh[k][ch][g]) alone gives rgb_ch = Y_k(dir)."""
    cam = synth.look_at_camera((0.3, 0.2, -4.0), (0.0, 0.0, 0.0), 64, 64, 64.0, 64.0)
    rng = np.random.default_rng(degree)
    K = (degree + 1) ** 2
    n = 3 * K
    means = rng.uniform(-0.5, 0.5, (n, 3))
    sh = np.zeros((K, 3, n), np.float32)
    for g in range(n):
        sh[g // 3, g % 3, g] = 1.0
    scene = dict(n=n, means=np.ascontiguousarray(means.T, np.float32),
                 scales=np.full((3, n), 0.05, np.float32),
                 quats=np.tile(np.array([[1], [0], [0], [0]], np.float32), (1, n)),
                 opacity=np.full(n, 0.5, np.float32), sh=sh, sh_degree=degree, rgb=None)
    out = orc.preprocess(cam, scene)
    assert (out["tiles_touched"] > 0).all()
    for g in range(n):
        k, ch = g // 3, g % 3
        d = scene["means"][:, g].astype(np.float64) - cam["campos"].astype(np.float64)
        d /= np.linalg.norm(d)
        l = int(np.floor(np.sqrt(k)))
        m = k - l * l - l
        want = np.zeros(3)
        want[ch] = real_sh_scipy(l, m, d)
        np.testing.assert_allclose(out["rgb"][g, :3], want, atol=2e-6)
        assert out["rgb"][g, 3] == 0.0


def test_dc_only_colour(orc):
    cam = synth.look_at_camera((0.0, 0.0, -4.0), (0.0, 0.0, 0.0), 64, 64, 64.0, 64.0)
    colour = np.array([0.2, 0.5, 0.9])
    y0 = 0.5 / np.sqrt(np.pi)
    sh = (colour / y0).astype(np.float32).reshape(1, 3, 1)
    scene = dict(n=1, means=np.zeros((3, 1), np.float32), scales=np.full((3, 1), 0.05, np.float32),
                 quats=np.array([[1], [0], [0], [0]], np.float32), opacity=np.full(1, 0.5, np.float32),
                 sh=sh, sh_degree=0, rgb=None)
    out = orc.preprocess(cam, scene)
    np.testing.assert_allclose(out["rgb"][0, :3], colour, rtol=1e-6)
