"""Pins for the oracle's appearance MLP (oracle/appearance.py).

  * the backward against central differences of the float64 forward (with
    the active set of hidden units held at the base point) for every latent
    and every weight, at three sizes including the largest (29 latents, 64
    hidden units);
  * the same gradients against torch autograd in float64 (an independent
    differentiation);
  * closed forms: zero weights give sigmoid(b2) and no latent or W1
    gradient; one latent and one hidden unit written out by hand;
  * the float32 activity decision agrees with the float64 one away from
    z = 0, and view directions are unit vectors from the camera centre.
"""
import numpy as np
import pytest

import synth
from oracle import appearance as app

SIZES = [(8, 32), (2, 5), (29, 64)]


def _case(seed, L, H, n=5):
    rng = np.random.default_rng(seed)
    cam = synth.look_at_camera((0.3, 0.2, -4.0), (0.0, 0.0, 0.0), 64, 64, 60.0, 60.0)
    means = rng.normal(0, 0.7, (3, n)).astype(np.float32)
    latent = rng.normal(0, 1.0, (L, n)).astype(np.float32)
    w = rng.normal(0, 1.0 / np.sqrt(L + 3), app.n_params(L, H)).astype(np.float32)
    g = rng.normal(0, 1.0, (3, n))
    return cam, means, latent, w, g


def _fwd_fixed(x, w64, act, L, H):
    W1, b1, W2, b2 = app.unpack(w64, L, H)
    z = W1 @ x + b1[:, None]
    h = np.where(act, z, 0.0)
    return 1.0 / (1.0 + np.exp(-(W2 @ h + b2[:, None])))


def _richardson(f, base, h):
    d1 = (f(base + h) - f(base - h)) / (2 * h)
    d2 = (f(base + h / 2) - f(base - h / 2)) / h
    return (4 * d2 - d1) / 3


@pytest.mark.parametrize("L,H", SIZES)
def test_backward_matches_finite_differences(L, H):
    cam, means, latent, w, g = _case(L * 100 + H, L, H)
    rgb, st = app.forward(cam, means, latent, w, L, H)
    dlat, dw = app.backward(cam, means, latent, w, L, H, g)
    x0, act = st["x"], st["act"]
    w64 = w.astype(np.float64)
    loss = lambda x, ww: float((g * _fwd_fixed(x, ww, act, L, H)).sum())
    # latents
    fd_lat = np.zeros_like(dlat)
    for j in range(L):
        for i in range(x0.shape[1]):
            def f(t, j=j, i=i):
                x = x0.copy()
                x[j, i] = t
                return loss(x, w64)
            fd_lat[j, i] = _richardson(f, x0[j, i], 1e-3)
    np.testing.assert_allclose(dlat, fd_lat, rtol=1e-7, atol=1e-9 * max(1, np.abs(fd_lat).max()))
    # every weight
    fd_w = np.zeros_like(dw)
    for p in range(w64.size):
        def f(t, p=p):
            ww = w64.copy()
            ww[p] = t
            return loss(x0, ww)
        fd_w[p] = _richardson(f, w64[p], 1e-3)
    np.testing.assert_allclose(dw, fd_w, rtol=1e-7, atol=1e-9 * max(1, np.abs(fd_w).max()))


@pytest.mark.parametrize("L,H", SIZES)
def test_backward_matches_torch_autograd(L, H):
    torch = pytest.importorskip("torch")
    cam, means, latent, w, g = _case(7 + L, L, H, n=40)
    rgb, st = app.forward(cam, means, latent, w, L, H)
    dlat, dw = app.backward(cam, means, latent, w, L, H, g)
    x = torch.tensor(st["x"], dtype=torch.float64, requires_grad=True)
    W1, b1, W2, b2 = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in app.unpack(w, L, H))
    act = torch.tensor(st["act"])
    z = W1 @ x + b1[:, None]
    h = torch.where(act, z, torch.zeros_like(z))
    out = torch.sigmoid(W2 @ h + b2[:, None])
    np.testing.assert_allclose(out.detach().numpy(), rgb, rtol=1e-12, atol=1e-14)
    (out * torch.tensor(g)).sum().backward()
    ref = np.concatenate([W1.grad.numpy().reshape(-1), b1.grad.numpy(), W2.grad.numpy().reshape(-1),
                          b2.grad.numpy()])
    np.testing.assert_allclose(dw, ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dlat, x.grad.numpy()[:L], rtol=1e-10, atol=1e-12)


def test_zero_weights_closed_form():
    L, H = 8, 32
    cam, means, latent, w, g = _case(3, L, H, n=7)
    W1, b1, W2, b2 = (a.copy() for a in app.unpack(w, L, H))
    W1[:] = 0.0
    W2[:] = 0.0
    w0 = np.concatenate([W1.reshape(-1), b1, W2.reshape(-1), b2])
    rgb, _ = app.forward(cam, means, latent, w0, L, H)
    np.testing.assert_allclose(rgb, np.repeat((1 / (1 + np.exp(-b2)))[:, None], 7, axis=1), rtol=1e-12)
    dlat, dw = app.backward(cam, means, latent, w0, L, H, g)
    assert not dlat.any()
    gW1, gb1, gW2, gb2 = app.unpack(dw, L, H)
    assert not gW1.any() and not gb1.any()
    s = 1 / (1 + np.exp(-b2))
    dy = g * (s * (1 - s))[:, None]
    np.testing.assert_allclose(gb2, dy.sum(1), rtol=1e-12)
    np.testing.assert_allclose(gW2, np.outer(dy.sum(1), np.maximum(b1, 0.0)), rtol=1e-12, atol=1e-15)


def test_one_latent_one_unit_by_hand():
    L, H = 1, 1
    cam = synth.look_at_camera((0.0, 0.0, -4.0), (0.0, 0.0, 0.0), 16, 16, 16.0, 16.0)
    means = np.array([[0.0], [0.0], [0.0]], np.float32)  # straight ahead: direction (0, 0, 1)
    latent = np.array([[0.75]], np.float32)
    w1, wdx, wdy, wdz, b1 = 0.5, 0.1, -0.2, 0.3, 0.05
    w2, b2 = np.array([1.0, -2.0, 0.5]), np.array([0.1, 0.0, -0.3])
    w = np.array([w1, wdx, wdy, wdz, b1, *w2, *b2], np.float32)
    rgb, _ = app.forward(cam, means, latent, w, L, H)
    z = w1 * 0.75 + wdz * 1.0 + b1
    expect = 1 / (1 + np.exp(-(np.float32(w2).astype(float) * z + np.float32(b2).astype(float))))
    np.testing.assert_allclose(rgb[:, 0], expect, rtol=1e-7)
    g = np.array([[1.0], [0.5], [-1.0]])
    dlat, dw = app.backward(cam, means, latent, w, L, H, g)
    s = expect
    dy = g[:, 0] * s * (1 - s)
    dz = float((np.float32(w2).astype(float) * dy).sum())
    np.testing.assert_allclose(dlat[0, 0], dz * np.float32(w1), rtol=1e-7)
    np.testing.assert_allclose(dw[0], dz * 0.75, rtol=1e-7)       # dW1 against the latent
    np.testing.assert_allclose(dw[3], dz * 1.0, rtol=1e-7)        # dW1 against dir z
    np.testing.assert_allclose(dw[4], dz, rtol=1e-7)              # db1


def test_activity_and_directions():
    L, H = 8, 32
    rng = np.random.default_rng(9)
    cam = synth.view_camera(4000, 4.0, 400, 400, 400.0)
    n = 20000
    means = rng.normal(0, 1, (3, n)).astype(np.float32)
    latent = rng.normal(0, 1, (L, n)).astype(np.float32)
    w = rng.normal(0, 0.4, app.n_params(L, H)).astype(np.float32)
    d = app.view_dirs(cam, means)
    np.testing.assert_allclose(np.linalg.norm(d.astype(np.float64), axis=0), 1.0, atol=3e-7)
    v = means.astype(np.float64) - np.asarray(cam["campos"], np.float64)[:, None]
    assert ((v * d).sum(0) > 0).all()
    _, st = app.forward(cam, means, latent, w, L, H)
    far = np.abs(st["z"]) > 1e-5
    assert np.array_equal(st["act"][far], (st["z"] > 0)[far])
