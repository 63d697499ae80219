"""Plain CPU oracle of the appearance MLP ("rigel" README, section
"Appearance MLP"): per Gaussian, a latent of L floats concatenated with the
unit view direction goes through one ReLU layer of H units and one sigmoid
layer of 3 units, giving the Gaussian's colour; the backward gives the
gradients of the latents and of all four weight arrays (the view direction
is a constant, as on that page).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may use it; the product path never does.

Arithmetic is float64 (numpy), with two exceptions that decide discrete
things in the kernels' precision:
  * the view direction is computed in float32 exactly as the preprocess
    computes the SH direction: v = mean - campos, |v| = sqrt((vx vx + vy vy)
    + vz vz), d = v / |v| (correctly rounded);
  * whether a hidden unit is active (z > 0) is decided on z evaluated in
    float32 in the order z = (((b1 + W1[i,0] x0) + W1[i,1] x1) + ...), each
    product and sum rounded (no fused multiply-add), which is how the
    kernels evaluate it.

Weights are packed in one float array: W1 [H][L+3] (row i = hidden unit i,
columns the latent then the direction x, y, z), b1 [H], W2 [3][H], b2 [3].
"""
from __future__ import annotations

import numpy as np

MAX_INPUTS = 32   # L + 3
MAX_HIDDEN = 64


def n_params(L: int, H: int) -> int:
    return H * (L + 3) + H + 3 * H + 3


def unpack(weights, L: int, H: int):
    w = np.asarray(weights, np.float64).reshape(-1)
    assert w.size == n_params(L, H)
    K = L + 3
    o = 0
    W1 = w[o:o + H * K].reshape(H, K); o += H * K
    b1 = w[o:o + H]; o += H
    W2 = w[o:o + 3 * H].reshape(3, H); o += 3 * H
    b2 = w[o:o + 3]
    return W1, b1, W2, b2


def view_dirs(cam: dict, means) -> np.ndarray:
    """[3, n] float32 unit directions normalize(mean - campos)."""
    m = np.asarray(means, np.float32)
    c = np.asarray(cam["campos"], np.float32).reshape(3, 1)
    v = m - c
    n = np.sqrt((v[0] * v[0] + v[1] * v[1]) + v[2] * v[2])
    return (v / n).astype(np.float32)


def _inputs(cam, means, latent, L):
    lat = np.asarray(latent, np.float32).reshape(L, -1)
    return np.concatenate([lat, view_dirs(cam, means)], axis=0)  # [L+3, n] float32


def _active(x32, weights, L, H):
    """z > 0 per hidden unit, z summed in float32 in input order."""
    w32 = np.asarray(weights, np.float32).reshape(-1)
    K = L + 3
    W1 = w32[:H * K].reshape(H, K)
    b1 = w32[H * K:H * K + H]
    z = np.repeat(b1[:, None], x32.shape[1], axis=1).astype(np.float32)
    for j in range(K):
        z = (z + (W1[:, j:j + 1] * x32[j:j + 1, :]).astype(np.float32)).astype(np.float32)
    return z > 0


def forward(cam: dict, means, latent, weights, L: int, H: int):
    """Returns rgb [3, n] float64 (sigmoid outputs) and the hidden state."""
    x32 = _inputs(cam, means, latent, L)
    W1, b1, W2, b2 = unpack(weights, L, H)
    x = x32.astype(np.float64)
    z = W1 @ x + b1[:, None]
    act = _active(x32, weights, L, H)
    h = np.where(act, z, 0.0)
    y = W2 @ h + b2[:, None]
    rgb = 1.0 / (1.0 + np.exp(-y))
    return rgb, dict(x=x, z=z, act=act, h=h, y=y)


def backward(cam: dict, means, latent, weights, L: int, H: int, grad_rgb):
    """Returns grad_latent [L, n] and grad_weights (packed, as weights), float64."""
    rgb, st = forward(cam, means, latent, weights, L, H)
    W1, b1, W2, b2 = unpack(weights, L, H)
    g = np.asarray(grad_rgb, np.float64).reshape(3, -1)
    dy = g * rgb * (1.0 - rgb)               # through the sigmoid
    dW2 = dy @ st["h"].T                     # [3, H]
    db2 = dy.sum(axis=1)
    dh = W2.T @ dy                           # [H, n]
    dz = np.where(st["act"], dh, 0.0)        # through the ReLU
    dW1 = dz @ st["x"].T                     # [H, L+3]
    db1 = dz.sum(axis=1)
    dx = W1.T @ dz                           # [L+3, n]; the direction rows are dropped
    grad_w = np.concatenate([dW1.reshape(-1), db1, dW2.reshape(-1), db2])
    return dx[:L], grad_w
