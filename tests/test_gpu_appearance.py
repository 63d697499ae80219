"""GPU parity of the appearance MLP (gs_appearance_fwd / gs_appearance_bwd)
against the oracle (oracle/appearance.py), at three sizes and at the
300k-Gaussian training shape, and end to end through the rasterizer
(colours from the MLP as rgb_in, gradients back to latents and weights).

Bar: colours within 1e-5 absolute; every gradient group (latents, W1, b1,
W2, b2) max|gpu - oracle| / max|oracle| <= 1e-3; weight gradients
bit-identical between two runs (fixed summation order).
"""
import sys

import numpy as np
import pytest

import synth
from gpu_helpers import GRAD_REL, to_np
from oracle import appearance as app

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _inputs(seed, n, L, H):
    rng = np.random.default_rng(seed)
    means = rng.normal(0, 1.0, (3, n)).astype(np.float32)
    latent = rng.normal(0, 1.0, (L, n)).astype(np.float32)
    w = rng.normal(0, 1.0 / np.sqrt(L + 3), app.n_params(L, H)).astype(np.float32)
    g = rng.normal(0, 1.0, (3, n)).astype(np.float32)
    return means, latent, w, g


def _groups(dw, L, H):
    W1, b1, W2, b2 = app.unpack(dw, L, H)
    return dict(W1=W1, b1=b1, W2=W2, b2=b2)


def _check(g_lat, g_w, o_lat, o_w, L, H):
    rep = {}
    pairs = dict(latent=(g_lat, o_lat))
    gg, og = _groups(g_w, L, H), _groups(o_w, L, H)
    for k in gg:
        pairs[k] = (gg[k], og[k])
    for k, (a, b) in pairs.items():
        scale = max(np.abs(b).max(), 1e-30)
        err = np.abs(a - b).max()
        rep[k] = (float(err), float(scale))
        assert err <= GRAD_REL * scale, (k, err, scale)
    return rep


@pytest.mark.parametrize("L,H,n", [(8, 32, 10000), (2, 5, 3001), (29, 64, 5000), (8, 32, 300000)])
def test_appearance_parity(L, H, n):
    import torch
    import gaussian_splatting_tile_amd as gs
    say(f"[appearance L={L} H={H} n={n}]")
    cam = synth.view_camera(4000, 4.0, 400, 400, 400.0)
    means, latent, w, g = _inputs(L * 1000 + H, n, L, H)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    rgb = gs.appearance_fwd(cam, t(means), t(latent), t(w), H)
    out = gs.appearance_bwd(cam, t(means), t(latent), t(w), H, t(g))
    out2 = gs.appearance_bwd(cam, t(means), t(latent), t(w), H, t(g))
    torch.cuda.synchronize()
    o_rgb, _ = app.forward(cam, means, latent, w, L, H)
    err = np.abs(to_np(rgb) - o_rgb).max()
    assert err <= 1e-5, err
    o_lat, o_w = app.backward(cam, means, latent, w, L, H, g)
    rep = _check(to_np(out["grad_latent"]).astype(np.float64), to_np(out["grad_weights"]).astype(np.float64),
                 o_lat, o_w, L, H)
    assert torch.equal(out["grad_weights"], out2["grad_weights"])  # deterministic
    say(f"[appearance L={L} H={H} n={n}] rgb err {err:.2e} {rep}")


@pytest.mark.parametrize("L,H", [(1, 1), (5, 7), (9, 16), (13, 33), (17, 20), (21, 64), (25, 3), (29, 64),
                                 (3, 9), (12, 1)])
def test_appearance_every_input_width(L, H):
    """The kernels are specialised on the input count L + 3 rounded up to a
    multiple of 4 (1..8 groups of four): every specialisation, with exact
    and padded widths, odd hidden widths and a ragged last workgroup."""
    import torch
    import gaussian_splatting_tile_amd as gs
    n = 1000 + 37 * L + H
    cam = synth.view_camera(4001, 4.0, 300, 200, 300.0)
    means, latent, w, g = _inputs(7 * L + H, n, L, H)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    rgb = gs.appearance_fwd(cam, t(means), t(latent), t(w), H)
    out = gs.appearance_bwd(cam, t(means), t(latent), t(w), H, t(g))
    torch.cuda.synchronize()
    o_rgb, _ = app.forward(cam, means, latent, w, L, H)
    err = np.abs(to_np(rgb) - o_rgb).max()
    assert err <= 1e-5, err
    o_lat, o_w = app.backward(cam, means, latent, w, L, H, g)
    rep = _check(to_np(out["grad_latent"]).astype(np.float64), to_np(out["grad_weights"]).astype(np.float64),
                 o_lat, o_w, L, H)
    say(f"[appearance width L={L} H={H} n={n}] rgb err {err:.2e} {rep}")


def test_appearance_through_the_rasterizer(orc):
    """MLP colours -> preprocess(rgb_in) -> render -> backward ->
    preprocess_bwd (grad_rgb_in) -> appearance_bwd, against the same chain
    in the oracle."""
    import torch
    import gaussian_splatting_tile_amd as gs
    L, H = 8, 32
    cam = synth.look_at_camera((0.2, -0.1, -4.0), (0.0, 0.0, 0.0), 160, 120, 120.0, 120.0)
    scene = synth.random_scene(3000, 17, cam, sh_degree=None, scale_lo=0.01, scale_hi=0.2, spread=1.2)
    n = scene["n"]
    rng = np.random.default_rng(5)
    latent = rng.normal(0, 1.0, (L, n)).astype(np.float32)
    w = rng.normal(0, 0.3, app.n_params(L, H)).astype(np.float32)
    dLdI = synth.upstream_gradient(23, cam["width"], cam["height"])
    # oracle chain
    o_rgb, _ = app.forward(cam, scene["means"], latent, w, L, H)
    s_o = dict(scene)
    s_o["rgb"] = o_rgb.astype(np.float32)
    of = orc.render_fwd(cam, s_o)
    ob = orc.composite_bwd(cam, n, of["ranges"], of["point_list"], of["xy_depth"], of["conic_op"], of["rgb"],
                           of["final_T"], of["n_contrib"], dLdI)
    op = orc.preprocess_bwd(cam, s_o, ob["grad_mean2d"], ob["grad_conic_op"], ob["grad_rgb"])
    o_lat, o_w = app.backward(cam, scene["means"], latent, w, L, H, op["grad_rgb_in"])
    # GPU chain
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    sc = gs.Scene.from_numpy(scene)
    lat_d, w_d = t(latent), t(w)
    sc.rgb = gs.appearance_fwd(cam, sc.means, lat_d, w_d, H)
    r = gs.Rasterizer(capacity=1 << 18)
    out = r.forward(cam, sc)
    grads = r.backward(cam, sc, out, t(dLdI), to_parameters=True)
    ga = gs.appearance_bwd(cam, sc.means, lat_d, w_d, H, grads["grad_rgb_in"])
    torch.cuda.synchronize()
    img_err = np.abs(to_np(out["image"]) - of["image"]).max()
    assert img_err <= 1e-4, img_err
    rep = _check(to_np(ga["grad_latent"]).astype(np.float64), to_np(ga["grad_weights"]).astype(np.float64),
                 o_lat, o_w, L, H)
    say(f"[appearance chain] image err {img_err:.2e} {rep}")


def test_appearance_zero_gaussians():
    import torch
    import gaussian_splatting_tile_amd as gs
    L, H = 8, 32
    cam = synth.view_camera(4000, 4.0, 400, 400, 400.0)
    e = torch.empty((3, 0), device="cuda")
    w = torch.ones(app.n_params(L, H), device="cuda")
    out = dict(grad_latent=torch.empty((L, 0), device="cuda"), grad_weights=torch.full_like(w, 7.0))
    gs.appearance_bwd(cam, e, torch.empty((L, 0), device="cuda"), w, H, e, out=out)
    torch.cuda.synchronize()
    assert not out["grad_weights"].any()
