"""GPU parity of the ellipse tile test (GS_TILES_ELLIPSE) against the
oracle's, and against the GPU's own square-span run: the preprocess,
tiles_touched, keys, sorted order, ranges and E bit-exact with the oracle;
the image and final_T bit-identical to the square-span run on the GPU when
each list is walked whole (the dropped tiles hold no pixel the splat
changes; the chunked forward groups T's product by list position, which the
shorter lists shift, so there the two agree to rounding); gradients within
the bar.
"""
import sys

import numpy as np
import pytest

import synth
from gpu_helpers import (assert_binning_equal, assert_preprocess_equal, compare_forward, compare_gradients,
                         gpu_backward, to_np)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _gpu_forward(cam, scene_np, tile_test, capacity=1 << 22, scheduled=None):
    import torch
    import gaussian_splatting_tile_amd as gs
    sc = gs.Scene.from_numpy(scene_np)
    r = gs.Rasterizer(capacity=capacity, tile_test=tile_test)
    out = r.forward(cam, sc, with_examined=True, scheduled=scheduled)
    torch.cuda.synchronize()
    res = {k: to_np(v) for k, v in out.items() if hasattr(v, "detach")}
    res["n_entries"] = out["n_entries"]
    res["keys"] = res["keys"].view(np.uint64)
    for k in ("point_list", "ranges", "tiles_touched", "n_contrib", "n_examined"):
        res[k] = res[k].view(np.uint32)
    return res, out, sc


@pytest.mark.parametrize("name", ["cfg0", "cfg1", "cfg2", "cfg3"])
def test_ellipse_forward_parity(orc, name):
    say(f"[ellipse {name}]")
    scene, cam, _ = synth.config_scene(name)
    o = orc.render_fwd(cam, scene, tile_test=1)
    g, _, _ = _gpu_forward(cam, scene, 1)
    assert_preprocess_equal(g, o)
    assert_binning_equal(g, o)
    rep = compare_forward(g, o)
    whole, _, _ = _gpu_forward(cam, scene, 1, scheduled=False)
    sq, _, _ = _gpu_forward(cam, scene, 0, scheduled=False)
    for k in ("image", "final_T"):
        assert whole[k].tobytes() == sq[k].tobytes(), k
    say(f"[ellipse {name}] E {sq['n_entries']} -> {g['n_entries']} {rep}")


def test_ellipse_backward_parity(orc):
    scene, cam, dLdI = synth.config_scene("cfg2")
    o = orc.render_fwd(cam, scene, tile_test=1)
    ob = orc.composite_bwd(cam, scene["n"], o["ranges"], o["point_list"], o["xy_depth"], o["conic_op"], o["rgb"],
                           o["final_T"], o["n_contrib"], dLdI, mass=True)
    g, out, sc = _gpu_forward(cam, scene, 1)
    grads = gpu_backward(cam, sc, out, dLdI)
    say("[ellipse cfg2 bwd]", compare_gradients(grads, ob))


def test_ellipse_small_and_ragged(orc):
    """Ragged images, SH degrees, huge and tiny splats, non-zero background."""
    for (W, H, n, deg, seed) in [(33, 17, 60, None, 1), (257, 129, 3000, 3, 2), (100, 75, 800, 1, 3)]:
        cam = synth.look_at_camera((0.2, -0.1, -4.0), (0.0, 0.0, 0.0), W, H, 0.6 * W, 0.6 * W)
        scene = synth.random_scene(n, seed, cam, sh_degree=deg, scale_lo=0.002, scale_hi=0.6, spread=1.5)
        o = orc.render_fwd(cam, scene, bg=(0.1, 0.2, 0.3), tile_test=1)
        import torch
        import gaussian_splatting_tile_amd as gs
        sc = gs.Scene.from_numpy(scene)
        r = gs.Rasterizer(capacity=1 << 18, tile_test=1)
        out = r.forward(cam, sc, bg=(0.1, 0.2, 0.3))
        torch.cuda.synchronize()
        g = {k: to_np(v) for k, v in out.items() if hasattr(v, "detach")}
        g["n_entries"] = out["n_entries"]
        g["keys"] = g["keys"].view(np.uint64)
        for k in ("point_list", "ranges", "tiles_touched", "n_contrib"):
            g[k] = g[k].view(np.uint32)
        assert_preprocess_equal(g, o)
        assert_binning_equal(g, o)
        compare_forward(g, o, (0.1, 0.2, 0.3))


def test_ellipse_async_views_match_blocking(orc):
    """The asynchronous binning with the ellipse test (as the batched views
    use it) gives the same keys and image as the blocking call."""
    import torch
    import gaussian_splatting_tile_amd as gs
    scene_np, _, _ = synth.config_scene("cfg4")
    cams = [synth.config_scene("cfg4", view=v)[1] for v in range(3)]
    sc = gs.Scene.from_numpy(scene_np)
    batch = gs.ViewBatch(cams, sc, capacity=1 << 21, streams=2, tile_test=1)
    batch.enqueue()
    E = batch.check()
    for i, cam in enumerate(cams):
        r = gs.Rasterizer(capacity=1 << 21, tile_test=1)
        out = r.forward(cam, sc)
        torch.cuda.synchronize()
        assert out["n_entries"] == E[i]
        v = batch.views[i]
        assert torch.equal(v["bins"].keys[:E[i]], out["keys"])
        assert torch.equal(v["fwd"]["image"], out["image"])
