"""GPU parity: the HIP path (through the C ABI and its binding) against the
oracle, on the seeded workloads and on edge cases.

Run on an MI355X:  python -m pytest tests -m gpu -x -v
"""
import sys

import numpy as np
import pytest

import synth
from gpu_helpers import (assert_binning_equal, assert_bits_equal, assert_preprocess_equal,
                         compare_forward, compare_gradients, gpu_backward, gpu_forward,
                         oracle_backward, oracle_forward)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="session", autouse=True)
def device():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    import gaussian_splatting_tile_amd as gs
    from gaussian_splatting_tile_amd import _lib
    _lib.load()
    say("device:", torch.cuda.get_device_name(0), "lib:", gs.LIB_PATH)
    return torch.device("cuda")


_cache = {}


def workload(orc, name):
    """(scene, cam, dLdI, oracle fwd, oracle bwd or None), cached per session."""
    if name not in _cache:
        scene, cam, dLdI = synth.config_scene(name)
        ofwd = oracle_forward(orc, cam, scene)
        obwd = oracle_backward(orc, cam, scene, ofwd, dLdI) if dLdI is not None else None
        _cache[name] = (scene, cam, dLdI, ofwd, obwd)
    return _cache[name]


@pytest.mark.parametrize("name", ["cfg0", "cfg1", "cfg2", "cfg3"])
def test_workload_forward_parity(orc, name):
    say(f"[{name}] forward parity")
    scene, cam, dLdI, ofwd, _ = workload(orc, name)
    g, out, sc, r = gpu_forward(cam, scene, capacity=1 << 16)
    assert_preprocess_equal(g, ofwd)
    assert_binning_equal(g, ofwd)
    rep = compare_forward(g, ofwd)
    say(f"[{name}] E={g['n_entries']} evals={int(g['n_examined'].sum())} oracle_evals={int(ofwd['n_examined'].sum())} {rep}")


@pytest.mark.parametrize("name", ["cfg2", "cfg3"])
def test_workload_backward_parity(orc, name):
    say(f"[{name}] backward parity")
    scene, cam, dLdI, ofwd, obwd = workload(orc, name)
    g, out, sc, r = gpu_forward(cam, scene, capacity=1 << 22)
    grads = gpu_backward(cam, sc, out, dLdI)
    rep = compare_gradients(grads, obwd)
    say(f"[{name}] end-to-end grads {rep}")
    # stage-isolated: the oracle's forward state fed to the GPU backward
    iso = gpu_backward(cam, sc, out, dLdI, final_T=ofwd["final_T"], n_contrib=ofwd["n_contrib"])
    rep2 = compare_gradients(iso, obwd)
    say(f"[{name}] isolated grads {rep2}")


def test_multiview_training_shape(orc):
    """Three of the sixteen 400x400 views over 300k Gaussians, dL/dI = sign(I - I_ref)
    with I and I_ref from the oracle."""
    import gaussian_splatting_tile_amd as gs
    rast = gs.Rasterizer(capacity=1 << 20)
    for view in (0, 7, 15):
        say(f"[cfg4 view {view}]")
        scene, cam, _ = synth.config_scene("cfg4", view)
        ref_scene, _, _ = synth.config_scene("cfg4_ref", view)
        ofwd = oracle_forward(orc, cam, scene)
        oref = oracle_forward(orc, cam, ref_scene)
        dLdI = np.sign(ofwd["image"] - oref["image"]).astype(np.float32)
        obwd = oracle_backward(orc, cam, scene, ofwd, dLdI)
        g, out, sc, _ = gpu_forward(cam, scene, rast=rast)
        assert_preprocess_equal(g, ofwd)
        assert_binning_equal(g, ofwd)
        compare_forward(g, ofwd)
        compare_gradients(gpu_backward(cam, sc, out, dLdI), obwd)


def _random_case(orc, W, H, n, seed, sh_degree=None, bg=(0.0, 0.0, 0.0), **kw):
    cam = synth.look_at_camera((0.3, -0.2, -4.0), (0.0, 0.1, 0.0), W, H, 0.9 * W, 0.9 * W)
    scene = synth.random_scene(n, seed, cam, sh_degree=sh_degree, **kw)
    return cam, scene


@pytest.mark.parametrize("W,H,n,deg", [(33, 17, 50, None), (1, 1, 10, 0), (64, 48, 300, 1),
                                       (100, 75, 800, 2), (257, 129, 2000, 3), (4001, 23, 3000, 3)])
def test_ragged_and_sh_degrees(orc, W, H, n, deg):
    say(f"[random {W}x{H} n={n} deg={deg}]")
    cam, scene = _random_case(orc, W, H, n, seed=W + H + n, sh_degree=deg, spread=1.4)
    bg = (0.2, 0.1, 0.3)
    ofwd = oracle_forward(orc, cam, scene, bg)
    g, out, sc, _ = gpu_forward(cam, scene, bg=bg, capacity=64)  # forces the capacity retry
    assert_preprocess_equal(g, ofwd)
    assert_binning_equal(g, ofwd)
    compare_forward(g, ofwd)
    dLdI = synth.upstream_gradient(n, W, H)
    obwd = oracle_backward(orc, cam, scene, ofwd, dLdI, bg)
    compare_gradients(gpu_backward(cam, sc, out, dLdI, bg), obwd)


def test_empty_and_fully_culled(orc):
    import gaussian_splatting_tile_amd as gs
    import torch
    cam = synth.look_at_camera((0, 0, -4), (0, 0, 0), 40, 24, 40.0, 40.0)
    # all Gaussians behind the camera
    scene = synth.random_scene(100, 1, cam)
    scene["means"] = np.ascontiguousarray(scene["means"] * np.float32(-1) - np.float32([[0], [0], [9]]))
    ofwd = oracle_forward(orc, cam, scene, bg=(0.5, 0.25, 1.0))
    assert ofwd["keys"].shape[0] == 0
    g, out, sc, _ = gpu_forward(cam, scene, bg=(0.5, 0.25, 1.0))
    assert g["n_entries"] == 0 and not g["tiles_touched"].any()
    assert (g["ranges"] == 0).all()
    np.testing.assert_array_equal(g["image"], ofwd["image"])
    assert (g["final_T"] == 1).all() and not g["n_contrib"].any()
    grads = gpu_backward(cam, sc, out, synth.upstream_gradient(0, 40, 24))
    for v in grads.values():
        assert not v.any()
    # n = 0 through every stage
    empty = dict(n=0, means=np.zeros((3, 0), np.float32), scales=np.zeros((3, 0), np.float32),
                 quats=np.zeros((4, 0), np.float32), opacity=np.zeros(0, np.float32),
                 rgb=np.zeros((3, 0), np.float32), sh=None, sh_degree=0)
    g0, out0, sc0, _ = gpu_forward(cam, empty)
    assert g0["n_entries"] == 0 and (g0["final_T"] == 1).all()


def test_non_finite_and_boundary_inputs(orc):
    cam = synth.look_at_camera((0, 0, -4), (0, 0, 0), 64, 64, 64.0, 64.0)
    scene = synth.random_scene(400, 5, cam, sh_degree=3)
    nan, inf = np.float32("nan"), np.float32("inf")
    scene["means"][0, 0] = nan
    scene["scales"][1, 1] = inf
    scene["scales"][2, 2] = nan
    scene["quats"][:, 3] = 0
    scene["opacity"][4] = nan
    scene["sh"][5, 1, 5] = inf
    # centre exactly on the near plane and one ulp beyond it
    R = np.asarray(cam["R"], np.float64).reshape(3, 3)
    for g, z in ((6, np.float32(0.05)), (7, np.nextafter(np.float32(0.05), np.float32(1)))):
        scene["means"][:, g] = (R.T @ (np.array([0.0, 0.0, float(z)]) - cam["t"].astype(np.float64))).astype(np.float32)
    # very large splat covering the whole screen
    scene["scales"][:, 8] = 5.0
    ofwd = oracle_forward(orc, cam, scene)
    assert ofwd["tiles_touched"][:6].sum() == 0
    g, out, sc, _ = gpu_forward(cam, scene)
    assert_preprocess_equal(g, ofwd)
    assert_binning_equal(g, ofwd)
    compare_forward(g, ofwd)


def test_equal_depth_ties_keep_index_order(orc):
    """A fronto-parallel sheet: every Gaussian has the same depth bits, so the
    tile lists are ordered by Gaussian index alone."""
    cam = dict(R=np.eye(3, dtype=np.float32).reshape(9), t=np.zeros(3, np.float32),
               campos=np.zeros(3, np.float32), fx=np.float32(50), fy=np.float32(50),
               cx=np.float32(48), cy=np.float32(40), width=96, height=80)
    rng = np.random.default_rng(3)
    n = 3000
    means = np.stack([rng.uniform(-1, 1, n), rng.uniform(-0.9, 0.9, n), np.full(n, 1.0)]).astype(np.float32)
    scene = dict(n=n, means=means, scales=np.full((3, n), 0.01, np.float32),
                 quats=np.tile(np.float32([[1], [0], [0], [0]]), (1, n)),
                 opacity=rng.uniform(0.1, 0.9, n).astype(np.float32),
                 rgb=rng.uniform(0, 1, (3, n)).astype(np.float32), sh=None, sh_degree=0)
    ofwd = oracle_forward(orc, cam, scene)
    vis = ofwd["tiles_touched"] > 0
    assert vis.sum() > 2000 and (ofwd["xy_depth"][vis, 2] == 1.0).all()
    g, out, sc, _ = gpu_forward(cam, scene)
    assert_binning_equal(g, ofwd)
    compare_forward(g, ofwd)


def test_repeat_runs_are_bit_identical(orc):
    scene, cam, dLdI, ofwd, _ = workload(orc, "cfg1")
    a, _, _, r = gpu_forward(cam, scene)
    b, _, _, _ = gpu_forward(cam, scene, rast=r)
    for k in ("xy_depth", "conic_op", "rgb", "tiles_touched", "keys", "point_list", "ranges",
              "image", "final_T", "n_contrib", "n_examined"):
        assert_bits_equal(a[k], b[k], k)


def _async_forward(cam, scene, capacity, bg=(0.0, 0.0, 0.0)):
    """Preprocess, asynchronous binning and ranges, forward compositing: no
    host wait until the results are read."""
    import gaussian_splatting_tile_amd as gs
    import torch
    from gpu_helpers import to_np
    sc = gs.Scene.from_numpy(scene)
    c = gs.camera(cam)
    bins = gs.BinBuffers(torch.device("cuda"), capacity=capacity)
    pre = gs.preprocess(c, sc.means, sc.scales, sc.quats, sc.opacity, sc.sh, sc.sh_degree, sc.rgb)
    keys, pl = gs.bin_and_sort_async(c, pre["xy_depth"], pre["tiles_touched"], bins)
    ranges = gs.tile_ranges_async(c, bins)
    fwd = gs.composite_fwd(c, ranges, pl, pre["xy_depth"], pre["conic_op"], pre["rgb"], bg)
    E = bins.entries()
    res = {k: to_np(v) for k, v in fwd.items()}
    res.update(n_entries=E, ranges=to_np(ranges).view(np.uint32),
               keys=to_np(keys).view(np.uint64), point_list=to_np(pl).view(np.uint32))
    return res


@pytest.mark.parametrize("W,H,n,seed", [(257, 129, 2000, 11), (720, 720, 20000, 12)])
def test_async_binning_matches_oracle(orc, W, H, n, seed):
    say(f"[async {W}x{H} n={n}]")
    cam, scene = _random_case(orc, W, H, n, seed=seed, sh_degree=1, spread=1.4)
    ofwd = oracle_forward(orc, cam, scene)
    E = int(ofwd["keys"].shape[0])
    res = _async_forward(cam, scene, capacity=E + 4097)
    assert res["n_entries"] == E
    assert_bits_equal(res["keys"][:E], ofwd["keys"], "keys")
    assert_bits_equal(res["point_list"][:E], ofwd["point_list"], "point_list")
    assert_bits_equal(res["ranges"], ofwd["ranges"], "ranges")
    assert (res["n_contrib"] == ofwd["n_contrib"]).mean() >= 0.999
    np.testing.assert_allclose(res["image"], ofwd["image"], atol=1e-4, rtol=0)


def test_async_overflow_renders_background(orc):
    """E > capacity: nothing is binned, every tile is empty, the image is the
    background and E is still reported."""
    cam, scene = _random_case(orc, 257, 129, 2000, seed=11, sh_degree=1, spread=1.4)
    ofwd = oracle_forward(orc, cam, scene)
    E = int(ofwd["keys"].shape[0])
    bg = (0.25, 0.5, 0.75)
    res = _async_forward(cam, scene, capacity=E // 2, bg=bg)
    assert res["n_entries"] == E
    assert not res["ranges"].any()
    assert (res["final_T"] == 1).all() and not res["n_contrib"].any()
    for ch in range(3):
        assert (res["image"][ch] == np.float32(bg[ch])).all()


def test_async_empty_scene():
    import gaussian_splatting_tile_amd as gs
    import torch
    cam = synth.look_at_camera((0, 0, -4), (0, 0, 0), 40, 24, 40.0, 40.0)
    c = gs.camera(cam)
    bins = gs.BinBuffers(torch.device("cuda"), capacity=1024)
    bins.n_entries_dev.fill_(12345)
    z = torch.zeros((0, 4), dtype=torch.float32, device="cuda")
    t = torch.zeros((0,), dtype=torch.int32, device="cuda")
    gs.bin_and_sort_async(c, z, t, bins)
    ranges = gs.tile_ranges_async(c, bins)
    assert bins.entries() == 0
    assert not ranges.any()


def test_tile_order_is_a_heaviest_first_schedule(orc):
    """The schedule from the ranges call is a permutation of the tiles in
    non-increasing length class, and rendering in it gives bit-identical
    forward results and equal gradients to tile-id order."""
    import gaussian_splatting_tile_amd as gs
    import torch
    from gpu_helpers import to_np
    scene, cam, dLdI, ofwd, obwd = workload(orc, "cfg2")
    g, out, sc, r = gpu_forward(cam, scene, capacity=1 << 22)
    order = to_np(out["tile_order"]).view(np.uint32).astype(np.int64)
    n_tiles = g["ranges"].shape[0]
    assert np.array_equal(np.sort(order), np.arange(n_tiles))
    L = (g["ranges"][:, 1].astype(np.int64) - g["ranges"][:, 0])[order]
    # length classes: 16 linear steps per octave (the 4 bits below the
    # leading one), empty tiles lowest; they never increase along the schedule
    msb = np.floor(np.log2(np.maximum(L, 1))).astype(np.int64)
    frac = ((L << (31 - msb)) >> 27) & 15
    cls = np.where(L == 0, -1, np.minimum(255, 1 + 16 * msb + frac))
    assert (np.diff(cls) <= 0).all()
    assert L[0] >= L.max() // 2
    c = gs.camera(cam)
    plain = gs.composite_fwd(c, out["ranges"], out["point_list"], out["xy_depth"], out["conic_op"], out["rgb"])
    torch.cuda.synchronize()
    for k in ("image", "final_T", "n_contrib"):
        assert_bits_equal(to_np(plain[k]), g[k], k)
    grads = gpu_backward(cam, sc, out, dLdI)
    ordered = gs.composite_bwd(c, sc.n, out["ranges"], out["point_list"], out["xy_depth"], out["conic_op"],
                               out["rgb"], out["final_T"], out["n_contrib"],
                               torch.from_numpy(np.ascontiguousarray(dLdI, np.float32)).cuda(),
                               order=out["tile_order"])
    torch.cuda.synchronize()
    compare_gradients({k: to_np(v).astype(np.float64) for k, v in ordered.items()}, obwd)
    compare_gradients(grads, obwd)
