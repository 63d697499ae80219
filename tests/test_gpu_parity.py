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
                         oracle_backward, oracle_forward, to_np)

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
    # lists walked in 256-entry chunks from the forward's checkpoints
    rep_c = compare_gradients(gpu_backward(cam, sc, out, dLdI, chunked=True), obwd)
    say(f"[{name}] chunked grads {rep_c}")
    # stage-isolated: the oracle's forward state fed to the GPU backward
    iso = gpu_backward(cam, sc, out, dLdI, final_T=ofwd["final_T"], n_contrib=ofwd["n_contrib"])
    rep2 = compare_gradients(iso, obwd)
    say(f"[{name}] isolated grads {rep2}")


@pytest.mark.parametrize("name", ["cfg2", "cfg3"])
def test_scheduled_forward_parity(orc, name):
    """The forward over the chunk schedule at 1080p: cfg3's lists average
    more than 256 entries, so they are composited in chunks and most pixels
    stop inside one, composited again from the combined state; cfg2's are
    whole items. Both against the oracle, with the chunked backward from
    that forward's state."""
    say(f"[{name}] scheduled forward")
    scene, cam, dLdI, ofwd, obwd = workload(orc, name)
    g, out, sc, r = gpu_forward(cam, scene, capacity=1 << 23, scheduled=True)
    rep = compare_forward(g, ofwd)
    stopped = ofwd["final_T"] < 1e-4
    say(f"[{name}] scheduled forward {rep}, pixels stopped {int(stopped.sum())}")
    if name == "cfg3":
        assert stopped.sum() > 100_000  # the re-walk path is exercised (12% of the pixels stop)
    rep_b = compare_gradients(gpu_backward(cam, sc, out, dLdI, chunked=True), obwd)
    say(f"[{name}] chunked backward after it {rep_b}")


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
        compare_gradients(gpu_backward(cam, sc, out, dLdI, chunked=True), obwd)


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
    compare_forward(g, ofwd, bg)
    dLdI = synth.upstream_gradient(n, W, H)
    obwd = oracle_backward(orc, cam, scene, ofwd, dLdI, bg)
    compare_gradients(gpu_backward(cam, sc, out, dLdI, bg), obwd)
    compare_gradients(gpu_backward(cam, sc, out, dLdI, bg, chunked=True), obwd)


def _sweep_case(seed):
    """A seeded random (camera, scene, background, tile test) drawn over the
    edges of the path: ragged image sizes down to one pixel, SH degrees 0-3
    or direct colours, means from behind the near plane to far away and up
    to three frames off-screen, scales from sub-pixel to larger than the
    image with random anisotropy, opacities at the 1/255 floor, ordinary, or
    saturating at 0.99, and either tile test."""
    rng = np.random.default_rng(7000 + seed)
    W = [1, 7, 16, 17, 31, 64, 97, 160, 255, 333][seed % 10]
    H = [1, 5, 16, 23, 48, 100, 129, 200, 257][(4 * seed) % 9]
    while True:
        eye = rng.normal(0.0, 1.0, 3)
        eye *= rng.uniform(2.5, 6.0) / np.linalg.norm(eye)
        target = rng.normal(0.0, 0.3, 3)
        d = (target - eye) / np.linalg.norm(target - eye)
        if abs(d[1]) < 0.9:  # the camera's up vector is +y
            break
    f = float(rng.uniform(0.5, 2.0)) * max(W, H)
    cam = synth.look_at_camera(tuple(eye), tuple(target), W, H, f, f * float(rng.uniform(0.8, 1.25)))
    n = int(rng.choice([1, 5, 60, 500, 2000, 4000]))
    deg = [None, 0, 1, 2, 3][seed % 5]
    scale_lo, scale_hi = [(0.001, 0.01), (0.01, 0.3), (0.001, 1.0), (0.2, 2.0)][int(rng.integers(4))]
    op_lo, op_hi = [(0.002, 0.01), (0.05, 0.99), (0.9, 1.0)][int(rng.integers(3))]
    depth_lo = float(rng.choice([0.05, 0.5, 1.0]))
    scene = synth.random_scene(n, 7000 + seed, cam, sh_degree=deg, scale_lo=scale_lo, scale_hi=scale_hi,
                               op_lo=op_lo, op_hi=op_hi, depth_lo=depth_lo,
                               depth_hi=depth_lo + float(rng.uniform(0.5, 8.0)),
                               spread=float(rng.choice([0.5, 1.2, 3.0])))
    bg = tuple(float(x) for x in rng.uniform(0.0, 1.0, 3))
    return cam, scene, bg, int(rng.integers(2)), dict(W=W, H=H, n=n, deg=deg, scales=(scale_lo, scale_hi),
                                                       opacity=(op_lo, op_hi), depth_lo=depth_lo)


@pytest.mark.parametrize("seed", range(16))
def test_random_scene_sweep(orc, seed):
    """Every stage against the oracle on a seeded random case (see
    _sweep_case): preprocess and binning bit-exact, the forward (whole lists
    and over the chunk schedule) and both backward forms within the bar."""
    import gaussian_splatting_tile_amd as gs
    cam, scene, bg, tile_test, desc = _sweep_case(seed)
    say(f"[sweep {seed}] tile_test={tile_test} {desc}")
    ofwd = orc.render_fwd(cam, scene, bg=bg, tile_test=tile_test)
    rast = gs.Rasterizer(capacity=64, tile_test=tile_test)  # small: forces the capacity retry
    g, out, sc, _ = gpu_forward(cam, scene, bg=bg, rast=rast)
    assert_preprocess_equal(g, ofwd)
    assert_binning_equal(g, ofwd)
    rep = compare_forward(g, ofwd, bg)
    say(f"[sweep {seed}] E={g['n_entries']} {rep}")
    dLdI = synth.upstream_gradient(seed + 11, cam["width"], cam["height"])
    obwd = oracle_backward(orc, cam, scene, ofwd, dLdI, bg)
    compare_gradients(gpu_backward(cam, sc, out, dLdI, bg), obwd)
    compare_gradients(gpu_backward(cam, sc, out, dLdI, bg, chunked=True), obwd)
    g2, out2, sc2, _ = gpu_forward(cam, scene, bg=bg, rast=rast, scheduled=True)
    compare_forward(g2, ofwd, bg)
    compare_gradients(gpu_backward(cam, sc2, out2, dLdI, bg, chunked=True), obwd)


def test_depth_order_with_a_large_tie_cluster(orc):
    """100,000 splats of which all but 2,048 (those at indices j N / 2048)
    share one depth, the others spread in front and behind: one run of about
    98,000 equal depth keys, spread over every workgroup of every depth pass,
    must come out in index order among spread keys, as the oracle's stable
    sort puts them."""
    n, W, H = 100_000, 256, 256
    cam = synth.look_at_camera((0.0, 0.0, -4.0), (0.0, 0.0, 0.0), W, H, 200.0, 200.0)
    rng = np.random.default_rng(17)
    sampled = (np.arange(2048, dtype=np.int64) * n) // 2048
    z = np.full(n, 1.0, np.float64)  # world z: depth 5 from the camera
    z[sampled] = rng.uniform(-2.0, 4.0, sampled.size)
    xy = rng.uniform(-0.55, 0.55, (2, n)) * (z + 4.0)  # inside the frame at each depth
    scene = synth.random_scene(n, 18, cam, scale_lo=0.002, scale_hi=0.006)
    scene["means"] = np.ascontiguousarray(np.stack([xy[0], xy[1], z]).astype(np.float32))
    ofwd = oracle_forward(orc, cam, scene)
    depth = ofwd["xy_depth"][2] if ofwd["xy_depth"].shape[0] == 4 else ofwd["xy_depth"][:, 2]
    say(f"[tie cluster] E={ofwd['keys'].shape[0]} distinct depths={np.unique(depth).size}")
    g, out, sc, _ = gpu_forward(cam, scene, capacity=1 << 20)
    assert_preprocess_equal(g, ofwd)
    assert_binning_equal(g, ofwd)
    compare_forward(g, ofwd)


def test_alpha_floor_decisions_match_exactly(orc):
    """The compositing kernels decide alpha >= 1/255 on the oracle's number
    (the correctly rounded exponential near the floor): single splats over
    one 16 x 16 tile, opacities chosen so that many pixels' alpha lies
    within a few ulp of the floor. n_contrib must match the oracle on every
    pixel, and T and the image to float32 rounding."""
    import math
    import torch
    import gaussian_splatting_tile_amd as gs
    cam = synth.look_at_camera((0, 0, -4), (0, 0, 0), 16, 16, 16.0, 16.0)
    rng = np.random.default_rng(23)
    dev = torch.device("cuda")
    ranges = torch.tensor([[0, 1]], dtype=torch.int32, device=dev)
    point_list = torch.zeros((1,), dtype=torch.int32, device=dev)
    near = 0
    for case in range(300):
        u, v = rng.uniform(2.0, 14.0, 2)
        A, C = np.exp(rng.uniform(np.log(0.02), np.log(1.0), 2))
        B = rng.uniform(-0.8, 0.8) * math.sqrt(A * C)
        # an opacity that puts the floor crossing at a random pixel's power
        px, py = rng.integers(0, 16, 2)
        dx, dy = px - u, py - v
        power = -0.5 * (A * dx * dx + C * dy * dy) - B * dx * dy
        o = min(1.0, (1.0 / 255.0) / math.exp(power) * (1.0 + rng.uniform(-3e-7, 3e-7)))
        xy = np.array([[u, v, 5.0, 20.0]], np.float32)
        co = np.array([[A, B, C, o]], np.float32)
        rgb = np.array([[0.2, 0.5, 0.8, 0.0]], np.float32)
        ref = orc.composite_fwd(cam, np.array([[0, 1]], np.uint32), np.array([0], np.uint32), xy, co, rgb)
        out = gs.composite_fwd(cam, ranges, point_list, torch.from_numpy(xy).to(dev), torch.from_numpy(co).to(dev),
                               torch.from_numpy(rgb).to(dev))
        torch.cuda.synchronize()
        nc = to_np(out["n_contrib"]).view(np.uint32)
        np.testing.assert_array_equal(nc, ref["n_contrib"], err_msg=f"case {case}")
        np.testing.assert_allclose(to_np(out["final_T"]), ref["final_T"], rtol=0, atol=2e-7)
        np.testing.assert_allclose(to_np(out["image"]), ref["image"], rtol=0, atol=2e-7)
        a = ref["final_T"]
        near += int((np.abs((1.0 - a[a < 1]) * 255.0 - 1.0) < 1e-5).sum())
    say(f"[alpha floor] pixels with alpha within 1e-5 of 1/255: {near}")
    assert near >= 50  # the cases do probe the floor


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
    for chunked in (False, True):
        grads = gpu_backward(cam, sc, out, synth.upstream_gradient(0, 40, 24), chunked=chunked)
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


def _sheet_camera(W, H):
    return dict(R=np.eye(3, dtype=np.float32).reshape(9), t=np.zeros(3, np.float32),
                campos=np.zeros(3, np.float32), fx=np.float32(50), fy=np.float32(50),
                cx=np.float32(W / 2), cy=np.float32(H / 2), width=W, height=H)


def _tile_confined_scene(cam, counts, opacity, seed):
    """counts[t] splats of projected sigma <= 0.8 px (radius 3) centred in tile
    t's interior of the top tile row, so each touches that tile alone and its
    list holds exactly counts[t] entries; depths in [1, 1.5]."""
    rng = np.random.default_rng(seed)
    fx, cx, cy = float(cam["fx"]), float(cam["cx"]), float(cam["cy"])
    cols = []
    for t, k in enumerate(counts):
        z = rng.uniform(1.0, 1.5, k)
        u = 16 * t + rng.uniform(4.0, 12.0, k)
        v = rng.uniform(4.0, 12.0, k)
        cols.append(np.stack([(u - cx) * z / fx, (v - cy) * z / fx, z]))
    means = np.concatenate(cols, axis=1).astype(np.float32)
    n = means.shape[1]
    return dict(n=n, means=means, scales=np.full((3, n), 0.016, np.float32),
                quats=np.tile(np.float32([[1], [0], [0], [0]]), (1, n)),
                opacity=rng.uniform(*opacity, n).astype(np.float32),
                rgb=rng.uniform(0, 1, (3, n)).astype(np.float32), sh=None, sh_degree=0)


def _block_confined_scene(cam, counts, seed, opacity=(0.02, 0.15)):
    """counts[(bx, by)] splats centred within 0.25 px of the centre of 4 x 4
    pixel block (bx, by) of the top-left 16 x 16 tile, small and faint enough
    (projected sigma <= 0.62 px with the 0.3 px^2 dilation, opacity <= 0.15:
    alpha >= 1/255 within 1.8 px) to reach no pixel outside that block;
    depths in [1, 1.5]."""
    rng = np.random.default_rng(seed)
    fx, cx, cy = float(cam["fx"]), float(cam["cx"]), float(cam["cy"])
    cols = []
    for (bx, by), k in sorted(counts.items()):
        z = rng.uniform(1.0, 1.5, k)
        u = 4 * bx + 1.5 + rng.uniform(-0.25, 0.25, k)
        v = 4 * by + 1.5 + rng.uniform(-0.25, 0.25, k)
        cols.append(np.stack([(u - cx) * z / fx, (v - cy) * z / fx, z]))
    means = np.concatenate(cols, axis=1).astype(np.float32)
    n = means.shape[1]
    perm = rng.permutation(n)  # blocks interleaved in index order too
    return dict(n=n, means=np.ascontiguousarray(means[:, perm]), scales=np.full((3, n), 0.006, np.float32),
                quats=np.tile(np.float32([[1], [0], [0], [0]]), (1, n)),
                opacity=rng.uniform(*opacity, n).astype(np.float32),
                rgb=rng.uniform(0, 1, (3, n)).astype(np.float32), sh=None, sh_degree=0)


@pytest.mark.parametrize("case", ["uneven", "one_block"])
def test_forward_quarters_with_uneven_lists(orc, case):
    """The forward walks, per 16-lane quarter (one 4 x 4 block), only the
    splats that reach its block. One tile whose sixteen blocks get very
    different counts (0 to 300, around multiples of the three-splat step,
    of 64 and of the 256-splat batch), so within a wave one quarter runs
    out or stops long before another; and one whose splats all sit in a
    single block. Forward and both backward forms against the oracle."""
    if case == "uneven":
        ks = [0, 1, 2, 3, 5, 63, 64, 65, 130, 255, 256, 257, 300, 7, 0, 11]
        counts = {(b % 4, b // 4): k for b, k in enumerate(ks) if k}
    else:
        counts = {(2, 1): 700}
    cam = _sheet_camera(32, 32)
    scene = _block_confined_scene(cam, counts, seed=len(counts) + 41)
    say(f"[block-confined {case}: n={scene['n']}]")
    bg = (0.1, 0.2, 0.3)
    ofwd = oracle_forward(orc, cam, scene, bg)
    assert ofwd["keys"].shape[0] >= scene["n"]  # every splat listed (some in two tiles)
    g, out, sc, _ = gpu_forward(cam, scene, bg=bg)
    assert_binning_equal(g, ofwd)
    compare_forward(g, ofwd, bg)
    # every pixel outside the loaded blocks of tile (0, 0) keeps the background
    img = np.asarray(g["image"])
    mask = np.zeros((32, 32), bool)
    for (bx, by) in counts:
        mask[4 * by:4 * by + 4, 4 * bx:4 * bx + 4] = True
    np.testing.assert_array_equal(img[:, ~mask], np.broadcast_to(np.float32(bg)[:, None], (3, int((~mask).sum()))))
    dLdI = synth.upstream_gradient(scene["n"] + 7, 32, 32)
    obwd = oracle_backward(orc, cam, scene, ofwd, dLdI, bg)
    compare_gradients(gpu_backward(cam, sc, out, dLdI, bg), obwd)
    compare_gradients(gpu_backward(cam, sc, out, dLdI, bg, chunked=True), obwd)


def test_chunked_backward_at_list_boundaries(orc):
    """The chunked backward on lists of 512 (a multiple of the chunk), 257 and
    255 entries, the last tile ragged (40 px wide), and on a one-tile image
    whose 600-entry list every pixel leaves within a few splats (the forward
    stops before its first checkpoint, so the later chunks find nothing to
    walk). Chunked and whole-list gradients both meet the bar against the
    oracle."""
    bg = (0.3, 0.6, 0.1)
    cam = _sheet_camera(40, 16)
    scene = _tile_confined_scene(cam, (512, 257, 255), (0.05, 0.5), seed=21)
    ofwd = oracle_forward(orc, cam, scene, bg)
    lens = (ofwd["ranges"][:, 1] - ofwd["ranges"][:, 0]).tolist()
    assert lens == [512, 257, 255], lens
    stopped = ofwd["final_T"] < 1e-4
    assert stopped.any() and (~stopped).any()
    assert ofwd["n_contrib"].max() > 256  # some pixel needs a checkpoint
    dLdI = synth.upstream_gradient(7, 40, 16)
    obwd = oracle_backward(orc, cam, scene, ofwd, dLdI, bg)
    g, out, sc, _ = gpu_forward(cam, scene, bg=bg)
    assert_binning_equal(g, ofwd)
    compare_forward(g, ofwd, bg)
    compare_gradients(gpu_backward(cam, sc, out, dLdI, bg), obwd)
    compare_gradients(gpu_backward(cam, sc, out, dLdI, bg, chunked=True), obwd)

    cam1 = _sheet_camera(16, 16)
    rng = np.random.default_rng(22)
    n = 600
    z = rng.uniform(1.0, 3.0, n)
    means = np.stack([rng.uniform(-0.05, 0.05, n) * z, rng.uniform(-0.05, 0.05, n) * z, z]).astype(np.float32)
    opaque = dict(n=n, means=means, scales=np.full((3, n), 0.3, np.float32),
                  quats=np.tile(np.float32([[1], [0], [0], [0]]), (1, n)),
                  opacity=rng.uniform(0.8, 0.95, n).astype(np.float32),
                  rgb=rng.uniform(0, 1, (3, n)).astype(np.float32), sh=None, sh_degree=0)
    o1 = oracle_forward(orc, cam1, opaque, bg)
    assert o1["keys"].shape[0] == n and (o1["final_T"] < 1e-4).all() and o1["n_contrib"].max() < 256
    dL1 = synth.upstream_gradient(8, 16, 16)
    ob1 = oracle_backward(orc, cam1, opaque, o1, dL1, bg)
    g1, out1, sc1, _ = gpu_forward(cam1, opaque, bg=bg)
    compare_forward(g1, o1, bg)
    compare_gradients(gpu_backward(cam1, sc1, out1, dL1, bg, chunked=True), ob1)


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


@pytest.mark.parametrize("extra", [0, 1])
def test_entry_count_at_the_32_bit_limit(orc, extra):
    """Splats that each cover the whole 1920x1080 grid (120 x 68 = 8160 tiles):
    n = floor(2^32 / 8160) of them give E = 2^32 - 256, which still fits in 32
    bits (GS_ERR_CAPACITY against a capacity of 1); one more gives
    E = 2^32 + 7904 (GS_ERR_OVERFLOW). Both report the exact E, which the
    oracle's 64-bit scan of its own tile counts fixes, and neither writes an
    entry; the asynchronous call leaves E in n_entries_dev and the ranges
    then stay empty."""
    import ctypes

    import gaussian_splatting_tile_amd as gs
    import torch
    from gaussian_splatting_tile_amd import _lib
    W, H = 1920, 1080
    cam = synth.look_at_camera((0.0, 0.0, -4.0), (0.0, 0.0, 0.0), W, H, 1100.0, 1100.0)
    n = (1 << 32) // 8160 + extra
    say(f"[entry count limit n={n}]")
    scene = synth.random_scene(n, 77, cam, scale_lo=20.0, scale_hi=40.0, depth_lo=2.0, depth_hi=3.0, spread=0.1)
    opre = orc.preprocess(cam, scene)
    assert (opre["tiles_touched"] == 8160).all(), "every splat must cover the whole grid"
    _, E = orc.exclusive_scan(opre["tiles_touched"])
    assert E == n * 8160 and (E >= 1 << 32) == bool(extra)

    sc = gs.Scene.from_numpy(scene)
    pre = gs.preprocess(cam, sc.means, sc.scales, sc.quats, sc.opacity, sc.sh, sc.sh_degree, sc.rgb)
    xy_depth, tt = pre["xy_depth"], pre["tiles_touched"]
    assert_bits_equal(tt.cpu().numpy().view(np.uint32), opre["tiles_touched"], "tiles_touched")

    lib = _lib.load()
    c = gs.camera(cam)
    keys = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    plist = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    need = ctypes.c_size_t(0)
    assert lib.gs_bin_and_sort(ctypes.byref(c), n, None, None, None, None, 1, None, ctypes.byref(need),
                               None, None) == _lib.GS_OK
    scratch = torch.empty((need.value,), dtype=torch.uint8, device="cuda")
    n_entries = ctypes.c_int64(-1)
    st = lib.gs_bin_and_sort(ctypes.byref(c), n, ctypes.c_void_p(xy_depth.data_ptr()),
                             ctypes.c_void_p(tt.data_ptr()), ctypes.c_void_p(keys.data_ptr()),
                             ctypes.c_void_p(plist.data_ptr()), 1, ctypes.c_void_p(scratch.data_ptr()),
                             ctypes.byref(need), ctypes.byref(n_entries), None)
    want = _lib.GS_ERR_OVERFLOW if extra else _lib.GS_ERR_CAPACITY
    assert st == want, (_lib.STATUS_NAMES.get(st), lib.gs_last_error())
    assert n_entries.value == E
    torch.cuda.synchronize()
    assert int(keys.item()) == -1 and int(plist.item()) == -1

    bins = gs.BinBuffers(torch.device("cuda"), capacity=1)
    bins.keys.fill_(-1)
    bins.point_list.fill_(-1)
    gs.bin_and_sort_async(c, xy_depth, tt, bins)
    ranges = gs.tile_ranges_async(c, bins)
    assert bins.entries() == E
    assert not ranges.any()
    assert int(bins.keys.item()) == -1 and int(bins.point_list.item()) == -1


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


def _chunk_class(L):
    msb = np.floor(np.log2(np.maximum(L, 1))).astype(np.int64)
    frac = ((L << (31 - msb)) >> 27) & 15
    return np.minimum(255, 1 + 16 * msb + frac)


def _check_chunk_schedule(chunks, ranges):
    """chunks: the schedule words; ranges [T, 2]. With the cut length C = 256
    when the lists average more than 256 entries, else no cut: every
    (tile, k) with k < ceil(L / 256) of each list longer than C exactly once
    and every other tile once as a whole item, in non-increasing class of
    L - 256 k (k = 0 for whole items, empty tiles last). Returns C (None:
    no cut)."""
    L = ranges[:, 1].astype(np.int64) - ranges[:, 0]
    cut = 256 if L.sum() > 256 * len(L) else None
    if cut is None:
        cut_len = np.iinfo(np.int64).max
    else:
        cut_len = cut
    count = int(chunks[0])
    items4 = chunks[4:4 + 4 * count].reshape(count, 4).astype(np.int64)
    assert np.array_equal(items4[:, 2], np.where(L[items4[:, 0]] > 0, ranges[items4[:, 0], 0], 0))
    assert np.array_equal(items4[:, 3], L[items4[:, 0]])
    whole = items4[:, 1] == 0xFFFFFFFF
    nch = np.where(L > cut_len, (L + 255) // 256, 0)
    assert count == int(nch.sum()) + int((L <= cut_len).sum()), (count, int(nch.sum()))
    assert np.array_equal(np.sort(items4[whole, 0]), np.nonzero(L <= cut_len)[0])
    items = items4[~whole, :2]
    want = np.concatenate([np.stack([np.full(k, t), np.arange(k)], 1) for t, k in enumerate(nch) if k] or
                          [np.zeros((0, 2), np.int64)])
    got_sorted = items[np.lexsort((items[:, 1], items[:, 0]))]
    assert np.array_equal(got_sorted, want)
    rest = L[items4[:, 0]] - 256 * np.where(whole, 0, items4[:, 1])
    assert (rest[~whole] > 0).all()
    cls = np.where(rest == 0, -1, _chunk_class(np.maximum(rest, 1)))
    assert (np.diff(cls) <= 0).all()
    return cut


def test_chunk_schedule_covers_every_chunk(orc):
    """The ranges call's schedule for the chunked backward, from a host entry
    count and from a device count with spare capacity and with an overflow
    (nothing to schedule): whole lists at cfg2 (lists average under 256
    entries), chunks at cfg3."""
    import gaussian_splatting_tile_amd as gs
    import torch
    from gpu_helpers import to_np
    for name, cut in (("cfg2", None), ("cfg3", 256)):
        say(f"[{name}] schedule")
        scene, cam, _, ofwd, _ = workload(orc, name)
        g, out, sc, r = gpu_forward(cam, scene, capacity=1 << 23)
        assert _check_chunk_schedule(to_np(out["chunks"]).view(np.uint32), g["ranges"]) == cut
        c = gs.camera(cam)
        for capacity in (g["n_entries"] + 5000, g["n_entries"] - 1):
            bins = gs.BinBuffers(torch.device("cuda"), capacity)
            gs.bin_and_sort_async(c, out["xy_depth"], out["tiles_touched"], bins)
            chunks = torch.full((gs.chunk_words(cam, capacity),), -1, dtype=torch.int32, device="cuda")
            ranges = gs.tile_ranges_async(c, bins, chunks=chunks)
            torch.cuda.synchronize()
            rg = to_np(ranges).view(np.uint32)
            if capacity >= g["n_entries"]:
                assert np.array_equal(rg, g["ranges"])
                assert _check_chunk_schedule(to_np(chunks).view(np.uint32), rg) == cut
            else:
                # every list empty: one whole item per tile
                assert not rg.any()
                assert _check_chunk_schedule(to_np(chunks).view(np.uint32), rg) is None


def test_ranges_ignore_stale_buffer_contents(orc):
    """The ranges call writes only run boundaries and then checks every tile's
    range against the sorted keys, so whatever the buffer held before (random
    words, another frame's ranges, those ranges shuffled over the tiles) the
    result is the oracle's, empty tiles (0, 0), with the same schedules."""
    import gaussian_splatting_tile_amd as gs
    import torch
    from gpu_helpers import to_np
    scene, cam, _, ofwd, _ = workload(orc, "cfg1")
    g, out, sc, r = gpu_forward(cam, scene, capacity=1 << 21)
    E = g["n_entries"]
    c = gs.camera(cam)
    n_tiles = ofwd["ranges"].shape[0]
    big = synth.look_at_camera((0.3, 0.2, -3.0), (0, 0, 0), cam["width"], cam["height"], 500.0, 500.0)
    other = orc.render_fwd(big, scene)["ranges"].astype(np.int64)
    rng = np.random.default_rng(5)
    fills = {"random words": rng.integers(0, 2**31, (n_tiles, 2)),
             "another frame": other,
             "shuffled own ranges": ofwd["ranges"].astype(np.int64)[rng.permutation(n_tiles)],
             "own ranges reversed": ofwd["ranges"].astype(np.int64)[:, ::-1].copy()}
    ref_order = None
    for what, fill in fills.items():
        ranges = torch.from_numpy(fill.astype(np.uint32).view(np.int32)).cuda()
        order = torch.full((n_tiles,), -1, dtype=torch.int32, device="cuda")
        chunks = torch.full((gs.chunk_words(cam, int(out["keys"].numel())),), -1, dtype=torch.int32, device="cuda")
        gs.tile_ranges(c, out["keys"], E, out=ranges, order=order, chunks=chunks)
        torch.cuda.synchronize()
        rg = to_np(ranges).view(np.uint32)
        assert_bits_equal(rg, ofwd["ranges"], f"ranges over {what}")
        od = to_np(order).view(np.uint32).astype(np.int64)
        assert np.array_equal(np.sort(od), np.arange(n_tiles)), what
        _check_chunk_schedule(to_np(chunks).view(np.uint32), rg)
        # plain call (no schedules): only the check of the ranges runs
        ranges2 = torch.from_numpy(fill.astype(np.uint32).view(np.int32)).cuda()
        gs.tile_ranges(c, out["keys"], E, out=ranges2)
        torch.cuda.synchronize()
        assert_bits_equal(to_np(ranges2).view(np.uint32), ofwd["ranges"], f"plain ranges over {what}")
