"""GPU: a batch of views composited as one stacked frame (ViewStack: view v
is the band of tile rows [v TY, v TY + TY)). Against the oracle run on each
view alone: the records of every view bit-exact (gs_preprocess_views), each
tile's list bit-exact (the stack's value v n + g is the view's Gaussian g),
the image and n_contrib to the forward bar, the gradients to the backward
bar; a HIP graph of the batch replays the eager run. Sizes: the training
shape (400 x 400, a multiple of the tile) as one stack, and a ragged one
(100 x 75, whose bands end in rows outside the image) cut into two stacks on
two streams, and into four stacks of one view each.
"""
import sys

import numpy as np
import pytest

import synth
from gpu_helpers import (GRAD_REL, assert_bits_equal, compare_forward, compare_gradients, oracle_backward,
                         oracle_forward, to_np)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _check_stack(orc, stack, scene_np, cams, dLdI):
    """Each view of every stack of the batch against the oracle on that view alone."""
    import torch
    torch.cuda.synchronize()
    E_all = stack.check()
    for grp, E in zip(stack.groups, E_all):
        _check_group(orc, stack, grp, E, scene_np, cams, dLdI)


def _check_group(orc, stack, grp, E, scene_np, cams, dLdI):
    n = scene_np["n"]
    pre = {k: to_np(v) for k, v in grp.pre.items()}
    keys = to_np(grp.bins.keys)[:E].view(np.uint64)
    pl = to_np(grp.bins.point_list)[:E].view(np.uint32)
    ranges = to_np(grp.ranges).view(np.uint32)
    TXY = ranges.shape[0] // grp.V
    E_sum = 0
    for v in range(grp.V):
        cam = cams[grp.first + v]
        vb = grp.first + v  # the view's place in the batch
        o = oracle_forward(orc, cam, scene_np)
        sl = slice(v * n, (v + 1) * n)
        for k in ("xy_depth", "conic_op", "rgb", "tiles_touched"):
            got = pre[k][sl].view(np.uint32) if k == "tiles_touched" else pre[k][sl]
            assert_bits_equal(got, o[k], f"view {v} {k}")
        # every tile's list: the oracle's for this view, values shifted by v n
        r = ranges[v * TXY:(v + 1) * TXY]
        L = (r[:, 1].astype(np.int64) - r[:, 0])
        oL = (o["ranges"][:, 1].astype(np.int64) - o["ranges"][:, 0])
        assert np.array_equal(L, oL), f"view {v} list lengths"
        for t in np.nonzero(L)[0]:
            got = pl[r[t, 0]:r[t, 1]].astype(np.int64) - v * n
            want = o["point_list"][o["ranges"][t, 0]:o["ranges"][t, 1]]
            if not np.array_equal(got, want):
                raise AssertionError(f"view {v} tile {t}: list differs")
            assert (keys[r[t, 0]:r[t, 1]] >> np.uint64(32) == np.uint64(v * TXY + t)).all()
        E_sum += int(L.sum())
        g = dict(image=to_np(stack.fwd["image"][vb]), final_T=to_np(stack.fwd["final_T"][vb]),
                 n_contrib=to_np(stack.fwd["n_contrib"][vb]).view(np.uint32))
        compare_forward(g, o)
        ob = oracle_backward(orc, cam, scene_np, o, dLdI[vb])
        gg = {k: to_np(t[vb * n:(vb + 1) * n]).astype(np.float64) for k, t in stack.grads.items()}
        compare_gradients(gg, ob)
    assert E_sum == E


@pytest.mark.parametrize("size,streams", [((400, 400), 1), ((100, 75), 2), ((100, 75), 4)])
def test_view_stack_matches_each_view(orc, size, streams):
    import torch
    import gaussian_splatting_tile_amd as gs
    W, H = size
    V = 4
    scene_np, _, _ = synth.config_scene("cfg4")
    cams = []
    for v in range(V):
        cam = dict(synth.config_scene("cfg4", view=v)[1])
        s = W / cam["width"]
        cam.update(width=W, height=H, fx=np.float32(cam["fx"] * s), fy=np.float32(cam["fy"] * s),
                   cx=np.float32(W / 2), cy=np.float32(H / 2))
        cams.append(cam)
    say(f"[stack] {V} views {W}x{H} as {streams} stack(s)")
    sc = gs.Scene.from_numpy(scene_np)
    rng = np.random.default_rng(5)
    dLdI = rng.standard_normal((V, 3, H, W)).astype(np.float32)
    dL = torch.from_numpy(dLdI).cuda()
    stack = gs.ViewStack(cams, sc, capacity=V * (1 << 20), streams=streams)
    loss = lambda first, image, out: out.copy_(dL[first:first + out.shape[0]])
    stack.enqueue(loss)
    _check_stack(orc, stack, scene_np, cams, dLdI)
    say(f"[stack] {W}x{H}: every view matches the oracle")
    # one HIP graph of the batch replays the eager run
    eager = {k: to_np(t).copy() for k, t in stack.fwd.items()}
    eg = {k: to_np(t).astype(np.float64) for k, t in stack.grads.items()}
    stack.capture(loss)
    for rep in range(2):
        stack.fwd["image"].fill_(float("nan"))
        for t in stack.grads.values():
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        stack.replay()
        torch.cuda.synchronize()
        for k, t in stack.fwd.items():
            assert to_np(t).tobytes() == eager[k].tobytes(), (rep, k)
        for k, t in stack.grads.items():
            a = to_np(t).astype(np.float64)
            assert np.abs(a - eg[k]).max() <= 1e-5 * max(np.abs(eg[k]).max(), 1e-30), (rep, k)
    say(f"[stack] {W}x{H}: graph replays match")
