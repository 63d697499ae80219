"""Host-side checks of the C ABI that need no GPU: the library loads, it
exports every function include/gs.h declares, its constants agree with the
oracle's, and argument validation rejects bad calls before launching."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gs.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(gs_[a-z_0-9]+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def gs():
    import gaussian_splatting_tile_amd as pkg
    from gaussian_splatting_tile_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libgs.so is not built: run __graft_entry__.build()")
    return _lib.load()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("gs_preprocess", "gs_bin_and_sort", "gs_tile_ranges", "gs_composite_fwd",
                     "gs_composite_bwd", "gs_last_error", "gs_constants"):
        assert required in names


def test_library_exports_every_declared_symbol(gs):
    from gaussian_splatting_tile_amd import _lib
    names = declared_functions()
    assert sorted(_lib.EXPORTS) == names
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (gs_[a-z_0-9]+)$", out, flags=re.M))
    for name in names:
        assert name in exported, name
        assert hasattr(gs, name)


def declared_arity():
    """Parameter count of every function include/gs.h declares."""
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    out = {}
    for m in re.finditer(r"\b(gs_[a-z_0-9]+)\s*\(([^;{]*?)\)\s*;", src):
        params = m.group(2).strip()
        out[m.group(1)] = 0 if params in ("", "void") else params.count(",") + 1
    return out


def test_binding_argument_counts_match_header(gs):
    """Every ctypes declaration passes as many arguments as the C prototype
    takes (a missing trailing pointer would shift the stream argument)."""
    arity = declared_arity()
    assert sorted(arity) == declared_functions()
    for name, n in arity.items():
        assert len(getattr(gs, name).argtypes) == n, name


def test_constants_match_oracle(gs, orc):
    import gaussian_splatting_tile_amd as pkg
    np.testing.assert_array_equal(pkg.constants(), orc.constants())
    assert pkg.version() == (0, 1, 0)


def _cam(**kw):
    from gaussian_splatting_tile_amd import _lib
    import synth
    from gaussian_splatting_tile_amd.rasterizer import camera
    c = synth.look_at_camera((0, 0, -4), (0, 0, 0), 64, 64, 64.0, 64.0)
    c.update(kw)
    return camera(c)


def test_invalid_arguments_rejected_before_launch(gs):
    from gaussian_splatting_tile_amd import _lib
    P = ctypes.c_void_p
    dummy = P(256)  # never dereferenced: validation fails first
    c = _cam()
    # NULL camera
    assert gs.gs_preprocess(None, 1, dummy, dummy, dummy, dummy, None, 0, dummy, dummy, dummy,
                            dummy, dummy, None) == _lib.GS_ERR_INVALID
    assert b"camera" in gs.gs_last_error()
    # negative n
    assert gs.gs_preprocess(ctypes.byref(c), -1, dummy, dummy, dummy, dummy, None, 0, dummy, dummy,
                            dummy, dummy, dummy, None) == _lib.GS_ERR_INVALID
    # sh degree out of range
    assert gs.gs_preprocess(ctypes.byref(c), 4, dummy, dummy, dummy, dummy, dummy, 4, None, dummy,
                            dummy, dummy, dummy, None) == _lib.GS_ERR_INVALID
    # no colour source
    assert gs.gs_preprocess(ctypes.byref(c), 4, dummy, dummy, dummy, dummy, None, 0, None, dummy,
                            dummy, dummy, dummy, None) == _lib.GS_ERR_INVALID
    # bad image sizes / focal lengths
    for bad in (_cam(width=0), _cam(height=-3), _cam(width=20000), _cam(fx=0.0),
                _cam(fy=float("nan")), _cam(cx=float("inf"))):
        assert gs.gs_tile_ranges(ctypes.byref(bad), None, 0, dummy, None, None) == _lib.GS_ERR_INVALID
    # n == 0 is a valid no-op
    assert gs.gs_preprocess(ctypes.byref(c), 0, None, None, None, None, None, 0, None, None, None,
                            None, None, None) == _lib.GS_OK
    # misaligned float4 buffer
    assert gs.gs_composite_fwd(ctypes.byref(c), dummy, dummy, P(260), dummy, dummy,
                               (ctypes.c_float * 3)(), dummy, dummy, dummy, None, None, None) == _lib.GS_ERR_INVALID


def test_preprocess_bwd_validates_before_launch(gs):
    from gaussian_splatting_tile_amd import _lib
    P = ctypes.c_void_p
    d = P(256)  # never dereferenced: validation fails first
    c = _cam()
    args = lambda **kw: [kw.get(k, d) for k in ("means", "scales", "quats")] + [kw.get("sh", None), kw.get("deg", 0)] + \
        [kw.get(k, d) for k in ("tt", "gm", "gc", "gr", "om", "os", "oq", "oo")] + [kw.get("osh", None), kw.get("orgb", d), None]
    ok = gs.gs_preprocess_bwd(ctypes.byref(c), 0, *args())
    assert ok == _lib.GS_OK  # n == 0: nothing to do
    assert gs.gs_preprocess_bwd(None, 4, *args()) == _lib.GS_ERR_INVALID
    assert gs.gs_preprocess_bwd(ctypes.byref(c), -2, *args()) == _lib.GS_ERR_INVALID
    assert gs.gs_preprocess_bwd(ctypes.byref(c), 4, *args(orgb=None)) == _lib.GS_ERR_INVALID
    assert b"grad_rgb_in" in gs.gs_last_error()
    assert gs.gs_preprocess_bwd(ctypes.byref(c), 4, *args(sh=d, deg=2)) == _lib.GS_ERR_INVALID
    assert b"grad_sh" in gs.gs_last_error()
    assert gs.gs_preprocess_bwd(ctypes.byref(c), 4, *args(sh=d, deg=5, osh=d)) == _lib.GS_ERR_INVALID
    assert gs.gs_preprocess_bwd(ctypes.byref(c), 4, *args(tt=None)) == _lib.GS_ERR_INVALID
    assert gs.gs_preprocess_bwd(ctypes.byref(c), 4, *args(gc=P(260))) == _lib.GS_ERR_INVALID
    assert b"aligned" in gs.gs_last_error()


def test_tile_test_flags_validated(gs):
    from gaussian_splatting_tile_amd import _lib
    P = ctypes.c_void_p
    d = P(256)
    c = _cam()
    # unknown flag bits
    assert gs.gs_preprocess_ex(ctypes.byref(c), 4, d, d, d, d, None, 0, d, d, d, d, d, 2, None) == _lib.GS_ERR_INVALID
    assert b"flags" in gs.gs_last_error()
    need = ctypes.c_size_t(0)
    assert gs.gs_bin_and_sort_ex(ctypes.byref(c), 10, None, None, None, None, None, 100, None,
                                 ctypes.byref(need), None, 0, None) == _lib.GS_OK and need.value > 0
    buf = ctypes.c_size_t(need.value)
    n_e = ctypes.c_int64(0)
    scratch = P(4096)  # 256-aligned, never dereferenced: validation fails first
    # the ellipse test without a conic
    assert gs.gs_bin_and_sort_ex(ctypes.byref(c), 10, d, None, d, d, d, 100, scratch, ctypes.byref(buf),
                                 ctypes.byref(n_e), _lib.GS_TILES_ELLIPSE, None) == _lib.GS_ERR_INVALID
    assert b"conic" in gs.gs_last_error()
    # a misaligned conic
    assert gs.gs_bin_and_sort_async_ex(ctypes.byref(c), 10, d, P(264), d, d, d, 100, scratch, ctypes.byref(buf),
                                       P(512), _lib.GS_TILES_ELLIPSE, None) == _lib.GS_ERR_INVALID
    assert gs.gs_bin_and_sort_async_ex(ctypes.byref(c), 10, d, d, d, d, d, 100, scratch, ctypes.byref(buf),
                                       P(512), 4, None) == _lib.GS_ERR_INVALID


def test_appearance_validates_before_launch(gs):
    from gaussian_splatting_tile_amd import _lib
    P = ctypes.c_void_p
    d = P(256)
    c = _cam()
    assert gs.gs_appearance_fwd(ctypes.byref(c), 10, d, d, 0, 32, d, d, None) == _lib.GS_ERR_INVALID
    assert b"n_latent" in gs.gs_last_error()
    assert gs.gs_appearance_fwd(ctypes.byref(c), 10, d, d, 30, 32, d, d, None) == _lib.GS_ERR_INVALID
    assert gs.gs_appearance_fwd(ctypes.byref(c), 10, d, d, 8, 65, d, d, None) == _lib.GS_ERR_INVALID
    assert b"n_hidden" in gs.gs_last_error()
    assert gs.gs_appearance_fwd(ctypes.byref(c), 10, d, None, 8, 32, d, d, None) == _lib.GS_ERR_INVALID
    need = ctypes.c_size_t(0)
    assert gs.gs_appearance_bwd(ctypes.byref(c), 1000, None, None, 8, 32, None, None, None, None, None,
                                ctypes.byref(need), None) == _lib.GS_OK
    assert need.value == 8 * 483 * 4  # ceil(1000 / 128) workgroups x 483 weights
    small = ctypes.c_size_t(need.value - 4)
    assert gs.gs_appearance_bwd(ctypes.byref(c), 1000, d, d, 8, 32, d, d, d, d, P(4096), ctypes.byref(small),
                                None) == _lib.GS_ERR_INVALID
    assert b"smaller" in gs.gs_last_error()


def test_bin_scratch_size_query(gs):
    from gaussian_splatting_tile_amd import _lib
    c = _cam()
    need = ctypes.c_size_t(0)
    assert gs.gs_bin_and_sort(ctypes.byref(c), 1000, None, None, None, None, 5000, None,
                              ctypes.byref(need), None, None) == _lib.GS_OK
    small = need.value
    assert small > 5000 * 12
    assert gs.gs_bin_and_sort(ctypes.byref(c), 1000, None, None, None, None, 50000, None,
                              ctypes.byref(need), None, None) == _lib.GS_OK
    assert need.value > small
    # a scratch buffer smaller than required is rejected
    nbytes = ctypes.c_size_t(small - 1)
    e = ctypes.c_int64(0)
    assert gs.gs_bin_and_sort(ctypes.byref(c), 1000, ctypes.c_void_p(256), ctypes.c_void_p(256),
                              ctypes.c_void_p(256), ctypes.c_void_p(256), 5000, ctypes.c_void_p(256),
                              ctypes.byref(nbytes), ctypes.byref(e), None) == _lib.GS_ERR_INVALID
    # capacity beyond 32-bit entry indices is rejected
    assert gs.gs_bin_and_sort(ctypes.byref(c), 10, None, None, None, None, 1 << 33, None,
                              ctypes.byref(need), None, None) == _lib.GS_ERR_INVALID


def test_binding_refuses_host_tensors(gs):
    import torch
    import gaussian_splatting_tile_amd as pkg
    import synth
    cam = synth.look_at_camera((0, 0, -4), (0, 0, 0), 64, 64, 64.0, 64.0)
    x = torch.zeros((3, 4))
    with pytest.raises(TypeError):
        pkg.preprocess(cam, x, x, torch.zeros((4, 4)), torch.zeros(4), rgb_in=x)


def test_async_entry_points_validate(gs):
    from gaussian_splatting_tile_amd import _lib
    P = ctypes.c_void_p
    c = _cam()
    need = ctypes.c_size_t(0)
    # the size query agrees with the blocking variant
    assert gs.gs_bin_and_sort_async(ctypes.byref(c), 1000, None, None, None, None, 5000, None,
                                    ctypes.byref(need), None, None) == _lib.GS_OK
    q = ctypes.c_size_t(0)
    assert gs.gs_bin_and_sort(ctypes.byref(c), 1000, None, None, None, None, 5000, None,
                              ctypes.byref(q), None, None) == _lib.GS_OK
    assert need.value == q.value
    # a missing or misaligned device count is rejected before launch
    nb = ctypes.c_size_t(need.value)
    for bad in (None, P(260)):
        assert gs.gs_bin_and_sort_async(ctypes.byref(c), 1000, P(256), P(256), P(256), P(256), 5000,
                                        P(256), ctypes.byref(nb), bad, None) == _lib.GS_ERR_INVALID
    assert gs.gs_tile_ranges_async(ctypes.byref(c), P(256), None, 10, P(256), None, None) == _lib.GS_ERR_INVALID
    assert gs.gs_tile_ranges_async(ctypes.byref(c), P(256), P(260), 10, P(256), None, None) == _lib.GS_ERR_INVALID
    assert gs.gs_tile_ranges_async(ctypes.byref(c), P(256), P(256), -1, P(256), None, None) == _lib.GS_ERR_INVALID


def test_chunked_composite_validates_before_launch(gs):
    from gaussian_splatting_tile_amd import _lib
    P = ctypes.c_void_p
    d = P(256)  # never dereferenced: validation fails first
    c = _cam()
    bg = (ctypes.c_float * 3)()
    fwd = lambda cap=100, ckpt=d, rgb=d, chunks=None, part=None, ranges=d, views=1: gs.gs_composite_fwd_ex(
        ctypes.byref(c), views, ranges, d, d, d, rgb, bg, d, d, d, None, None, cap, ckpt, chunks, part, None)
    assert fwd(cap=-1) == _lib.GS_ERR_INVALID
    assert b"capacity" in gs.gs_last_error()
    assert fwd(cap=1 << 32) == _lib.GS_ERR_INVALID
    assert fwd(ckpt=P(264)) == _lib.GS_ERR_INVALID  # checkpoints are float4 rows
    assert b"aligned" in gs.gs_last_error()
    assert fwd(chunks=d) == _lib.GS_ERR_INVALID  # the scheduled forward needs its workspace
    assert b"part" in gs.gs_last_error()
    assert fwd(chunks=P(264), part=d) == _lib.GS_ERR_INVALID
    assert fwd(chunks=d, part=P(260)) == _lib.GS_ERR_INVALID
    assert fwd(ranges=None) == _lib.GS_ERR_INVALID  # without a schedule the ranges are read
    for bad in (0, -1, 33):
        assert fwd(views=bad) == _lib.GS_ERR_INVALID
        assert b"n_views" in gs.gs_last_error()
    # the workspace size: (ceil(capacity / 256) + tiles) rows of 256 (float4 + uint32)
    tiles = 4 * 4  # the 64 x 64 test camera
    assert gs.gs_composite_part_bytes(ctypes.byref(c), 1, 1000) == (4 + tiles) * 256 * 20
    assert gs.gs_composite_part_bytes(ctypes.byref(c), 3, 1000) == (4 + 3 * tiles) * 256 * 20
    assert gs.gs_composite_part_bytes(ctypes.byref(c), 1, 0) == tiles * 256 * 20
    assert gs.gs_composite_part_bytes(ctypes.byref(c), 1, -1) == 0
    assert gs.gs_composite_part_bytes(ctypes.byref(c), 0, 10) == 0
    assert gs.gs_composite_part_bytes(None, 1, 10) == 0
    bwd = lambda n=4, chunks=d, cap=100, image=d, ckpt=d, gm=d, views=1: gs.gs_composite_bwd_ex(
        ctypes.byref(c), views, n, d, d, chunks, cap, d, d, d, bg, image, d, d, ckpt, d, gm, d, d, None)
    assert bwd(ckpt=None) == _lib.GS_ERR_INVALID  # the chunked walk needs the checkpoints
    assert b"ckpt" in gs.gs_last_error()
    assert bwd(image=None) == _lib.GS_ERR_INVALID
    assert bwd(chunks=None) == _lib.GS_ERR_INVALID
    assert bwd(cap=-5) == _lib.GS_ERR_INVALID
    assert bwd(n=-1) == _lib.GS_ERR_INVALID
    assert bwd(gm=None) == _lib.GS_ERR_INVALID
    assert bwd(chunks=P(264)) == _lib.GS_ERR_INVALID
    assert bwd(ckpt=P(264)) == _lib.GS_ERR_INVALID
    assert bwd(views=0) == _lib.GS_ERR_INVALID and b"n_views" in gs.gs_last_error()
    rng = lambda n_e=10, n_dev=None, cap=100, keys=d, ranges=d, chunks=d, views=1: gs.gs_tile_ranges_ex(
        ctypes.byref(c), views, keys, n_e, n_dev, cap, ranges, None, chunks, None)
    assert rng(n_e=101) == _lib.GS_ERR_INVALID  # more entries than the keys hold
    assert b"n_entries" in gs.gs_last_error()
    assert rng(n_e=-1) == _lib.GS_ERR_INVALID
    assert rng(cap=-1) == _lib.GS_ERR_INVALID
    assert rng(ranges=None) == _lib.GS_ERR_INVALID
    assert rng(keys=None) == _lib.GS_ERR_INVALID
    assert rng(chunks=P(264)) == _lib.GS_ERR_INVALID
    assert rng(n_dev=P(516)) == _lib.GS_ERR_INVALID
    assert rng(views=33) == _lib.GS_ERR_INVALID and b"n_views" in gs.gs_last_error()


def test_header_chunk_schedule_size_matches_binding():
    """The size gs.h states for the chunk schedule of gs_tile_ranges_ex, read
    from the header and evaluated, equals what the binding allocates, for
    single views and view stacks (the compositing launches index up to that
    many items)."""
    import math
    import re
    from gaussian_splatting_tile_amd.rasterizer import chunk_words
    text = open(os.path.join(ROOT, "include", "gs.h")).read()
    m = re.search(r"\*\s+chunks\s+out uint32 \[(.+?)\],", text)
    assert m, "chunk schedule size not found in gs.h"
    expr = m.group(1)
    for (W, H, views, cap) in [(64, 64, 1, 1000), (400, 400, 4, 2_560_000), (100, 75, 16, 12345),
                               (1920, 1080, 1, 1_600_000), (33, 17, 32, 0)]:
        TX, TY = -(-W // 16), -(-H // 16)
        want = eval(expr, {"__builtins__": {}}, dict(TX=TX, TY=TY, n_views=views, capacity=cap, ceil=math.ceil))
        assert want == chunk_words(dict(width=W, height=H), cap, views), (W, H, views, cap)


def test_view_stack_validates_before_launch(gs):
    """gs_preprocess_views and gs_bin_and_sort_views_async check the stack
    (camera count and sizes, the splat total, the tile count) before any
    launch."""
    from gaussian_splatting_tile_amd import _lib
    P = ctypes.c_void_p
    d = P(256)  # never dereferenced: validation fails first
    cams = (_lib.GsCamera * 3)(_cam(), _cam(), _cam())
    pre = lambda cs=cams, views=3, n=10, sh=None, rgb=d, out=d: gs.gs_preprocess_views(
        ctypes.cast(cs, P) if cs is not None else None, views, n, d, d, d, d, sh, 0, rgb, out, d, d, d, 0, None)
    assert pre(cs=None) == _lib.GS_ERR_INVALID
    for bad in (0, 33):
        assert pre(views=bad) == _lib.GS_ERR_INVALID and b"n_views" in gs.gs_last_error()
    odd = (_lib.GsCamera * 2)(_cam(), _cam(width=80))
    assert pre(cs=odd, views=2) == _lib.GS_ERR_INVALID  # one size for the whole stack
    assert b"camera 1" in gs.gs_last_error()
    assert pre(n=-1) == _lib.GS_ERR_INVALID
    assert pre(n=(1 << 24) // 3 + 1) == _lib.GS_ERR_INVALID  # the stack's records exceed GS_MAX_GAUSSIANS
    assert pre(sh=None, rgb=None) == _lib.GS_ERR_INVALID
    assert pre(out=P(264)) == _lib.GS_ERR_INVALID
    assert pre(n=0) == _lib.GS_OK  # nothing to do
    c = _cam()
    need = ctypes.c_size_t(0)
    assert gs.gs_bin_and_sort_views_async(ctypes.byref(c), 3, 10, None, None, None, None, None, 100, None,
                                          ctypes.byref(need), None, 0, None) == _lib.GS_OK and need.value > 0
    one = ctypes.c_size_t(0)
    assert gs.gs_bin_and_sort(ctypes.byref(c), 30, None, None, None, None, 100, None, ctypes.byref(one),
                              None, None) == _lib.GS_OK
    assert one.value == need.value  # the scratch of n_views n splats
    big = _cam(width=16384, height=16384)  # 2^20 tiles per view
    assert gs.gs_bin_and_sort_views_async(ctypes.byref(big), 32, 10, None, None, None, None, None, 100, None,
                                          ctypes.byref(need), None, 0, None) == _lib.GS_ERR_INVALID
    assert b"2^24 tiles" in gs.gs_last_error()
    assert gs.gs_bin_and_sort_views_async(ctypes.byref(c), 0, 10, None, None, None, None, None, 100, None,
                                          ctypes.byref(need), None, 0, None) == _lib.GS_ERR_INVALID
