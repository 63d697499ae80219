"""Pins for the oracle's scan, duplication, sort and tile ranges.

Expected values: the zenn page's worked examples (tests/golden), numpy's
stable argsort (a library routine), the learn-gs notebook's three CPU claims,
and brute-force tile membership.
"""
import json
import os

import numpy as np
import pytest

import synth

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "zenn_worked_examples.json")))


@pytest.mark.parametrize("case", [c for c in GOLDEN["exclusive_scan"] if "exclusive" in c],
                         ids=lambda c: c["section"][:12])
def test_exclusive_scan_worked_examples(orc, case):
    offsets, total = orc.exclusive_scan(case["input"])
    assert list(offsets) == case["exclusive"]
    assert total == sum(case["input"])
    if "inclusive" in case:
        assert list(offsets + np.asarray(case["input"])) == case["inclusive"]
    if "slices" in case:
        assert [[int(o), int(o) + c] for o, c in zip(offsets, case["input"])] == case["slices"]


def test_exclusive_scan_random_and_capacity(orc):
    rng = np.random.default_rng(0)
    c = rng.integers(0, 200, 100_000).astype(np.uint32)
    off, total = orc.exclusive_scan(c)
    assert total == int(c.astype(np.uint64).sum())
    np.testing.assert_array_equal(off, np.concatenate([[0], np.cumsum(c.astype(np.uint64))[:-1]]))
    cap = [x for x in GOLDEN["exclusive_scan"] if "capacity" in x][0]
    assert cap["workgroup_size"] ** cap["levels"] == cap["capacity"]
    # totals beyond 32 bits are carried exactly (the caller must reject them)
    big = np.full(4, 0xFFFFFFFF, np.uint32)
    assert orc.exclusive_scan(big)[1] == 4 * 0xFFFFFFFF


def _records_with_counts(counts, TX, TY):
    """xy_depth records whose tile spans are 1 x count rectangles on row 0."""
    recs = np.zeros((len(counts), 4), np.float32)
    for g, c in enumerate(counts):
        # radius 1 at x = 8 + 16k covers one tile column; widen by choosing the
        # centre between columns: span = [x0, x0 + c) via r = 8 c - 1
        r = 8 * c - 1 if c > 0 else 0
        recs[g] = (8 * c, 8.0, 1.0 + g, r)
    return recs


def test_duplicate_writes_private_slices(orc):
    ex = GOLDEN["duplicate"]
    cam = dict(R=np.eye(3, dtype=np.float32).reshape(9), t=np.zeros(3, np.float32),
               campos=np.zeros(3, np.float32), fx=1, fy=1, cx=0, cy=0, width=16 * 8, height=16)
    counts = ex["tiles_touched"]
    recs = _records_with_counts(counts, 8, 1)
    for g, c in enumerate(counts):
        x0, x1, y0, y1 = orc.tile_span(*recs[g][[0, 1, 3]], 8, 1)
        assert (x1 - x0) * (y1 - y0) == c
    offsets, total = orc.exclusive_scan(counts)
    assert list(offsets) == ex["offsets"]
    keys, vals = orc.duplicate(cam, recs, counts, offsets, total)
    for g, (s, e) in enumerate(ex["slices"]):
        assert (vals[s:e] == g).all()
        assert ((keys[s:e] & 0xFFFFFFFF) == np.float32(recs[g, 2]).view(np.uint32)).all()
        tiles = keys[s:e] >> 32
        assert list(tiles) == sorted(tiles)  # row-major span order


def test_key_packs_tile_and_depth_bits(orc):
    cam = synth.config_scene("cfg0")[1]
    pre = orc.preprocess(cam, synth.config_scene("cfg0")[0])
    offsets, total = orc.exclusive_scan(pre["tiles_touched"])
    keys, vals = orc.duplicate(cam, pre["xy_depth"], pre["tiles_touched"], offsets, total)
    depth = pre["xy_depth"][vals, 2]
    np.testing.assert_array_equal((keys & 0xFFFFFFFF).astype(np.uint32), depth.view(np.uint32))
    TX, TY = orc.tiles_xy(cam)
    assert ((keys >> 32) < TX * TY).all()


def test_sort_histogram_example(orc):
    ex = GOLDEN["radix_histogram"]
    d = np.asarray(ex["digits"], np.uint64)
    k, v = orc.sort_pairs(d, np.arange(len(d), dtype=np.uint32))
    assert list(k) == ex["sorted"]
    hist = np.bincount(np.asarray(ex["digits"]), minlength=5)
    assert list(hist) == ex["histogram"]
    assert list(np.searchsorted(k, np.arange(5))) == ex["bin_starts"]


def test_sort_workgroup_offsets_example(orc):
    """Concatenating three workgroups' elements and sorting stably puts each
    workgroup's bin-0 elements in the ranges the page derives."""
    ex = GOLDEN["radix_workgroup_offsets"]
    digits, wg = [], []
    for w, counts in enumerate(ex["counts_per_workgroup"]):
        for b, c in enumerate(counts):
            digits += [b] * c
            wg += [w] * c
    k, v = orc.sort_pairs(np.asarray(digits, np.uint64), np.asarray(wg, np.uint32))
    assert list(np.searchsorted(k, np.arange(3))) == ex["bin_starts"]
    for w, (s, e) in enumerate(ex["bin0_workgroup_ranges"]):
        assert (v[s:e] == w).all() and (k[s:e] == 0).all()


def test_sort_flag_bit_rank_example(orc):
    ex = GOLDEN["radix_rank"]
    bins = np.asarray(ex["bins"], np.uint64)
    k, v = orc.sort_pairs(bins, np.arange(len(bins), dtype=np.uint32))
    b = ex["bins"][ex["thread"]]
    start = int(np.searchsorted(k, b))
    assert v[start + ex["rank_in_bin"]] == ex["thread"]


def test_sort_matches_numpy_stable_argsort(orc):
    rng = np.random.default_rng(1)
    keys = (rng.integers(0, 40, 50_000).astype(np.uint64) << np.uint64(32)) | rng.integers(0, 5, 50_000).astype(np.uint64)
    vals = np.arange(50_000, dtype=np.uint32)
    k, v = orc.sort_pairs(keys, vals)
    order = np.argsort(keys, kind="stable")
    np.testing.assert_array_equal(k, keys[order])
    np.testing.assert_array_equal(v, vals[order])


def test_positive_float_bits_sort_like_floats(orc):
    """learn-gs claim 1: the bit patterns of positive floats order like the floats."""
    rng = np.random.default_rng(11)
    d = (rng.uniform(0, 1, 20_000) * 50 + 0.05).astype(np.float32)
    k, v = orc.sort_pairs(d.view(np.uint32).astype(np.uint64), np.arange(d.size, dtype=np.uint32))
    assert (np.diff(d[v]) >= 0).all()


@pytest.mark.parametrize("case", GOLDEN["tile_ranges"], ids=lambda c: c["section"][:8])
def test_tile_range_examples(orc, case):
    tiles = np.asarray(case["tile_ids"], np.uint64)
    n_tiles = int(tiles.max()) + 1
    cam = dict(R=np.eye(3, dtype=np.float32).reshape(9), t=np.zeros(3, np.float32),
               campos=np.zeros(3, np.float32), fx=1, fy=1, cx=0, cy=0, width=16 * n_tiles, height=16)
    ranges = orc.tile_ranges(cam, tiles << np.uint64(32))
    if "ranges" in case:
        assert [list(r) for r in ranges[:len(case["ranges"])]] == case["ranges"]
    if "empty_tile" in case:
        assert list(ranges[case["empty_tile"]]) == case["empty_range"]


@pytest.mark.parametrize("name", ["cfg0", "cfg1"])
def test_binning_invariants_and_brute_force(orc, name):
    """E = sum tiles_touched = sum(end - start); ranges partition the list;
    depth nondecreasing (index increasing on ties) in each tile (learn-gs
    claim 3); tile t lists exactly {g : t in span(g)}."""
    scene, cam, _ = synth.config_scene(name)
    pre = orc.preprocess(cam, scene)
    keys, pl = orc.bin_and_sort(cam, pre["xy_depth"], pre["tiles_touched"])
    ranges = orc.tile_ranges(cam, keys)
    E = keys.shape[0]
    assert E == int(pre["tiles_touched"].astype(np.int64).sum())
    lens = ranges[:, 1].astype(np.int64) - ranges[:, 0]
    assert lens.sum() == E
    nz = np.nonzero(lens)[0]
    assert ranges[nz[0], 0] == 0 and ranges[nz[-1], 1] == E
    assert (ranges[nz[1:], 0] == ranges[nz[:-1], 1]).all()
    assert (ranges[lens == 0] == 0).all()
    TX, TY = orc.tiles_xy(cam)
    xy = pre["xy_depth"]
    u, v, z, r = xy[:, 0].astype(np.float64), xy[:, 1].astype(np.float64), xy[:, 2], xy[:, 3].astype(np.float64)
    vis = pre["tiles_touched"] > 0
    step = 1 if name == "cfg0" else 97
    for t in range(0, TX * TY, step):
        s, e = int(ranges[t, 0]), int(ranges[t, 1])
        seg = pl[s:e]
        assert ((keys[s:e] >> 32) == t).all()
        dz = z[seg]
        assert (np.diff(dz) >= 0).all()
        ties = np.diff(dz) == 0
        assert (np.diff(seg.astype(np.int64))[ties] > 0).all()
        tx, ty = t % TX, t // TX
        brute = np.nonzero(vis & (tx * 16 <= u + r) & ((tx + 1) * 16 > u - r)
                           & (ty * 16 <= v + r) & ((ty + 1) * 16 > v - r))[0]
        assert sorted(seg.tolist()) == brute.tolist()
