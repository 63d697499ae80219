"""Benchmark: forward + backward frames/s of the tile-based Gaussian
Splatting rasterizer on one MI355X.

A step is one pass of the whole path over one frame: preprocess, binning
(depth order, scan, duplication, radix sort on the tile bits), tile ranges,
forward compositing, backward compositing. Binning and ranges use the
asynchronous entry points, which keep the entry count in device memory, so
a frame is enqueued without a host wait; the count is checked against the
capacity after the timed region. Inputs (Gaussians, camera, upstream
gradient dL/dI) are resident in HBM before timing starts.

Workload (default): 160,000-Gaussian procedural scene (60% sphere shell,
20% helix, 20% checkered plane), SH degree 3, 1920x1080, fx = fy = 1100,
dL/dI ~ N(0, 1).

Prints one JSON line (rank 0). Per-stage times come from HIP events
recorded on the stream the kernels run on.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fwd+bwd frames/s @160k Gaussians 1920x1080; pixel-splat evals/s vs VALU peak"
WORKLOADS = {
    "cfg0": "1,000 Gaussians on a jittered unit sphere, precomputed RGB, 64x64, forward + backward with "
            "dL/dI ~ N(0,1)",
    "cfg2": "160,000-Gaussian procedural scene (60% sphere shell, 20% helix, 20% checkered plane), "
            "SH degree 3, 1920x1080, fx=fy=1100, forward + backward with dL/dI ~ N(0,1)",
    "cfg3": "1,000,000-Gaussian dense-overdraw scene (80% thick shell, 20% cube), SH degree 3, "
            "1920x1080, forward + backward with dL/dI ~ N(0,1)",
    "cfg1": "160,000-Gaussian procedural scene, SH degree 3, 720x720, forward + backward",
    "cfg4": "training-step shape: 300,000-Gaussian dense scene, 16 views at 400x400 per step, forward + "
            "backward with dL/dI = sign(I - I_ref) against a second scene's render; the 16 views are "
            "recorded once as a HIP graph and replayed",
}
# Algorithmic work per unit: a forward pixel-splat evaluation is ~25 fp32
# flop-equivalents (the quadratic form, one exponential counted as 8, the
# clamp, the colour and transmittance updates); a backward one ~45 plus its
# share of the per-splat reduction.
FLOPS_PER_FWD_EVAL = 25.0
FLOPS_PER_BWD_EVAL = 45.0
PEAK_FP32_VECTOR = 157.3e12   # MI355X fp32 vector (packed) FLOP/s
PEAK_HBM = 8.0e12             # MI355X HBM3E bytes/s
EVENT_EVERY = 10  # one timed step in this many brackets its compositing kernels with HIP events
STAGES = ("preprocess", "bin_and_sort", "tile_ranges", "composite_fwd", "composite_bwd")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model() -> str:
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_threads() -> int:
    """Host threads for the threaded oracle run: the CPUs this process may
    use, capped by OMP_NUM_THREADS when it is set."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    try:
        n = min(n, int(os.environ.get("OMP_NUM_THREADS", n)))
    except ValueError:
        pass
    return max(1, n)


def _oracle_frames(name: str, min_seconds: float, max_frames: int):
    """Whole frames of the workload through the oracle, stage by stage:
    (frames, total seconds, median ms per stage)."""
    import numpy as np

    import oracle
    import synth
    scene, cam, dLdI = synth.config_scene(name)
    if dLdI is None:
        dLdI = synth.upstream_gradient(3001, cam["width"], cam["height"])
    frames, total = 0, 0.0
    stage = {s: [] for s in STAGES}
    while frames < max_frames and (frames == 0 or total < min_seconds):
        t = [time.perf_counter()]
        pre = oracle.preprocess(cam, scene)
        t.append(time.perf_counter())
        keys, point_list = oracle.bin_and_sort(cam, pre["xy_depth"], pre["tiles_touched"])
        t.append(time.perf_counter())
        ranges = oracle.tile_ranges(cam, keys)
        t.append(time.perf_counter())
        fwd = oracle.composite_fwd(cam, ranges, point_list, pre["xy_depth"], pre["conic_op"], pre["rgb"])
        t.append(time.perf_counter())
        oracle.composite_bwd(cam, scene["n"], ranges, point_list, pre["xy_depth"], pre["conic_op"], pre["rgb"],
                             fwd["final_T"], fwd["n_contrib"], dLdI)
        t.append(time.perf_counter())
        for i, s in enumerate(STAGES):
            stage[s].append(1e3 * (t[i + 1] - t[i]))
        total += t[-1] - t[0]
        frames += 1
    return frames, total, {s: round(float(np.median(v)), 3) for s, v in stage.items()}


def cpu_baseline(name: str, min_seconds: float = 10.0, max_frames: int = 8):
    """Time the oracle (as it stands) on whole frames of the same workload,
    forward and backward: single-threaded (the reported value), repeating the
    frame until about min_seconds of CPU work have been timed; then its
    threaded run (the preprocess and compositing over all host threads the
    process may use; the binning and sort stay single-threaded) for about
    half that time."""
    import oracle
    frames, total, stage_ms = _oracle_frames(name, min_seconds, max_frames)
    threads = oracle_threads()
    try:
        oracle.set_threads(threads)
        mframes, mtotal, mstage_ms = _oracle_frames(name, min_seconds / 2, 4 * max_frames)
    finally:
        oracle.set_threads(1)
    return {"value": round(frames / total, 4), "unit": "frames/s", "cores": 1, "kind": "oracle",
            "sample": f"{frames} full {name} frame(s) (preprocess, bin, sort, ranges, forward and "
                      f"backward compositing), single-threaded, {total:.2f} s in total",
            "seconds": round(total, 3), "stage_ms_median": stage_ms, "cpu_model": cpu_model(),
            "threaded": {"value": round(mframes / mtotal, 4), "unit": "frames/s", "threads": threads,
                         "sample": f"{mframes} full {name} frame(s), preprocess and compositing over "
                                   f"{threads} threads (OpenMP), {mtotal:.2f} s in total",
                         "seconds": round(mtotal, 3), "stage_ms_median": mstage_ms}}


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "k_composite_bwd_cfg2_hbm_traffic.md")
KERNEL_SOURCE = os.path.join(ROOT, "gaussian_splatting_tile_amd", "csrc", "composite.hip")
BIN_TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "bin_and_sort_cfg2_hbm_traffic.md")
BIN_SOURCE = os.path.join(ROOT, "gaussian_splatting_tile_amd", "csrc", "binning.hip")


def _summary_figure(summary: str, source: str, workload: str, field: str):
    """One machine-readable figure (`- field: `value``) of a committed
    rocprofv3 counter summary, or None when the summary is missing, covers
    another workload, or was taken on a different version of the source it
    names by hash."""
    import hashlib
    try:
        text = open(summary).read()
        src = hashlib.sha256(open(source, "rb").read()).hexdigest()
    except OSError:
        return None
    fields = dict(re.findall(r"^- (\w+): `([^`]*)`", text, flags=re.M))
    if fields.get("workload") != workload or fields.get("source_sha256") != src:
        return None
    try:
        return float(fields[field])
    except (KeyError, ValueError):
        return None


def measured_traffic(workload: str):
    """HBM bytes per launch of the backward compositing kernel, from the
    committed counter summary (FETCH_SIZE and WRITE_SIZE, each scaled by what
    the counter reads for a copy of known size)."""
    return _summary_figure(TRAFFIC_SUMMARY, KERNEL_SOURCE, workload, "hbm_bytes_per_launch")


def measured_binning_traffic(workload: str):
    """HBM bytes of one gs_bin_and_sort_async call (every kernel it launches,
    square spans), from the committed counter summary, scaled as above."""
    return _summary_figure(BIN_TRAFFIC_SUMMARY, BIN_SOURCE, workload, "hbm_bytes_per_call")


def sort_dup_bytes(n: int, E: int, TX: int, TY: int) -> int:
    """Bytes the binning of this design must move at the least: per splat,
    its depth read (4 B) and key/id pair written (8 B), four 8-bit passes
    over the pairs (16 B each), the tile count read and entry offset written
    in the last pass (8 B), and the duplication's reads (record 16 B, offset
    and id 8 B); per entry, the (key, id) written by the duplication (12 B)
    and every 8-bit pass over the tile-id bits (12 B read, 12 B written)."""
    tile_bits = max(1, (TX * TY - 1).bit_length())
    passes = -(-tile_bits // 8)
    return n * (4 + 8 + 4 * 16 + 8 + 24) + E * (12 + 24 * passes)


def sort_dup_record(n, E, TX, TY, seconds, counter_bytes):
    """The binning against the HBM roofline: algorithmic bytes (above) and,
    when a current counter summary exists, the measured HBM bytes, each over
    the stage's median time."""
    alg = sort_dup_bytes(n, E, TX, TY)
    rec = {"ms": round(seconds * 1e3, 4), "alg_bytes": alg, "alg_GBps": round(alg / seconds / 1e9, 1),
           "alg_frac": round(alg / seconds / PEAK_HBM, 4), "counter_bytes": None, "counter_GBps": None,
           "counter_frac": None}
    if counter_bytes:
        rec.update(counter_bytes=int(counter_bytes), counter_GBps=round(counter_bytes / seconds / 1e9, 1),
                   counter_frac=round(counter_bytes / seconds / PEAK_HBM, 4))
    return rec


def copy_calibration(mib: int, repeats: int = 3):
    """Device-to-device copies of a known size, so that a counter run over
    this process also records what FETCH_SIZE and WRITE_SIZE read for a
    plain copy kernel (mib MiB read and mib MiB written per launch)."""
    import torch
    n = (mib << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(repeats):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: {repeats} copies of {mib} MiB ({n * 4} bytes read and written each)")
    del src, dst


def bench_views(args):
    """The training-step shape: one step renders 16 views of a 300k-Gaussian
    scene forward and backward (dL/dI = sign(I - I_ref), I_ref rendered once
    from a second scene), enqueued without host waits and replayed as one HIP
    graph. frames/s counts views."""
    import numpy as np
    import torch

    import synth
    import gaussian_splatting_tile_amd as gs

    dev = torch.device("cuda:0")
    n_views = 16
    scene_np, _, _ = synth.config_scene("cfg4")
    ref_np, _, _ = synth.config_scene("cfg4_ref")
    cams = [synth.config_scene("cfg4", view=v)[1] for v in range(n_views)]
    sc, ref_sc = gs.Scene.from_numpy(scene_np, device=dev), gs.Scene.from_numpy(ref_np, device=dev)
    rast = gs.Rasterizer(device=dev, capacity=1 << 21)
    refs, E_max = [], 0
    for cam in cams:
        out = rast.forward(cam, ref_sc)
        refs.append(out["image"].clone())
        E_max = max(E_max, rast.forward(cam, sc)["n_entries"])
    torch.cuda.synchronize()

    if args.batch == "stack":
        # the 16 views as bands of stacked frames: --streams stacks, one launch sequence each
        ref_all = torch.stack(refs)

        def loss_grad(first, image, out):
            out.copy_(image).sub_(ref_all[first:first + image.shape[0]]).sign_()

        per_stack = -(-n_views // max(1, min(args.streams, n_views)))
        batch = gs.ViewStack(cams, sc, capacity=int(E_max * per_stack * 1.25) + 1024, device=dev,
                             streams=args.streams)
    else:
        def loss_grad(i, image, out):
            out.copy_(image).sub_(refs[i]).sign_()

        batch = gs.ViewBatch(cams, sc, capacity=int(E_max * 1.25) + 1024, device=dev, streams=args.streams,
                             chunked=args.backward == "chunked")
    batch.enqueue(loss_grad)
    E = batch.check()
    st = torch.cuda.current_stream()
    # eager: every call launched from the host each step
    for _ in range(args.warmup):
        batch.enqueue(loss_grad)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        batch.enqueue(loss_grad)
    torch.cuda.synchronize()
    eager_s = (time.perf_counter() - t0) / args.steps
    # graph: the whole step recorded once
    batch.capture(loss_grad)
    for _ in range(args.warmup):
        batch.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(st)
    for _ in range(args.steps):
        batch.replay()
    e1.record(st)
    torch.cuda.synchronize()
    graph_s = (time.perf_counter() - t0) / args.steps
    if batch.check() != E:
        raise SystemExit("entry counts changed between runs")
    return {
        "metric": METRIC, "value": round(n_views / graph_s, 3), "unit": "frames/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(1e3 * graph_s, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"cfg4: {WORKLOADS['cfg4']}", "n_gaussians": sc.n, "views_per_step": n_views,
                   "batch": args.batch, "streams": args.streams,
                   "backward": args.backward,
                   "width": 400, "height": 400, "entries_total": int(sum(E)) if isinstance(E, list) else int(E)},
        "secondary": {"eager_frames_per_s": round(n_views / eager_s, 3),
                      "graph_event_ms_per_step": round(e0.elapsed_time(e1) / args.steps, 4)},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="cfg2", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tile-order", choices=("heavy-first", "index"), default="heavy-first",
                    help="tile schedule of the compositing kernels (results are identical)")
    ap.add_argument("--backward", choices=("chunked", "whole"), default="chunked",
                    help="backward compositing over 256-entry chunks of each list (from the forward's "
                         "checkpoints) or over whole lists (results agree to float32 rounding)")
    ap.add_argument("--batch", choices=("stack", "streams"), default="stack",
                    help="cfg4: the 16 views as bands of --streams stacked frames (one launch sequence "
                         "per stack), or one launch sequence per view spread over --streams streams")
    ap.add_argument("--streams", type=int, default=4,
                    help="cfg4: streams the 16 views are spread over (fork/join inside the graph)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run device copies of this many MiB (for HBM counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path. Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import gaussian_splatting_tile_amd as gs

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    if args.workload == "cfg4":
        result = bench_views(args)
        if not args.no_cpu_baseline:
            log("[bench] timing the oracle on the host (cpu_baseline, one 400x400 view per frame)")
            result["cpu_baseline"] = cpu_baseline("cfg4")
        print(json.dumps(result), flush=True)
        return
    if args.copy_calibration_mib > 0:
        copy_calibration(args.copy_calibration_mib)

    log(f"[bench] generating {args.workload}")
    scene_np, cam, dLdI_np = synth.config_scene(args.workload)
    if dLdI_np is None:
        dLdI_np = synth.upstream_gradient(3001, cam["width"], cam["height"])
    scene = gs.Scene.from_numpy(scene_np, device=dev)
    dLdI = torch.from_numpy(dLdI_np).to(dev)
    c = gs.camera(cam)
    W, H = cam["width"], cam["height"]
    TX, TY = gs.tiles_xy(cam)
    n = scene.n

    # Preallocated outputs: the timed loop allocates nothing.
    f32, i32 = torch.float32, torch.int32
    pre = dict(xy_depth=torch.empty((n, 4), dtype=f32, device=dev),
               conic_op=torch.empty((n, 4), dtype=f32, device=dev),
               rgb=torch.empty((n, 4), dtype=f32, device=dev),
               tiles_touched=torch.empty((n,), dtype=i32, device=dev))
    bins = gs.BinBuffers(dev, capacity=1 << 16)
    ranges = torch.empty((TX * TY, 2), dtype=i32, device=dev)
    order = torch.empty((TX * TY,), dtype=i32, device=dev) if args.tile_order == "heavy-first" else None
    fwd = dict(image=torch.empty((3, H, W), dtype=f32, device=dev),
               final_T=torch.empty((H, W), dtype=f32, device=dev),
               n_contrib=torch.empty((H, W), dtype=i32, device=dev))
    grads = dict(grad_mean2d=torch.empty((n, 2), dtype=f32, device=dev),
                 grad_conic_op=torch.empty((n, 4), dtype=f32, device=dev),
                 grad_rgb=torch.empty((n, 4), dtype=f32, device=dev))

    # Units of work of this frame (computed once, outside the timed region).
    gs.preprocess(c, scene.means, scene.scales, scene.quats, scene.opacity, scene.sh, scene.sh_degree,
                  scene.rgb, out=pre)
    keys, pl, E = gs.bin_and_sort(c, pre["xy_depth"], pre["tiles_touched"], bins)
    bins._ensure(int(E * 1.1) + 1024)  # headroom so timed frames never regrow
    chunked = args.backward == "chunked"
    ckpt = torch.empty((gs.ckpt_rows(bins.capacity), 4), dtype=f32, device=dev) if chunked else None
    chunks = torch.empty((gs.chunk_words(cam, bins.capacity),), dtype=i32, device=dev) if chunked else None
    # the forward over the chunk schedule on small tile grids with long lists,
    # as the Rasterizer chooses it
    sched_fwd = chunked and gs.scheduled_forward(cam) and E > 256 * TX * TY
    part = torch.empty((gs.part_bytes(cam, bins.capacity),), dtype=torch.uint8, device=dev) if sched_fwd else None
    gs.tile_ranges(cam, keys, E, out=ranges)
    probe = gs.composite_fwd(cam, ranges, pl, pre["xy_depth"], pre["conic_op"], pre["rgb"],
                             with_examined=True)
    torch.cuda.synchronize()
    evals_fwd = int(probe["n_examined"].to(torch.int64).sum())
    evals_bwd = int(probe["n_contrib"].to(torch.int64).sum())
    del probe
    log(f"[bench] n={n} E={E} evals fwd={evals_fwd} bwd={evals_bwd}")

    def step(marks=None, stage_marks=False, tile_test=0):
        """One frame. `marks` (a list) receives HIP events recorded on the
        kernels' stream: around the two compositing kernels, or at every
        stage boundary when stage_marks is set."""
        def mark(always):
            if marks is not None and (always or stage_marks):
                e = torch.cuda.Event(enable_timing=True)
                e.record(stream)
                marks.append(e)
        mark(False)
        gs.preprocess(c, scene.means, scene.scales, scene.quats, scene.opacity, scene.sh,
                      scene.sh_degree, scene.rgb, out=pre, tile_test=tile_test)
        mark(False)
        k, p = gs.bin_and_sort_async(c, pre["xy_depth"], pre["tiles_touched"], bins, conic_op=pre["conic_op"],
                                     tile_test=tile_test)
        mark(False)
        gs.tile_ranges_async(c, bins, out=ranges, order=order, chunks=chunks)
        mark(True)
        gs.composite_fwd(c, ranges, p, pre["xy_depth"], pre["conic_op"], pre["rgb"], out=fwd, order=order,
                         ckpt=ckpt, capacity=bins.capacity, chunks=chunks if sched_fwd else None, part=part)
        mark(True)
        gs.composite_bwd(c, n, ranges, p, pre["xy_depth"], pre["conic_op"], pre["rgb"],
                         fwd["final_T"], fwd["n_contrib"], dLdI, out=grads, order=order, chunks=chunks,
                         image=fwd["image"] if chunked else None, ckpt=ckpt, capacity=bins.capacity)
        mark(True)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup done, timing {args.steps} steps")
    # Timed region. Each event record holds the queue (the next dispatch
    # waits for its timestamp, about 5 us of idle GPU), so the compositing
    # kernels are bracketed with events on every EVENT_EVERY-th step only:
    # events on every step slowed the measured frames by 10 us. Every step
    # runs the same work, so the sampled launches give the kernels' mean
    # duration; the stage breakdown is taken afterwards.
    timed = []
    t0 = time.perf_counter()
    for i in range(args.steps):
        if i % EVENT_EVERY == 0:
            m = []
            step(m)
            timed.append(m)
        else:
            step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    E_last = bins.entries()
    if E_last != E:  # every timed frame binned the same scene into enough capacity
        raise SystemExit(f"entry count {E_last} != {E} (capacity {bins.capacity})")
    fwd_ms = [m[0].elapsed_time(m[1]) for m in timed]
    bwd_ms = [m[1].elapsed_time(m[2]) for m in timed]

    # Stage breakdown (not part of the timed region): events at every boundary.
    staged = []
    for _ in range(args.steps):
        m = []
        step(m, stage_marks=True)
        staged.append(m)
    torch.cuda.synchronize()
    stage_ms = {}
    for i, s in enumerate(STAGES):
        vals = [m[i].elapsed_time(m[i + 1]) for m in staged]
        stage_ms[s] = (float(np.median(vals)), float(np.mean(vals)), float(np.percentile(vals, 10)),
                       float(np.percentile(vals, 90)))
    # The same frames with the ellipse tile test (identical image, shorter
    # lists): timed the same way, reported as a secondary figure.
    for _ in range(args.warmup):
        step(tile_test=1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(tile_test=1)
    torch.cuda.synchronize()
    ellipse_fps = args.steps / (time.perf_counter() - t0)
    E_ellipse = bins.entries()
    step()  # back to the square spans for what follows
    torch.cuda.synchronize()

    # The projection backward (gs_preprocess_bwd) is the step after this
    # path: timed on its own, over the same frame's splat gradients.
    pgrads = gs.preprocess_bwd(c, scene.means, scene.scales, scene.quats, scene.sh, scene.sh_degree,
                               pre["tiles_touched"], grads["grad_mean2d"], grads["grad_conic_op"],
                               grads["grad_rgb"])
    pb = []
    for _ in range(args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        gs.preprocess_bwd(c, scene.means, scene.scales, scene.quats, scene.sh, scene.sh_degree,
                          pre["tiles_touched"], grads["grad_mean2d"], grads["grad_conic_op"],
                          grads["grad_rgb"], out=pgrads)
        e1.record(stream)
        pb.append((e0, e1))
    torch.cuda.synchronize()
    pbwd_s = float(np.mean([a.elapsed_time(b) for a, b in pb])) * 1e-3
    n_coef = (scene.sh_degree + 1) ** 2 if scene.sh is not None else 1
    # per Gaussian: means, scales, quats, tiles_touched, the three upstream
    # records (8 + 16 + 16 B) and the SH (or RGB) read; eleven gradient
    # floats and the SH (or RGB) gradient written
    pbwd_bytes = n * (44 + 40 + 12 * n_coef + 44 + 12 * n_coef)

    # The appearance MLP (8 latents, 32 hidden units) over the same
    # Gaussians, forward and backward: the alternative colour source.
    gen = torch.Generator(device=dev).manual_seed(5)
    app_L, app_H = 8, 32
    latent = torch.randn((app_L, n), device=dev, generator=gen)
    app_w = 0.3 * torch.randn((gs.appearance_params(app_L, app_H),), device=dev, generator=gen)
    app_rgb = gs.appearance_fwd(c, scene.means, latent, app_w, app_H)
    app_g = gs.appearance_bwd(c, scene.means, latent, app_w, app_H, app_rgb)
    ev = []
    for _ in range(args.steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        gs.appearance_fwd(c, scene.means, latent, app_w, app_H, out=app_rgb)
        e[1].record(stream)
        gs.appearance_bwd(c, scene.means, latent, app_w, app_H, app_rgb, out=app_g)
        e[2].record(stream)
        ev.append(e)
    torch.cuda.synchronize()
    app_fwd_ms = float(np.mean([x[0].elapsed_time(x[1]) for x in ev]))
    app_bwd_ms = float(np.mean([x[1].elapsed_time(x[2]) for x in ev]))

    ms_per_step = 1e3 * elapsed / args.steps
    fps = args.steps / elapsed

    # Dominant kernel: the backward compositing (ALU-bound: no dense
    # contraction, so no MFMA). achieved = algorithmic flops / mean launch time.
    bwd_s = float(np.mean(bwd_ms)) * 1e-3
    fwd_s = float(np.mean(fwd_ms)) * 1e-3
    achieved = evals_bwd * FLOPS_PER_BWD_EVAL / bwd_s
    sort_s = stage_ms["bin_and_sort"][1] * 1e-3
    result = {
        "metric": METRIC,
        "value": round(fps, 3),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {WORKLOADS[args.workload]}", "tile_order": args.tile_order,
                   "backward": args.backward,
                   "forward": "chunk schedule" if sched_fwd else "whole lists",
                   "n_gaussians": n, "width": W, "height": H, "n_entries": E,
                   "evals_fwd": evals_fwd, "evals_bwd": evals_bwd},
        "pixel_splat_evals_per_s": round((evals_fwd + evals_bwd) * fps, 1),
        "stage_ms_median": {s: round(v[0], 4) for s, v in stage_ms.items()},
        "stage_ms_p10_p90": {s: [round(v[2], 4), round(v[3], 4)] for s, v in stage_ms.items()},
        "timed_kernel_ms_mean": {"composite_fwd": round(fwd_s * 1e3, 4),
                                 "composite_bwd": round(bwd_s * 1e3, 4)},
        "roofline": {"bound": "alu", "kernel": "k_composite_bwd<true>" if chunked else "k_composite_bwd<false>",
                     "achieved": round(achieved / 1e12, 4), "peak": PEAK_FP32_VECTOR / 1e12,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP32_VECTOR, 5),
                     "traffic": measured_traffic(args.workload) if chunked else None,
                     "per_unit": f"{FLOPS_PER_BWD_EVAL:.0f} flop per backward pixel-splat eval "
                                 f"x {evals_bwd} evals per launch"},
        "secondary": {
            "composite_fwd_tflops": round(evals_fwd * FLOPS_PER_FWD_EVAL / fwd_s / 1e12, 4),
            "composite_fwd_frac": round(evals_fwd * FLOPS_PER_FWD_EVAL / fwd_s / PEAK_FP32_VECTOR, 5),
            "entries_per_s": round(E / sort_s, 1),
            "sort_dup": sort_dup_record(n, E, TX, TY, stage_ms["bin_and_sort"][0] * 1e-3,
                                        measured_binning_traffic(args.workload)),
            "ellipse_tile_test_frames_per_s": round(ellipse_fps, 3),
            "ellipse_tile_test_n_entries": E_ellipse,
            "preprocess_bwd_ms": round(pbwd_s * 1e3, 4),
            "appearance_mlp_8x32_fwd_ms": round(app_fwd_ms, 4),
            "appearance_mlp_8x32_bwd_ms": round(app_bwd_ms, 4),
            "preprocess_bwd_hbm_frac": round(pbwd_bytes / pbwd_s / PEAK_HBM, 4),
        },
        "baseline_context": {"value": 25.8, "unit": "frames/s", "hardware": "Tesla T4",
                             "note": "derived 1000/(4.60 ms fwd + 34.12 ms bwd) for the pages' "
                                     "160k-Gaussian gallery scene at 1920x1080; another machine "
                                     "and scene, context only"},
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host (cpu_baseline)")
        result["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
