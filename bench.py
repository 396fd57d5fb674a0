"""Benchmark: train steps/s of one 3D Gaussian Splatting training step on one
MI355X (forward + backward + sparse Adam), on the mid workload: 1,000,000
seeded synthetic Gaussians, four 1920x1080 ring views per step.

    python bench.py [--steps K] [--warmup W] [--config 2] [--no-cpu-baseline]

Prints ONE JSON line.  `value` = steps/s with every input resident in HBM
when the timed region starts.  Protocol: W warm-up steps from the seeded
parameters; the state they leave (parameters, Adam moments, step count) is
kept as a device copy and restored before every block of RESTORE_EVERY
steps, outside the timed region, so every block trains the same ten steps
from the same scene instead of a drifting one.  Each block is bracketed by device
synchronisations; `value` = K / (sum of the blocks' wall times); every step
is also bracketed by HIP events on the caller's stream (median reported).
Inside the timed blocks HIP events on the stream the library launches on
bracket one raster backward per step (the dominant kernel; the view
rotates with the step and the block), whose roofline uses them: an event
pair between two launches idles the stream for several microseconds, so
nothing else is bracketed there.  The steps run as a training loop runs
them, without the per-tile processed counts.
A counting pass (one block with the raster backward's visit counter on,
outside the timed region) gives the back-propagated (pixel, entry) pairs of
the timed launches, the roofline's unit.  The other stages' times come from
a block with every stage bracketed, and the step without the next step's
first preprocess fused into the Adam pass from another block.
`cpu_baseline` is the oracle timed on the host's cores over one step of the
same workload (bounded: see cpu_baseline).  `view_coupling` times the
coupling graph of 1,024 flight views over the aerial scene (see
view_coupling_bench).
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "train steps/sec (fwd+bwd+Adam), 1M Gaussians @1080p; % of HBM peak"
HBM_PEAK = 8.0e12              # bytes/s, MI355X HBM3E
CUS, CLOCK = 256, 2.4e9        # MI355X compute units, peak engine clock
VALU_PEAK = CUS * 64 * CLOCK   # 32-bit VALU operations/s: one wave64 instruction per CU per clock
TILE = 16
RESTORE_EVERY = 10

# Algorithmic 32-bit operations of one back-propagated (pixel, entry) pair:
# the canonical rule's arithmetic once per pair that composited the entry
# (mul/add/sub/min/fma/rcp/rint/ldexp = 1 each):
#   dx, dy 2 + power 5 + written exp 12 + alpha 2 + 1 - alpha and T / (1 - alpha) 3
#   + weight 1 + dL/dalpha 7 + suffix colour 6 + dL/dpower, dL/dopacity 2
#   + mean / conic products 5 + colour gradients 3 + nine sums 9        = 57
# and of one composited pair in the forward:
#   dx, dy 2 + power 5 + exp 12 + alpha 2 + T (1 - alpha) 2 + weight 1
#   + three colour fma 3                                                 = 27
OPS_PER_VISIT = {"render_fwd": 27, "render_bwd": 57}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic_bytes(N, views, U):
    """Compulsory HBM bytes of one step (each stage's inputs read once, its
    outputs written once; the sort at its floor of one read + one write of
    each pair; the rasterisers on the processed prefix M_proc only), per
    the scope table: per view with V visible, M pairs, P pixels, T tiles,
    then Adam once over the U union rows.  Returns (total, per-stage)."""
    st = {k: 0.0 for k in ("preprocess", "bin_sort", "render_fwd", "loss", "render_bwd", "project_bwd",
                           "sparse_adam")}
    for v in views:
        V, M, Mp, P, T = v["V"], v["M"], v["M_proc"], v["P"], v["T"]
        st["preprocess"] += 288 * N + 16 * N                  # params in, records out; scan + visible list
        st["bin_sort"] += 16 * V + 12 * M + 24 * M + 4 * M + 8 * T   # duplication, sort floor, ranges
        st["render_fwd"] += 40 * Mp + 20 * P
        st["loss"] += 36 * P
        st["render_bwd"] += 40 * Mp + 20 * P + 72 * V
        st["project_bwd"] += 744 * V
    st["sparse_adam"] = 1892 * U
    return sum(st.values()), st


def recorded_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a copy kernel's reading), or
    None when the summary is for another workload or the kernel's sources
    have changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.json")
    try:
        with open(path) as f:
            rec = json.load(f)["kernels"][kernel]
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
    except (OSError, KeyError, ValueError):
        return None
    return float(rec["bytes_per_launch"]) if h.hexdigest() == rec["sources_sha256"] else None


def cpu_baseline(work, budget_s=30.0):
    """The oracle as it stands, timed on the host's cores over one training
    step of the same workload at its initial parameters: per view the plain
    one-view stage (projection once, binning into tile lists, render, loss,
    backward; no error-magnitude pass), gradients summed over the views,
    then Adam over the union of the visible sets.  Views are taken in order
    until the step is complete or `budget_s` has passed; the view part is
    then scaled by (views in the step) / (views run).  Beside it, the same
    one-view stage single-threaded on the small workload's view (1297x840,
    100,000 Gaussians)."""
    import numpy as np

    import oracle
    import synth
    t = time.perf_counter
    nv = len(work.cameras)
    grads = np.zeros((59, work.n))
    seen = np.zeros(work.n, bool)
    t0 = t()
    done = 0
    for cam, tgt in zip(work.cameras, work.targets):
        oracle.train_view(work.params, cam, tgt, work.w_l1, work.w_ssim, grads)
        done += 1
        if t() - t0 > budget_s:
            break
    t_views = (t() - t0) * nv / done
    for cam in work.cameras:         # (the union, outside the timed part)
        seen |= oracle.preprocess(work.params, cam)["visible"]
    rows = np.flatnonzero(seen).astype(np.int32)
    zeros = np.zeros_like(grads)
    t1 = t()
    oracle.adam(work.params, grads, zeros, zeros, rows, work.lr, work.beta1, work.beta2, work.eps)
    t_adam = t() - t1
    t_step = t_views + t_adam
    threads = oracle.num_threads()
    small = synth.workload(1)
    oracle.set_threads(1)
    try:
        t2 = t()
        oracle.train_view(small.params, small.cameras[0], small.targets[0], small.w_l1, small.w_ssim)
        t_one = t() - t2
    finally:
        oracle.set_threads(threads)
    return {"value": 1.0 / t_step, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": f"one step at the initial parameters: {done} of {nv} views (full size, one projection per "
                      f"view, no error-magnitude pass) in {t_views * done / nv:.1f} s" +
                      (f", scaled x{nv / done:.2f}" if done < nv else "") +
                      f", Adam over {rows.shape[0]:,} rows in {t_adam:.1f} s",
            "single_thread": {"value": 1.0 / t_one, "unit": "steps/s", "cores": 1,
                              "sample": "one training step of the small workload (100,000 Gaussians, one "
                                        f"1297x840 view, sparse Adam not included): {t_one:.1f} s"}}


def view_coupling_bench(calls=20, views=1024, width=1920, height=1080):
    """gs_view_overlap (counts + Jaccard weights) over the visible lists of
    ``views`` flight views of the aerial scene (3,000,000 Gaussians), timed
    per call with HIP events on the stream it launches on; its oracle timed
    on three of the lists."""
    import numpy as np
    import torch

    import differentiable_gaussian_splatting_dgs_amd as gs
    import oracle
    import synth

    log(f"[bench] view coupling: aerial scene, {views} flight views")
    work = synth.workload(3)
    cams = synth.flight_cameras(width, height, views)
    vc = gs.ViewCoupling(work.n, views, "cuda:0")
    dp = torch.from_numpy(work.params).cuda()
    vc.visible_lists(dp, work.n, cams)
    vc.overlap()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for a, b in ev:
        a.record(st)
        vc.overlap()
        b.record(st)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    words = (work.n + 31) // 32
    pairs = views * (views + 1) // 2
    ops = 2.0 * pairs * words          # one AND and one popcount-accumulate per word of a pair
    counts = vc.counts.cpu().numpy()
    del vc, dp
    torch.cuda.empty_cache()
    # the oracle on three of the lists (their own visible lists, untimed)
    sample = [0, 417, 1023]
    olists = [oracle.visible_list(work.params, cams[v]) for v in sample]
    t0 = time.perf_counter()
    oracle.view_overlap(olists)
    t_or = time.perf_counter() - t0
    return {
        "workload": f"aerial scene: {work.n:,} Gaussians, {views} flight views of {width}x{height}, "
                    "visible lists from the preprocess",
        "views": views, "n": work.n, "pairs": pairs, "mean_list_len": float(counts.mean()),
        "ms_per_call": ms, "pairs_per_s": pairs / (ms * 1e-3), "calls": calls,
        "roofline": {"kernel": "k_overlap", "bound": "alu", "achieved": ops / (ms * 1e-3) / 1e12,
                     "peak": VALU_PEAK / 1e12, "unit": "Tops/s (32-bit VALU)",
                     "frac": ops / (ms * 1e-3) / VALU_PEAK, "traffic": None,
                     "ops_per_call": ops, "timed": "whole gs_view_overlap call (zero fill, bitmaps, "
                                                   "pair tiles, weights)"},
        "cpu_oracle": {"value": 6 / t_or, "unit": "pairs/s", "cores": 1, "kind": "oracle",
                       "sample": "np.intersect1d over the 6 pairs (with the diagonal) of 3 of the lists"},
    }


def shard_bench(step, work, K=8, calls=20):
    """gs_tile_partition, gs_pack_records and gs_unpack_grads on view 0 of
    the step's workload, cut into K tile blocks by the rasteriser's
    per-tile counts of the last step; each call timed with HIP events."""
    import numpy as np
    import torch

    import differentiable_gaussian_splatting_dgs_amd as gs

    log(f"[bench] tile blocks and the all-to-all's two ends, K={K}")
    vw = step.views[0]
    n = step.n
    proj = torch.empty((n, gs.GS_PROJ_WORDS), dtype=torch.float32, device=step.device)
    vis = torch.empty(n, dtype=torch.int32, device=step.device)
    cnt = torch.zeros(1, dtype=torch.int64, device=step.device)
    ws_pre = torch.empty(gs.gs_workspace_size(gs.GS_OP_PREPROCESS, n), dtype=torch.uint8, device=step.device)
    gs.gs_preprocess(step.params, n, step.ld, vw.cam, proj, vis, cnt, None, ws_pre)
    cost = vw.tile_processed
    bounds = torch.empty(K + 1, dtype=torch.int32, device=step.device)
    offs = torch.empty(K + 1, dtype=torch.int64, device=step.device)
    ws = torch.empty(gs.gs_workspace_size(gs.GS_OP_PACK, n, K), dtype=torch.uint8, device=step.device)
    gs.gs_tile_partition(cost, vw.T, K, bounds)
    gs.gs_pack_records(proj, n, vis, cnt, vw.W, vw.H, bounds, K, 0, offs, None, None, ws)
    total = int(offs[K].item())
    idx = torch.empty(total, dtype=torch.int32, device=step.device)
    rec = torch.empty((total, gs.GS_PROJ_WORDS), dtype=torch.float32, device=step.device)
    recv = torch.randn((total, gs.GS_GRAD2D_WORDS), dtype=torch.float32, device=step.device)
    grad = torch.zeros((n, gs.GS_GRAD2D_WORDS), dtype=torch.float32, device=step.device)
    st = torch.cuda.current_stream()
    calls_by = {
        "partition": lambda: gs.gs_tile_partition(cost, vw.T, K, bounds),
        "pack": lambda: gs.gs_pack_records(proj, n, vis, cnt, vw.W, vw.H, bounds, K, total, offs, idx, rec, ws),
        "unpack": lambda: gs.gs_unpack_grads(recv, offs, idx, K, total, grad, n),
    }
    ms = {}
    for name, fn in calls_by.items():
        fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
        for a, b in ev:
            a.record(st)
            fn()
            b.record(st)
        torch.cuda.synchronize()
        ms[name] = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    V = int(cnt.item())
    pack_bytes = 68.0 * V + 68.0 * total          # index + record in, per visible; index + record out, per entry
    unpack_bytes = 148.0 * total                   # row + index in, Gaussian row read and written, per entry
    return {
        "workload": f"{work.name} view 0: {n:,} Gaussians, {vw.W}x{vw.H}, {K} tile blocks by the last "
                    "step's per-tile processed counts",
        "blocks": K, "visible": V, "packed": total, "bounds": bounds.cpu().tolist(),
        "ms_per_call": ms,
        "pack_roofline": {"bound": "hbm", "achieved": pack_bytes / (ms["pack"] * 1e-3) / 1e9,
                          "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                          "frac": pack_bytes / (ms["pack"] * 1e-3) / HBM_PEAK, "bytes_per_call": pack_bytes},
        "unpack_roofline": {"bound": "hbm", "achieved": unpack_bytes / (ms["unpack"] * 1e-3) / 1e9,
                            "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                            "frac": unpack_bytes / (ms["unpack"] * 1e-3) / HBM_PEAK,
                            "bytes_per_call": unpack_bytes},
    }


def densify_bench(step, calls=20):
    """gs_densify_stats (one view's visible rows) and gs_densify over the
    step's parameters and Adam state, with seeded statistics whose
    thresholds clone or split about a fifth of the Gaussians; each call
    timed with HIP events."""
    import numpy as np
    import torch

    import differentiable_gaussian_splatting_dgs_amd as gs

    log("[bench] densification")
    n, dev = step.n, step.device
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    grad2d = torch.randn((n, gs.GS_GRAD2D_WORDS), generator=gen, device=dev)
    accum = torch.zeros(n, dtype=torch.float32, device=dev)
    denom = torch.zeros(n, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream()

    def timed(fn):
        fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
        for a, b in ev:
            a.record(st)
            fn()
            b.record(st)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ev]))

    ms_stats = timed(lambda: gs.gs_densify_stats(grad2d, step.vis_idx[0], step.vis_count[0:1], n, accum, denom))
    p = step.params[:, :n]
    g = accum / denom.clamp(min=1).float()
    thr = float(torch.quantile(g[:1 << 20], 0.8).item())
    lst = float(torch.quantile(p[3:6, :1 << 20].max(0).values, 0.5).item())
    lgt = float(torch.quantile(p[10, :1 << 20], 0.05).item())
    normals = torch.randn((2, 3, n), generator=gen, device=dev)
    ld_out = 2 * n
    out = [torch.empty((59, ld_out), dtype=torch.float32, device=dev) for _ in range(3)]
    out_n = torch.zeros(1, dtype=torch.int64, device=dev)
    ws = torch.empty(gs.gs_workspace_size(gs.GS_OP_DENSIFY, n), dtype=torch.uint8, device=dev)
    ms_dens = timed(lambda: gs.gs_densify(step.params, step.m, step.v, n, step.ld, accum, denom, normals, thr, lst,
                                          lgt, float(np.log(1.6)), out[0], out[1], out[2], ld_out, out_n, ws))
    N = int(out_n.item())
    dens_bytes = 3 * 236.0 * n + 3 * 236.0 * N + n * 13.0   # planes in and out, statistics and normals of a row
    return {
        "workload": f"step parameters and Adam state, {n:,} Gaussians; seeded statistics with thresholds at their "
                    "80th percentile (gradient), median (largest log-scale) and 5th percentile (opacity logit)",
        "n_out": N, "ms_per_call": {"stats_one_view": ms_stats, "densify": ms_dens},
        "densify_roofline": {"bound": "hbm", "achieved": dens_bytes / (ms_dens * 1e-3) / 1e9,
                             "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                             "frac": dens_bytes / (ms_dens * 1e-3) / HBM_PEAK, "bytes_per_call": dens_bytes},
    }


def recorded_step_traffic(workload):
    """Measured HBM bytes of one whole training step (FETCH_SIZE +
    WRITE_SIZE of every kernel of a step, scaled by a copy kernel's
    reading) from the committed counter summary, or None when the library's
    sources have changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.json")
    try:
        with open(path) as f:
            rec = json.load(f)["step"]
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
    except (OSError, KeyError, ValueError):
        return None
    return float(rec["bytes_per_step"]) if h.hexdigest() == rec["sources_sha256"] else None


def recorded_valu_issue(kernel, workload):
    """SQ_INSTS_VALU per launch of `kernel` from the committed counter
    summary (same source-hash rule as recorded_traffic), or None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"sq_counters_{workload}.json")
    try:
        with open(path) as f:
            rec = json.load(f)["kernels"][kernel]
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
    except (OSError, KeyError, ValueError):
        return None
    return float(rec["valu_insts_per_launch"]) if h.hexdigest() == rec["sources_sha256"] else None


def device_copy_GBps(nbytes=1 << 30, reps=10):
    """Measured device-to-device copy rate (bytes read + written per second)
    of a plain 1 GiB copy, for context beside the HBM peak."""
    import torch
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        b.copy_(a)
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    torch.cuda.empty_cache()
    return 2.0 * nbytes / (ms * 1e-3) / 1e9


def run_block(step, init, nsteps, timed_stages=None, timed_view=None):
    """`nsteps` training steps from the restored state `init` (restored
    before the clock starts), bracketed by device synchronisations; every
    step bracketed by HIP events on the caller's stream.  With
    timed_stages, those stages' launches are bracketed too (with
    timed_view(i), only view timed_view(i)'s launch in step i).  Returns
    the block's wall time (s), per-step event times (ms) and the stage
    events."""
    import torch
    step.load_state(init)
    step.timer = {} if timed_stages is not None else None
    step.timer_stages = timed_stages if timed_stages else None
    st = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nsteps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i, (a, b) in enumerate(evs):
        step.timer_views = None if timed_view is None else {timed_view(i)}
        a.record(st)
        step.step()
        b.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timer, step.timer, step.timer_stages, step.timer_views = step.timer, None, None, None
    return wall, [a.elapsed_time(b) for a, b in evs], timer


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-coupling", action="store_true", help="skip the view-coupling measurement")
    ap.add_argument("--quick", action="store_true",
                    help="the step's line only (no CPU baseline, side measurements or coupling): for profiling")
    ap.add_argument("--coupling-only", action="store_true",
                    help="print only the view-coupling measurement (for profiling it alone)")
    ap.add_argument("--shard-only", action="store_true",
                    help="one step, then print only the tile-block / all-to-all measurement")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the step's sharding over "
              "several GPUs is described in the design notes, not implemented)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import differentiable_gaussian_splatting_dgs_amd as gs
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.coupling_only:
        print(json.dumps({"view_coupling": view_coupling_bench()}), flush=True)
        return
    log(f"[bench] generating workload {args.config}")
    work = synth.workload(args.config)
    N = work.n
    nv = len(work.cameras)
    step = gs.from_workload(work, device="cuda:0", record_tiles=args.shard_only)
    torch.cuda.synchronize()
    if args.shard_only:
        step.step()
        torch.cuda.synchronize()
        print(json.dumps({"shard": shard_bench(step, work), "densify": densify_bench(step)}), flush=True)
        return
    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step.step()
    torch.cuda.synchronize()
    # the state every timed block starts from: after the warm-up steps
    init = step.state()

    # The objects alive after set-up (torch's, numpy's, the workload's) are
    # moved out of the garbage collector's generations: a full collection
    # over them takes tens of milliseconds on this interpreter and, landing
    # inside the timed loop, stalls the host between two kernel launches
    # while the GPU drains its queue.  Host-side only; every GPU stage runs.
    gc.collect()
    gc.freeze()

    # counting block (untimed): the RESTORE_EVERY steps every timed block
    # runs, with the raster backward's visit counter on; sizes per step
    log(f"[bench] counting block of {RESTORE_EVERY} steps")
    step.load_state(init)
    step.visits = torch.zeros(nv, dtype=torch.int64, device=step.device)
    step.record_tiles = True          # per-tile processed counts: M_proc
    sizes = []
    visits_by = []                    # [cycle step][view]: back-propagated pairs of that launch
    for _ in range(RESTORE_EVERY):
        step.step()
        torch.cuda.synchronize()
        visits_by.append([int(x) for x in step.visits.tolist()])
        step.visits.zero_()
        views = [dict(V=int(step.vis_count[k].item()), M=vw.num_pairs,
                      M_proc=int(vw.tile_processed.to(torch.int64).sum().item()), P=vw.W * vw.H, T=vw.T)
                 for k, vw in enumerate(step.views)]
        sizes.append((views, int(step.union_count.item())))
    step.visits = None
    step.record_tiles = False
    visits_per_launch = sum(map(sum, visits_by)) / (RESTORE_EVERY * nv)
    B_steps = [algorithmic_bytes(N, v, U) for v, U in sizes]
    B = float(np.mean([b[0] for b in B_steps]))
    B_stage = {k: float(np.mean([b[1][k] for b in B_steps])) for k in B_steps[0][1]}

    # timed blocks, restored before each
    log(f"[bench] timing {args.steps} steps in blocks of {RESTORE_EVERY}")
    # (one raster backward per step is bracketed, the view rotating with the
    # step and the block, so the sampled launches cover every (step, view)
    # of the cycle; their visits come from the counting block)
    wall, step_ms, raster_ev, sampled_visits = 0.0, [], {}, []
    left, blk = args.steps, 0
    while left > 0:
        k = min(RESTORE_EVERY, left)
        view_of = (lambda i, b=blk: (i + b) % nv)
        w, ms, ev = run_block(step, init, k, timed_stages={"render_bwd"}, timed_view=view_of)
        wall += w
        step_ms += ms
        for name, pairs in ev.items():
            raster_ev.setdefault(name, []).extend(pairs)
        sampled_visits += [visits_by[i][view_of(i)] for i in range(k)]
        left -= k
        blk += 1
    ms_per_step = 1e3 * wall / args.steps
    steps_per_s = args.steps / wall
    raster = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in raster_ev.items()}
    launches = {k: len(v) for k, v in raster_ev.items()}

    # the full per-stage breakdown from a block with every stage bracketed
    log("[bench] stage breakdown block")
    _, _, all_stages = run_block(step, init, RESTORE_EVERY, timed_stages=set())
    stage_t = {k: [a.elapsed_time(b) for a, b in v] for k, v in all_stages.items()}
    stages = {k: float(np.mean(v)) for k, v in stage_t.items()}
    # view 0's projection runs inside the previous step's Adam pass (its
    # preprocess stage only lists the visible rows); views 1.. are projected
    # in one pass over the parameters (stage preprocess_views): the
    # parameters read once, each view's records, flags and list written
    pv_t = stage_t.get("preprocess_views", [])
    pv_bytes = 236.0 * N + (nv - 1) * 80.0 * N

    # roofline of the dominant raster kernel (one launch per view): the
    # back-propagated (pixel, entry) pairs the counting block measured,
    # times the canonical rule's operations per pair, over the launch time
    raster.setdefault("render_fwd", stages["render_fwd"])    # (from the breakdown block)
    launches.setdefault("render_fwd", len(stage_t["render_fwd"]))
    dom = max(("render_fwd", "render_bwd"), key=lambda k: raster.get(k, 0.0))
    kname = "k_render_bwd" if dom == "render_bwd" else "k_render_fwd"
    # the sampled backward launches' own pairs (the forward: the average)
    vpl = float(np.mean(sampled_visits)) if dom == "render_bwd" else visits_per_launch
    ops = vpl * OPS_PER_VISIT[dom]
    achieved = ops / (raster[dom] * 1e-3)
    wl = {2: "mid_1080p"}.get(args.config)
    valu = recorded_valu_issue(kname, wl) if wl else None
    roofline = {"kernel": kname, "bound": "alu", "achieved": achieved / 1e12, "peak": VALU_PEAK / 1e12,
                "unit": "Tops/s (32-bit VALU)", "frac": achieved / VALU_PEAK,
                "traffic": recorded_traffic(kname, wl) if wl else None,
                "avg_launch_ms": raster[dom], "launches": launches[dom], "ops_per_launch": ops,
                "visits_per_launch": vpl, "ops_per_visit": OPS_PER_VISIT[dom],
                "valu_issue_frac": (valu / (CUS * CLOCK * raster[dom] * 1e-3)) if valu else None}

    def hbm_frac(b, ms):
        return b / (ms * 1e-3) / HBM_PEAK

    def alu_frac(o, ms):
        return o / (ms * 1e-3) / VALU_PEAK

    per_view = {k: v / nv for k, v in B_stage.items()}
    fused_bytes = float(np.mean([1416 * U + 96 * sum(v["V"] for v in vs) + 64 * U for vs, U in sizes]))
    stage_bound = {
        "preprocess": {"bound": "hbm", "frac": hbm_frac(pv_bytes, float(np.mean(pv_t))) if pv_t else None,
                       "note": "views 1.. in one pass over the parameters (236 B in, 80 B out per Gaussian and "
                               "view; view 0 is projected in the Adam pass)"},
        "bin_sort": {"bound": "hbm", "frac": hbm_frac(per_view["bin_sort"], stages["bin_sort"])},
        "render_fwd": {"bound": "alu", "frac": alu_frac(visits_per_launch * OPS_PER_VISIT["render_fwd"],
                                                        stages["render_fwd"]),
                       "hbm_frac": hbm_frac(per_view["render_fwd"], stages["render_fwd"])},
        "loss": {"bound": "hbm", "frac": hbm_frac(per_view["loss"], stages["loss"])},
        "render_bwd": {"bound": "alu", "frac": alu_frac(visits_per_launch * OPS_PER_VISIT["render_bwd"],
                                                        stages["render_bwd"]),
                       "hbm_frac": hbm_frac(per_view["render_bwd"], stages["render_bwd"])},
        "sparse_adam": {"bound": "hbm", "frac": hbm_frac(fused_bytes, stages["sparse_adam"]),
                        "alg_bytes": fused_bytes,
                        "note": "every view's projection backward and the next step's first projection fused "
                                "into the Adam pass: 1416 B per union row (parameters and moments in and out) "
                                "+ 96 B per (view, visible row) (screen gradients read and re-zeroed) + 64 B "
                                "per row (the next record)"},
    }

    last_views, U = sizes[-1]
    out = {
        "metric": METRIC,
        "value": steps_per_s,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{work.name}: {N:,} Gaussians, {nv} views of "
                               f"{work.cameras[0].width}x{work.cameras[0].height}, sparse Adam",
                   "n": N, "views": nv, "width": work.cameras[0].width, "height": work.cameras[0].height},
        "images_per_s": steps_per_s * nv,
        "median_ms_per_step": float(np.median(step_ms)),
        "protocol": f"state restored from a device copy before every block of {RESTORE_EVERY} steps (outside "
                    "the timed region); value = steps / summed block wall time",
        "hbm": {"alg_bytes_per_step": B, "alg_GBps": B / (ms_per_step * 1e-3) / 1e9,
                "frac_of_peak": B / (ms_per_step * 1e-3) / HBM_PEAK,
                "measured_bytes_per_step": recorded_step_traffic(wl) if wl else None},
        "raster_ms_per_launch": raster,
        "stages_ms_per_launch": stages,
        "stage_bound_frac": stage_bound,
        "sizes": {"V": [v["V"] for v in last_views], "M": [v["M"] for v in last_views],
                  "M_proc": [v["M_proc"] for v in last_views], "U": U,
                  "visits_per_view": visits_per_launch},
        "roofline": roofline,
    }
    if not args.quick:
        log("[bench] step without the next preprocess in the Adam pass")
        step.fuse_next_preprocess = False
        w, ms, _ = run_block(step, init, RESTORE_EVERY)
        step.fuse_next_preprocess = True
        out["ms_per_step_next_preprocess_unfused"] = 1e3 * w / RESTORE_EVERY
        out["hbm"]["device_copy_GBps"] = device_copy_GBps()
    if not (args.no_cpu_baseline or args.quick):
        log("[bench] oracle cpu baseline")
        out["cpu_baseline"] = cpu_baseline(work)
    if not args.quick:
        out["shard"] = shard_bench(step, work)
        out["densify"] = densify_bench(step)
    if not (args.no_coupling or args.quick):
        del step
        torch.cuda.empty_cache()
        out["view_coupling"] = view_coupling_bench()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
