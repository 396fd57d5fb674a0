"""Benchmark: train steps/s of one 3D Gaussian Splatting training step on one
MI355X (forward + backward + sparse Adam), on the mid workload: 1,000,000
seeded synthetic Gaussians, four 1920x1080 ring views per step.

    python bench.py [--steps K] [--warmup W] [--config 2] [--no-cpu-baseline]

Prints ONE JSON line.  `value` = steps/s with every input resident in HBM
when the timed region starts.  Inside the timed region HIP events on the
stream the library launches on bracket the two raster entry points
(render_bwd: the k_render_bwd launch; render_fwd: a counter fill and the
k_render_fwd launch); the dominant one's roofline uses them.  The other
stages' times come from a shorter pass after it with every stage bracketed.
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
FP32_VECTOR_PEAK = 157.3e12    # flop/s, MI355X fp32 vector (packed)
TILE = 16

# Algorithmic flops of one pixel examining one list entry, counted from the
# canonical rule (mul/add/sub/div = 1, fma = 2; rint, ldexp, compares free):
#   forward : dx, dy 2 + power 7 + exp 19 + alpha 1 + 1 - alpha, T(1 - alpha) 2
#             + weight 1 + 3 colour fma 6                                  = 38
#   backward: the forward's alpha 29 + T_i 2 + weight 1 + dL/dc 3
#             + dL/dalpha 9 + suffix colour 10 + opacity/power 2
#             + conic 9 + mean 8 + conic recovery 3                        = 76
FLOPS_PER_EVAL = {"render_fwd": 38, "render_bwd": 76}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic_bytes(N, views, U):
    """Compulsory HBM bytes of one step: each stage's inputs read once and
    outputs written once; sort at its floor of one read + one write of each
    pair; rasterisers count only the processed prefix M_proc.  Per view with
    V visible, M pairs, P pixels, T tiles."""
    total = 0
    for v in views:
        V, M, Mp, P, T = v["V"], v["M"], v["M_proc"], v["P"], v["T"]
        total += (288 * N                 # preprocess: 236 B params in, 52 B projected out
                  + 16 * N                # visibility scan + visible list
                  + 16 * V + 12 * M       # key duplication
                  + 24 * M                # sort floor
                  + 4 * M + 8 * T         # tile ranges
                  + 40 * Mp + 20 * P      # raster forward
                  + 36 * P                # loss
                  + 40 * Mp + 20 * P + 48 * V   # raster backward (screen-space gradients out)
                  + 96 * V)               # projection backward: screen-space gradients in, re-zeroed
    # projection backward of every view fused with sparse Adam: per updated
    # row 236 B parameters and 472 B moments in, 708 B parameters and moments out
    return total + 1416 * U


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
    step of the same workload at its initial parameters: per view
    preprocess, binning, render, loss and backward (gradients summed over
    views), then Adam over the union of the visible sets.  Views are taken
    in order until the step is complete or `budget_s` has passed; the view
    part is then scaled by (views in the step) / (views run)."""
    import numpy as np

    import oracle
    t = time.perf_counter
    nv = len(work.cameras)
    grads = None
    seen = np.zeros(work.n, bool)
    t0 = t()
    done = 0
    for cam, tgt in zip(work.cameras, work.targets):
        pre = oracle.preprocess(work.params, cam)
        oracle.bin_sort(work.params, cam)
        img, _, _, _ = oracle.render(work.params, cam)
        _, dL, _, _ = oracle.loss(img, tgt, work.w_l1, work.w_ssim)
        _, _, g, _ = oracle.backward(work.params, cam, dL)
        grads = g if grads is None else grads + g
        seen |= pre["visible"]
        done += 1
        if t() - t0 > budget_s:
            break
    t_views = (t() - t0) * nv / done
    rows = np.flatnonzero(seen).astype(np.int32)
    zeros = np.zeros_like(grads)
    t1 = t()
    oracle.adam(work.params, grads, zeros, zeros, rows, work.lr, work.beta1, work.beta2, work.eps)
    t_adam = t() - t1
    t_step = t_views + t_adam
    return {"value": 1.0 / t_step, "unit": "steps/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"one step at the initial parameters: {done} of {nv} views (full size) in "
                      f"{t_views * done / nv:.1f} s" + (f", scaled x{nv / done:.2f}" if done < nv else "") +
                      f", Adam over {rows.shape[0]:,} rows in {t_adam:.1f} s"}


VALU_INT_PEAK = 256 * 64 * 2.4e9   # 32-bit VALU ops/s: 256 CUs x 64 lanes/clock x 2.4 GHz


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
                     "peak": VALU_INT_PEAK / 1e12, "unit": "Tops/s (32-bit VALU)",
                     "frac": ops / (ms * 1e-3) / VALU_INT_PEAK, "traffic": None,
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-coupling", action="store_true", help="skip the view-coupling measurement")
    ap.add_argument("--coupling-only", action="store_true",
                    help="print only the view-coupling measurement (for profiling it alone)")
    ap.add_argument("--shard-only", action="store_true",
                    help="one step, then print only the tile-block / all-to-all measurement")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported by this build "
              "(the multi-GPU sharding is a design in DESIGN.md, not code)", file=sys.stderr)
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
    step = gs.from_workload(work, device="cuda:0", record_tiles=True)
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

    # The objects alive after set-up (torch's, numpy's, the workload's) are
    # moved out of the garbage collector's generations: a full collection
    # over them takes tens of milliseconds on this interpreter and, landing
    # inside the timed loop, stalls the host between two kernel launches
    # while the GPU drains its queue.  Host-side only; every GPU stage runs.
    gc.collect()
    gc.freeze()
    log(f"[bench] timing {args.steps} steps")
    # HIP events around the two raster kernels only: an event pair between
    # two launches leaves the stream idle for several microseconds, and
    # around every stage (six per view) they cost about 3 % of the step
    step.timer = {}
    step.timer_stages = {"render_fwd", "render_bwd"}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step.step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timer = step.timer
    ms_per_step = 1e3 * wall / args.steps
    steps_per_s = args.steps / wall
    # the full per-stage breakdown from a shorter pass with every stage timed
    step.timer, step.timer_stages = {}, None
    for _ in range(min(args.steps, 10)):
        step.step()
    torch.cuda.synchronize()
    all_stages, step.timer = step.timer, None
    stages = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in all_stages.items()}
    raster = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in timer.items()}
    launches = {k: len(v) for k, v in timer.items()}

    # sizes of the last step (scene drifts slowly under Adam; sizes are re-read)
    views = []
    for vw, k in zip(step.views, range(len(step.views))):
        views.append(dict(V=int(step.vis_count[k].item()), M=vw.num_pairs,
                          M_proc=int(vw.tile_processed.to(torch.int64).sum().item()),
                          P=vw.W * vw.H, T=vw.T))
    U = int(step.union_count.item())
    B = algorithmic_bytes(N, views, U)

    # roofline of the dominant raster kernel (one launch per view)
    dom = max(("render_fwd", "render_bwd"), key=lambda k: raster.get(k, 0.0))
    evals = float(np.mean([TILE * TILE * v["M_proc"] for v in views]))
    flops = evals * FLOPS_PER_EVAL[dom]
    achieved = flops / (raster[dom] * 1e-3)
    kname = "k_render_bwd" if dom == "render_bwd" else "k_render_fwd"
    wl = {2: "mid_1080p"}.get(args.config)
    roofline = {"kernel": kname, "bound": "alu",
                "achieved": achieved / 1e12, "peak": FP32_VECTOR_PEAK / 1e12, "unit": "TFLOP/s",
                "frac": achieved / FP32_VECTOR_PEAK,
                "traffic": recorded_traffic(kname, wl) if wl else None,
                "avg_launch_ms": raster[dom], "launches": launches[dom], "flops_per_launch": flops,
                "evals_per_launch": evals, "flops_per_eval": FLOPS_PER_EVAL[dom]}

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
        "config": {"workload": f"{work.name}: {N:,} Gaussians, {len(work.cameras)} views of "
                               f"{work.cameras[0].width}x{work.cameras[0].height}, sparse Adam",
                   "n": N, "views": len(work.cameras), "width": work.cameras[0].width,
                   "height": work.cameras[0].height},
        "images_per_s": steps_per_s * len(work.cameras),
        "hbm": {"alg_bytes_per_step": B, "alg_GBps": B / (ms_per_step * 1e-3) / 1e9,
                "frac_of_peak": B / (ms_per_step * 1e-3) / HBM_PEAK},
        "raster_ms_per_launch": raster,
        "stages_ms_per_launch": stages,
        "sizes": {"V": [v["V"] for v in views], "M": [v["M"] for v in views],
                  "M_proc": [v["M_proc"] for v in views], "U": U},
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        log("[bench] oracle cpu baseline")
        out["cpu_baseline"] = cpu_baseline(work)
    out["shard"] = shard_bench(step, work)
    out["densify"] = densify_bench(step)
    if not args.no_coupling:
        del step
        torch.cuda.empty_cache()
        out["view_coupling"] = view_coupling_bench()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
