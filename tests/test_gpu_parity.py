"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Integers (visible lists, rectangles, radii, tile counts, sort keys, values,
tile ranges, pair counts, per-pixel `last`, per-tile processed counts) must
be bit-identical.  Floating point: projection <= 1e-6 relative (expected
bit-identical), image <= 1e-4 absolute (expected bit-identical), final
transmittance <= 1e-6, loss <= 1e-5 relative, gradients elementwise within
1e-3 relative + 1e-4 of the oracle's magnitude bound (the sum of |terms|,
which fp32 summation order can move by a few ulps), Adam as derived in
check_adam.  Inputs are the seeded synthetic workloads, cut down so the
oracle finishes in seconds while spanning many tiles and ragged edges.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import check_forward, check_grad, proj_fields, run_gpu_step, say, step_keys

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def workload_case(name):
    if name == "tiny":
        return synth.workload(0)
    if name == "small_cut":      # ragged 300x200 (18.75 x 12.5 tiles), SSIM loss
        return synth.cut_down(synth.workload(1), 300, 200, n=20000)
    if name == "mid_cut":        # batch of 4 ring views, union + accumulation
        return synth.cut_down(synth.workload(2), 320, 180, n=30000)
    if name == "aerial_cut":     # empty sky rows, heavy-tailed scales
        return synth.cut_down(synth.aerial(n=200_000), 480, 272, n=40000)
    if name == "small_full":     # the whole small workload, 1297x840
        return synth.workload(1)
    if name == "capacity_cut":   # 10 of the capacity batch's ring views: more than the step fuses
        return synth.capacity(n=20000, width=200, height=120, views=10)
    raise KeyError(name)


def check_adam(res, ref, work, p0, tol_g):
    """First step (t = 1): p' = p - lr g / (|g| + eps), m' = (1 - b1) g,
    v' = (1 - b2) g^2 (bias-corrected, m = v = 0 before).  Each is monotone
    in g (v in |g|), so the GPU's value must lie in the image of
    [g - tol_g, g + tol_g] under the same map, widened by the fp32 rounding
    of the update (2 ulp of p; the bias-correction scalars rounded to fp32
    move the ratio by < 2e-5 of lr)."""
    U = ref["union"]
    assert np.array_equal(res["union"], U), "union list"
    assert not res["union_flags"].any(), "union flags not cleared"
    assert not res["grads_after"].any(), "consumed gradients not zeroed"
    rows = np.zeros(work.n, bool)
    rows[U] = True
    # untouched rows keep p, m, v
    assert np.array_equal(res["params"][:, ~rows], p0[:, ~rows])
    assert not res["m"][:, ~rows].any() and not res["v"][:, ~rows].any()
    g = ref["grads"][:, rows]
    tg = tol_g[:, rows]
    lr, b1, b2, eps = work.lr, work.beta1, work.beta2, work.eps
    p = p0[:, rows].astype(np.float64)
    f = lambda x: x / (np.abs(x) + eps)
    lo = p - lr * f(g + tg)
    hi = p - lr * f(g - tg)
    slack = 2 * np.spacing(np.abs(p).astype(np.float32)).astype(np.float64) + 2e-5 * lr
    pg = res["params"][:, rows].astype(np.float64)
    bad = (pg < lo - slack) | (pg > hi + slack)
    amb = int((np.abs(g) <= tg).sum())
    say(f"  adam: rows={rows.sum()} sign-ambiguous={amb} bad={int(bad.sum())}")
    assert not bad.any(), f"adam params: {int(bad.sum())} outside the interval"
    mg = res["m"][:, rows].astype(np.float64)
    assert np.all(np.abs(mg - (1 - b1) * g) <= (1 - b1) * tg + 1e-6 * np.abs(mg) + 1e-38), "adam m"
    vg = res["v"][:, rows].astype(np.float64)
    gl = np.maximum(np.abs(g) - tg, 0.0)
    gh = np.abs(g) + tg
    assert np.all((vg >= (1 - b2) * gl * gl * (1 - 2e-5) - 1e-38) & (vg <= (1 - b2) * gh * gh * (1 + 2e-5) + 1e-38)), "adam v"


def check_loss_grad(gv, ov, w_ssim):
    dL, odL = gv["dL"], ov["dL_dimage"]
    err = np.abs(dL - odL)
    scale = np.max(np.abs(odL))
    say(f"  loss {gv['loss']:.8f} vs {ov['loss']:.8f}; dL/dI max|err|={err.max():.3g} (max|dL|={scale:.3g})")
    assert abs(gv["loss"] - ov["loss"]) <= 1e-5 * abs(ov["loss"]) + 1e-7
    if w_ssim == 0.0:
        assert np.all(err <= 1e-6 * np.abs(odL) + 1e-30)
    else:
        assert np.all(err <= 1e-4 * scale + 1e-4 * np.abs(odL))


# image-gradient tolerance: 1e-4 of max|dL/dI| + 1e-4 relative (fp32 separable
# window against the fp64 direct one); propagated into the gradient bounds
DL_TOL = (1e-4, 1e-4)


@pytest.mark.parametrize("case", ["tiny", "small_cut", "mid_cut", "aerial_cut", "small_full"])
def test_training_step_parity(case):
    """The whole step on the GPU's own intermediate results."""
    work = workload_case(case)
    say(f"[{case}] n={work.n} views={len(work.cameras)} {work.cameras[0].width}x{work.cameras[0].height}")
    p0 = work.params.copy()
    res, _ = run_gpu_step(work)
    ref = oracle.step(work, dl_tol=DL_TOL)
    for k, (cam, gv, ov) in enumerate(zip(work.cameras, res["views"], ref["views"])):
        pre = oracle.preprocess(work.params, cam)
        okeys, ovals, oranges = oracle.bin_sort(work.params, cam)
        check_forward(gv, pre, okeys, ovals, oranges, ov["image"], ov["T_final"], ov["last"],
                      ov["tile_processed"], tag=f"{case}/v{k}")
        check_loss_grad(gv, ov, work.w_ssim)
        vis = pre["visible"]
        check_grad(f"{case}/v{k} grad2d", gv["grad2d"][vis], ov["g2d"][vis], ov["m2d"][vis], ov["m2d_dl"][vis])
        assert not gv["grad2d_after"].any(), "screen-space gradients not re-zeroed"
    check_grad(f"{case} grads", res["grads"], ref["grads"], ref["mags"], ref["mags_dl"])
    tol_g = 1e-3 * np.abs(ref["grads"]) + 1e-4 * ref["mags"] + ref["mags_dl"]
    check_adam(res, ref, work, p0, tol_g)


@pytest.mark.parametrize("case", ["mid_cut", "small_cut"])
def test_pipelined_step_matches_oracle(case):
    """The step as bench.py runs it: view k + 1 prepared on a second stream
    while view k renders and back-propagates.  Images, losses, accumulated
    gradients and the Adam update against the oracle; then a second step
    (buffer sets reused across steps) against the first one's images."""
    import differentiable_gaussian_splatting_dgs_amd as gs
    work = workload_case(case)
    p0 = work.params.copy()
    ref = oracle.step(work, dl_tol=DL_TOL)
    step = gs.from_workload(work, record_tiles=True)
    step.run_views()
    torch.cuda.synchronize()
    for k, (vw, ov) in enumerate(zip(step.views, ref["views"])):
        img = vw.image.cpu().numpy()
        assert float(np.max(np.abs(img - ov["image"]))) <= 1e-4, f"{case}/v{k} image"
        assert np.array_equal(vw.last.cpu().numpy().view(np.uint32), ov["last"]), f"{case}/v{k} last"
        assert abs(float(vw.loss.item()) - ov["loss"]) <= 1e-5 * abs(ov["loss"]) + 1e-7, f"{case}/v{k} loss"
    grads = step.grads.cpu().numpy().copy()
    check_grad(f"{case} grads (pipelined)", grads, ref["grads"], ref["mags"], ref["mags_dl"])
    step.adam()
    torch.cuda.synchronize()
    U = int(step.union_count.item())
    res = dict(grads=grads, params=step.params.cpu().numpy(), m=step.m.cpu().numpy(), v=step.v.cpu().numpy(),
               union=step.union_idx[:U].cpu().numpy().copy(), grads_after=step.grads.cpu().numpy(),
               union_flags=step.union_flags[: step.n].cpu().numpy().copy())
    tol_g = 1e-3 * np.abs(ref["grads"]) + 1e-4 * ref["mags"] + ref["mags_dl"]
    check_adam(res, ref, work, p0, tol_g)
    # second step on the updated parameters, sequential vs pipelined
    seq = gs.from_workload(work, record_tiles=True)
    seq.params.copy_(step.params)
    for k in range(len(seq.views)):
        seq.forward_view(k)
        seq.backward_view(k)
    step.run_views()
    torch.cuda.synchronize()
    for k, (a, b) in enumerate(zip(step.views, seq.views)):
        assert torch.equal(a.image, b.image), f"{case}/v{k} second-step image"
        assert torch.equal(a.last, b.last), f"{case}/v{k} second-step last"
        assert torch.equal(a.ranges, b.ranges), f"{case}/v{k} second-step ranges"


@pytest.mark.parametrize("case,max_fused", [("mid_cut", None), ("small_cut", None), ("capacity_cut", None),
                                            ("capacity_cut", 8)])
def test_fused_step_matches_oracle(case, max_fused):
    """TrainStep.step() as bench.py runs it: the projection backward of the
    last views (all of them, up to GS_MAX_FUSED_VIEWS; 8 in the last case)
    fused into the Adam pass, that of any earlier view (capacity_cut with 8
    fused: two of ten) accumulated into the gradient planes first.  The update against the oracle's gradients (as check_adam),
    screen-space buffers left zero; the union flags the pass leaves are the
    next step's first view's visibility (its preprocess of the updated
    rows)."""
    import differentiable_gaussian_splatting_dgs_amd as gs
    work = workload_case(case)
    p0 = work.params.copy()
    ref = oracle.step(work, dl_tol=DL_TOL)
    kw = {} if max_fused is None else dict(max_fused_views=max_fused)
    step = gs.from_workload(work, record_tiles=True, **kw)
    assert step.nfirst == max(0, len(work.cameras) - (max_fused or gs.GS_MAX_FUSED_VIEWS))
    step.step()
    torch.cuda.synchronize()
    U = int(step.union_count.item())
    res = dict(params=step.params.cpu().numpy(), m=step.m.cpu().numpy(), v=step.v.cpu().numpy(),
               union=step.union_idx[:U].cpu().numpy().copy(), grads_after=step.grads.cpu().numpy(),
               union_flags=step.union_flags[: step.n].cpu().numpy().copy())
    nxt = oracle.preprocess(res["params"], work.cameras[0])["visible"]
    assert np.array_equal(res["union_flags"], nxt.astype(np.uint8)), "union flags of the next step's view 0"
    res["union_flags"] = np.zeros_like(res["union_flags"])
    tol_g = 1e-3 * np.abs(ref["grads"]) + 1e-4 * ref["mags"] + ref["mags_dl"]
    check_adam(res, ref, work, p0, tol_g)
    for g2 in step.g2d:
        assert not g2.any().item(), "screen-space gradients not re-zeroed"


def test_pipelined_step_grows_an_overflowing_pair_buffer():
    """A pair capacity far below M: the non-blocking binning leaves empty
    ranges, the step sees the counts before Adam, grows the buffers and runs
    the batch again; gradients then match the oracle."""
    import differentiable_gaussian_splatting_dgs_amd as gs
    work = workload_case("mid_cut")
    ref = oracle.step(work, dl_tol=DL_TOL)
    step = gs.from_workload(work, record_tiles=True, pair_capacity=1000)
    step.run_views()
    torch.cuda.synchronize()
    assert all(ps.capacity >= vw.num_pairs for vw, ps in
               zip(step.views, [step.sets[k % step.nsets] for k in range(len(step.views))]))
    for k, (vw, ov) in enumerate(zip(step.views, ref["views"])):
        assert float(np.max(np.abs(vw.image.cpu().numpy() - ov["image"]))) <= 1e-4, f"v{k} image"
    check_grad("grown grads", step.grads.cpu().numpy(), ref["grads"], ref["mags"], ref["mags_dl"])


def test_async_bin_sort_overflow_leaves_empty_ranges():
    import differentiable_gaussian_splatting_dgs_amd as gs
    work = workload_case("small_cut")
    step = gs.from_workload(work)
    step.forward_view(0)
    torch.cuda.synchronize()
    vw = step.views[0]
    M = vw.num_pairs
    keys = torch.full((M,), -1, dtype=torch.int64, device="cuda")
    vals = torch.full((M,), -1, dtype=torch.int32, device="cuda")
    ranges = torch.full((vw.T, 2), 7, dtype=torch.int32, device="cuda")
    m_dev = torch.zeros(1, dtype=torch.int64, device="cuda")
    ws = torch.empty(gs.gs_workspace_size(gs.GS_OP_BIN_SORT, step.n, 0, 0, M - 1), dtype=torch.uint8, device="cuda")
    gs.gs_bin_sort_async(step.proj, step.n, step.vis_idx[0], step.vis_count[0:1], vw.W, vw.H, keys, vals, M - 1,
                         m_dev, ranges, ws)
    torch.cuda.synchronize()
    assert int(m_dev.item()) == M
    assert not ranges.any().item(), "ranges not empty after an overflow"
    assert bool((keys == -1).all().item()) and bool((vals == -1).all().item()), "pairs written after an overflow"
    # with room: the same outputs as the blocking call
    ws = torch.empty(gs.gs_workspace_size(gs.GS_OP_BIN_SORT, step.n, 0, 0, M), dtype=torch.uint8, device="cuda")
    gs.gs_bin_sort_async(step.proj, step.n, step.vis_idx[0], step.vis_count[0:1], vw.W, vw.H, keys, vals, M,
                         m_dev, ranges, ws)
    torch.cuda.synchronize()
    assert int(m_dev.item()) == M
    assert np.array_equal(keys.cpu().numpy().view(np.uint64), step_keys(step, vw, M))
    assert torch.equal(vals, step.vals[:M]) and torch.equal(ranges, vw.ranges)
    # without keys (what the training step passes): the same values and ranges
    vals2 = torch.full((M,), -1, dtype=torch.int32, device="cuda")
    ranges2 = torch.full((vw.T, 2), 7, dtype=torch.int32, device="cuda")
    gs.gs_bin_sort_async(step.proj, step.n, step.vis_idx[0], step.vis_count[0:1], vw.W, vw.H, None, vals2, M,
                         m_dev, ranges2, ws)
    torch.cuda.synchronize()
    assert torch.equal(vals2, vals) and torch.equal(ranges2, ranges)
    # from the dense copy of the records' last words: the same again; an
    # overflow again leaves the ranges empty
    assert step.vbin[0] is not None
    keys3 = torch.full((M,), -1, dtype=torch.int64, device="cuda")
    vals3 = torch.full((M,), -1, dtype=torch.int32, device="cuda")
    ranges3 = torch.full((vw.T, 2), 7, dtype=torch.int32, device="cuda")
    gs.gs_bin_sort_async(step.proj, step.n, step.vis_idx[0], step.vis_count[0:1], vw.W, vw.H, keys3, vals3, M - 1,
                         m_dev, ranges3, ws, proj_bin=step.vbin[0])
    torch.cuda.synchronize()
    assert int(m_dev.item()) == M and not ranges3.any().item()
    gs.gs_bin_sort_async(step.proj, step.n, step.vis_idx[0], step.vis_count[0:1], vw.W, vw.H, keys3, vals3, M,
                         m_dev, ranges3, ws, proj_bin=step.vbin[0])
    torch.cuda.synchronize()
    assert int(m_dev.item()) == M
    assert torch.equal(keys3, keys) and torch.equal(vals3, vals) and torch.equal(ranges3, ranges)
    # in two calls (depth sort, then pairs), other work between them: the same
    keys4 = torch.full((M,), -1, dtype=torch.int64, device="cuda")
    vals4 = torch.full((M,), -1, dtype=torch.int32, device="cuda")
    ranges4 = torch.full((vw.T, 2), 7, dtype=torch.int32, device="cuda")
    m_dev.zero_()
    args = (step.proj, step.n, step.vis_idx[0], step.vis_count[0:1], vw.W, vw.H, keys4, vals4, M, m_dev, ranges4, ws)
    gs.gs_bin_sort_async(*args, proj_bin=step.vbin[0], part=gs.GS_BIN_DEPTH)
    torch.cuda.synchronize()
    assert int(m_dev.item()) == M, "the depth part writes the pair count"
    scratch = torch.ones(1 << 20, device="cuda") * 2.0          # unrelated work in between
    gs.gs_bin_sort_async(*args, proj_bin=step.vbin[0], part=gs.GS_BIN_PAIRS)
    torch.cuda.synchronize()
    assert float(scratch.sum().item()) == 2.0 * (1 << 20)
    assert torch.equal(keys4, keys) and torch.equal(vals4, vals) and torch.equal(ranges4, ranges)


@pytest.mark.parametrize("case", ["small_cut", "mid_cut"])
def test_backward_stages_in_isolation(case):
    """Raster and projection backward fed the oracle's image gradient: only
    the backward's own fp32 rounding separates the results."""
    work = workload_case(case)
    ref = oracle.step(work)
    res, _ = run_gpu_step(work, dL_override=[vw["dL_dimage"] for vw in ref["views"]])
    for k, (cam, gv, ov) in enumerate(zip(work.cameras, res["views"], ref["views"])):
        vis = oracle.preprocess(work.params, cam)["visible"]
        check_grad(f"{case}/v{k} grad2d (isolated)", gv["grad2d"][vis], ov["g2d"][vis], ov["m2d"][vis])
    check_grad(f"{case} grads (isolated)", res["grads"], ref["grads"], ref["mags"])


@pytest.mark.parametrize("case", ["small_cut", "mid_cut"])
def test_render_bwd_parameter_mode_and_visit_count(case):
    """gs_render_bwd with the view's projection backward chained on in the
    same call (parameters, camera and visible list given, dL/dparams added
    to the [59][n] planes): the batch's accumulated gradients against the
    oracle on the oracle's image gradient, the screen-space buffers left
    zero; and the backward's count of back-propagated (pixel, entry) pairs
    equal to the oracle's count of composited ones, exactly."""
    import differentiable_gaussian_splatting_dgs_amd as gs
    work = workload_case(case)
    ref = oracle.step(work)
    step = gs.from_workload(work, record_tiles=True)
    step.visits = torch.zeros(len(work.cameras), dtype=torch.int64, device="cuda")
    total = 0
    for k, cam in enumerate(work.cameras):
        step.forward_view(k)
        step.views[k].dL.copy_(torch.as_tensor(np.asarray(ref["views"][k]["dL_dimage"], np.float32)))
        step.backward_view(k)
        torch.cuda.synchronize()
        cnt = oracle.composited_counts(work.params, cam).astype(np.int64)
        total += int(cnt.sum())
        say(f"  {case}/v{k}: composited (pixel, entry) pairs {int(cnt.sum())}, GPU {int(step.visits[k].item())}")
        assert int(step.visits[k].item()) == int(cnt.sum()), f"{case}/v{k} visits"
        assert int(step.visits.sum().item()) == total
    check_grad(f"{case} grads (render_bwd parameter mode)", step.grads.cpu().numpy(), ref["grads"], ref["mags"])
    for g2 in step.g2d:
        assert not g2.any().item(), "screen-space gradients not re-zeroed"


def split_pool_counts(step, vw):
    """Per pool of the split workspace: states requested by the last view's
    forward (the counter runs on past the pool size) and the pool size.
    The layout: states [slots][64] float4, owners and items [slots] u32,
    segment counts [quarters] u32, then 64 pools x 32 counter words."""
    import torch

    quarters = ((vw.W + 15) // 16) * ((vw.H + 15) // 16) * 4
    pool_slots = max(64, (quarters + 63) // 64)
    slots = 64 * pool_slots
    off = slots * 64 * 16 + 8 * slots + 4 * quarters
    c = step.split_ws[off:off + 64 * 32 * 4].view(torch.int32).view(64, 32).cpu().numpy()
    return c[:, 0].astype(np.int64), pool_slots


@pytest.mark.parametrize("case,seg", [("small_cut", 64), ("mid_cut", 64), ("mid_cut", 256), ("small_full", 64),
                                      ("small_full", 512)])
def test_split_backward_matches_whole_list_backward(case, seg):
    """The raster backward with long lists walked in segments (helper waves
    starting from the forward's recorded states) against the oracle and
    against the one-wave-per-quarter backward, on the oracle's image
    gradient; short segments so that many quarters of these workloads are
    split several times, and on the whole small workload so many that some
    pools run out of states (those quarters keep the rest of their list
    whole); and the whole small workload at the 512-entry segments the
    training step uses for 1080p views (its longest lists span three)."""
    work = workload_case(case)
    ref = oracle.step(work)
    dl = [vw["dL_dimage"] for vw in ref["views"]]
    split, step = run_gpu_step(work, dL_override=dl, segment_len=seg)
    requested, pool_slots = split_pool_counts(step, step.views[-1])
    whole, _ = run_gpu_step(work, dL_override=dl, segment_len=0)
    longest = 0
    for k, (cam, gs_, gw, ov) in enumerate(zip(work.cameras, split["views"], whole["views"], ref["views"])):
        vis = oracle.preprocess(work.params, cam)["visible"]
        check_grad(f"{case}/v{k} grad2d (split {seg})", gs_["grad2d"][vis], ov["g2d"][vis], ov["m2d"][vis])
        check_grad(f"{case}/v{k} split vs whole", gs_["grad2d"][vis], gw["grad2d"][vis].astype(np.float64),
                   ov["m2d"][vis], rel=1e-4, mtol=2e-5)
        assert np.array_equal(gs_["last"], gw["last"]) and np.array_equal(gs_["image"], gw["image"])
        longest = max(longest, int(gs_["last"].max()))
    say(f"  {case}: longest composited prefix {longest} (segments of {seg}); states requested per pool "
        f"max {requested.max()} of {pool_slots}, total {requested.sum()}")
    assert longest > 3 * seg, "no quarter spans several segments"
    if case == "small_full" and seg == 64:
        assert requested.max() > pool_slots, "no pool ran out of states"


@pytest.mark.parametrize("case", ["small_cut", "mid_cut", "ring_18"])
def test_touched_map_reads_only_marked_rows(case):
    """The fused views' raster backward marks the rows it reaches in the
    touched map; the fused Adam pass with the map reads only those rows'
    screen-space gradients.  Every row with a non-zero screen-space word has
    its view's byte set; parameters, moments, the next view's records and
    flags after the pass are bit for bit those of the pass without the map;
    the map is zero afterwards.  18 ring views: 16 fused (slots 0-15), the
    first two projected separately (they mark nothing)."""
    import differentiable_gaussian_splatting_dgs_amd as gs
    if case == "ring_18":
        work = synth.plane_scene(4, 8000, 160, 96, [2 * math.pi * j / 18 for j in range(18)], 4, name="ring")
    else:
        work = workload_case(case)
    step = gs.from_workload(work)
    step.use_touched = True
    step.step()                                    # a step with the map
    step.run_views(defer_projection=True)
    torch.cuda.synchronize()
    ks = list(range(step.nfirst, len(step.views)))
    g2 = [step.g2d[step._gbuf(k)] for k in ks]
    tm = step.touched[: step.n].cpu().numpy()
    assert not tm[:, len(ks):].any(), "bytes beyond the fused views"
    marked = 0
    for w, g in enumerate(g2):
        nz = (g[: step.n] != 0).any(dim=1).cpu().numpy()
        assert np.all(tm[nz, w] != 0), f"fused view {w}: a non-zero row unmarked"
        marked += int((tm[:, w] != 0).sum())
    save = dict(params=step.params.clone(), m=step.m.clone(), v=step.v.clone(), grads=step.grads.clone(),
                uf=step.union_flags.clone(), nf=step.next_flags.clone(), tm=step.touched.clone(),
                g2=[g.clone() for g in g2])
    outs = []
    for use in (True, False):
        step.params.copy_(save["params"]); step.m.copy_(save["m"]); step.v.copy_(save["v"])
        step.grads.copy_(save["grads"]); step.union_flags.copy_(save["uf"]); step.next_flags.copy_(save["nf"])
        step.touched.copy_(save["tm"])
        for g, s0 in zip(g2, save["g2"]):
            g.copy_(s0)
        step.use_touched = use
        step.adam(fused=True)
        step.t -= 1                                # (the same bias corrections both times)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy().copy() for t in (step.params, step.m, step.v, step.vproj[0], step.vbin[0],
                                                      step.next_flags, step.union_flags)])
        if use:
            assert not step.touched.any().item(), "map not cleared"
            assert all(not g.any().item() for g in g2), "screen-space rows left"
    for name, a, b in zip(("params", "m", "v", "next records", "next dense copy", "next flags", "union flags"),
                          outs[0], outs[1]):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), name
    say(f"  {case}: {len(ks)} fused views, {marked} marked (row, view) of {step.n * len(ks)}")


@pytest.mark.parametrize("case", ["small_cut", "mid_cut"])
def test_next_step_preprocess_in_the_optimiser_pass(case):
    """step() projects the updated rows for the next step's first view inside
    the Adam pass.  After one step: view 0's records (visible rows, every
    row's tile count), its visible list and the union flags, against the
    oracle's preprocess of the parameters the step produced; then the next
    step's first binning from them against the oracle's."""
    import differentiable_gaussian_splatting_dgs_amd as gs
    work = workload_case(case)
    step = gs.from_workload(work, record_tiles=True)
    step.step()
    torch.cuda.synchronize()
    assert step._pre0
    p1 = step.params.cpu().numpy()
    cam = work.cameras[0]
    pre = oracle.preprocess(p1, cam)
    vis = pre["visible"]
    assert np.array_equal(step.union_flags[: step.n].cpu().numpy(), vis.astype(np.uint8)), "union flags"
    # the dense copy the binning reads: the records' last four words, every
    # row (updated rows from the pass, the rest from the first preprocess)
    assert np.array_equal(step.vbin[0][: step.n].cpu().numpy().view(np.uint32),
                          step.vproj[0][: step.n, 12:16].cpu().numpy().view(np.uint32)), "dense copy"
    step.prepare_view(0)                       # visible list from the pass's flags, then binning
    torch.cuda.synchronize()
    assert not step._pre0 and not step.next_flags.any().item(), "flags not consumed"
    vw = step.views[0]
    M = vw.num_pairs
    V = int(step.vis_count[0].item())
    gv = dict(proj=step.vproj[0][: step.n].cpu().numpy(), vis=step.vis_idx[0][:V].cpu().numpy(), M=M,
              keys=step_keys(step, vw, M), vals=step.vals[:M].cpu().numpy(),
              ranges=vw.ranges.cpu().numpy().view(np.uint32))
    okeys, ovals, oranges = oracle.bin_sort(p1, cam)
    check_forward(gv, pre, okeys, ovals, oranges, None, None, None, None, tag=f"{case} next v0")
    say(f"  {case}: view 0 after one step: {V} visible, {M} pairs")


def test_determinism_of_integer_outputs():
    work = workload_case("small_cut")
    a, _ = run_gpu_step(work)
    b, _ = run_gpu_step(work)
    for x, y in zip(a["views"], b["views"]):
        for key in ("vis", "keys", "vals", "ranges", "last", "tile_processed", "image", "T_final"):
            assert np.array_equal(x[key], y[key]), key


def forward_only_parity(one, tag):
    """First view of `one` through preprocess, binning and the forward:
    projection, visible list, every sort key and value, tile ranges, the
    image, and the loss."""
    import differentiable_gaussian_splatting_dgs_amd as gs
    step = gs.from_workload(one, record_tiles=True)
    step.forward_view(0)
    torch.cuda.synchronize()
    vw = step.views[0]
    M = vw.num_pairs
    gv = dict(proj=step.proj.cpu().numpy(), vis=step.vis_idx[0][: int(step.vis_count[0].item())].cpu().numpy(),
              M=M, keys=step_keys(step, vw, M), vals=step.vals[:M].cpu().numpy(),
              ranges=vw.ranges.cpu().numpy().view(np.uint32), image=vw.image.cpu().numpy(),
              T_final=vw.T_final.cpu().numpy(), last=vw.last.cpu().numpy().view(np.uint32),
              tile_processed=vw.tile_processed.cpu().numpy().view(np.uint32))
    say(f"[{tag}] M={M}")
    cam = one.cameras[0]
    pre = oracle.preprocess(one.params, cam)
    okeys, ovals, oranges = oracle.bin_sort(one.params, cam)
    img, Tf, last, proc = oracle.render(one.params, cam)
    check_forward(gv, pre, okeys, ovals, oranges, img, Tf, last, proc, tag=tag)
    L, dL, _, _ = oracle.loss(img, one.targets[0], one.w_l1, one.w_ssim)
    assert abs(float(vw.loss.item()) - L) <= 1e-5 * L


def first_view(work, name):
    return synth.Workload(work.config, name, work.params, work.cameras[:1], work.targets[:1], work.w_l1,
                          work.w_ssim, work.lr, work.beta1, work.beta2, work.eps)


def test_mid_full_view_forward():
    """The 1M-Gaussian 1080p workload at full size, first view."""
    forward_only_parity(first_view(synth.workload(2), "mid_v0"), "mid_full/v0")


@pytest.mark.parametrize("shape", [(4128, 96), (96, 4128)])
def test_more_than_256_tile_columns_or_rows(shape):
    """Images over 256 tiles wide or tall take the plain 64-bit key passes
    of the binning instead of the column/row passes; same outputs."""
    w, h = shape
    work = synth.cut_down(synth.workload(1), w, h, n=20000, views=1)
    forward_only_parity(work, f"wide_{w}x{h}")


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

def _tiny_work(params, width=64, height=48):
    cam = synth.ring_camera(width, height, 0.0)
    tgt = np.random.default_rng(9).uniform(size=(3, height, width)).astype(np.float32)
    return synth.Workload(0, "edge", params, [cam], [tgt], 0.8, 0.2, 1e-3, 0.9, 0.999, 1e-15)


def test_no_gaussians():
    work = _tiny_work(np.zeros((59, 0), np.float32))
    res, _ = run_gpu_step(work)
    v = res["views"][0]
    assert v["M"] == 0 and v["vis"].size == 0
    assert not v["image"].any() and np.all(v["T_final"] == 1.0) and not v["last"].any()
    assert res["union"].size == 0


def test_nothing_visible_leaves_state_untouched():
    p = np.zeros((59, 300), np.float32)
    p[6] = 1.0
    p[2] = -10.0                                 # all behind the camera
    work = _tiny_work(p)
    res, _ = run_gpu_step(work)
    v = res["views"][0]
    assert v["M"] == 0 and v["vis"].size == 0 and not v["image"].any()
    assert not res["grads"].any() and res["union"].size == 0
    assert np.array_equal(res["params"], p)


def test_non_finite_parameters_are_culled():
    work = synth.cut_down(synth.workload(0), 96, 80, n=1500)
    p = work.params.copy()
    p[0, 3] = np.nan
    p[4, 10] = np.inf
    p[7, 20] = np.nan
    p[30, 40] = -np.inf
    p[10, 50] = np.inf
    p[6:10, 60] = 0.0                             # zero quaternion
    work.params = p
    res, _ = run_gpu_step(work)
    cam = work.cameras[0]
    pre = oracle.preprocess(p, cam)
    assert not pre["visible"][[3, 10, 20, 40, 50, 60]].any()
    ref = oracle.step(work)
    gv, ov = res["views"][0], ref["views"][0]
    okeys, ovals, oranges = oracle.bin_sort(p, cam)
    check_forward(gv, pre, okeys, ovals, oranges, ov["image"], ov["T_final"], ov["last"], ov["tile_processed"],
                  tag="nonfinite")
    assert np.all(np.isfinite(res["grads"]))


def test_capacity_error_reports_the_pair_count():
    import differentiable_gaussian_splatting_dgs_amd as gs
    work = synth.workload(0)
    step = gs.from_workload(work)
    step.forward_view(0)
    M = step.views[0].num_pairs
    vw = step.views[0]
    keys = torch.empty(M - 1, dtype=torch.int64, device="cuda")
    vals = torch.empty(M - 1, dtype=torch.int32, device="cuda")
    ws = torch.empty(gs.gs_workspace_size(gs.GS_OP_BIN_SORT, step.n, 0, 0, M - 1), dtype=torch.uint8,
                     device="cuda")
    with pytest.raises(gs.GSError) as ei:
        gs.gs_bin_sort(step.proj, step.n, step.vis_idx[0], step.vis_count[0:1], vw.W, vw.H, keys, vals, M - 1,
                       vw.ranges, ws)
    assert ei.value.status == gs.GS_ERR_CAPACITY and ei.value.num_pairs == M


def test_single_gaussian_matches_closed_form_on_gpu():
    cam = synth.ring_camera(128, 128, 0.0)
    p = np.zeros((59, 1), np.float32)
    p[6] = 1.0
    p[2] = -1.0
    p[3:6] = math.log(0.03)
    p[10] = 0.7
    p[11:14, 0] = [0.9, -0.3, 0.2]
    work = synth.Workload(0, "one", p, [cam], [np.zeros((3, 128, 128), np.float32)], 1.0, 0.0, 1e-3, 0.9,
                          0.999, 1e-15)
    res, _ = run_gpu_step(work)
    s = math.exp(float(np.float32(math.log(0.03))))
    var = (float(np.float32(cam.fx)) * s / 3.0) ** 2 + 0.3
    o = 1 / (1 + math.exp(-float(np.float32(0.7))))
    xs = np.arange(128) + 0.5 - 64.0
    alpha = np.minimum(0.99, o * np.exp(-(xs[:, None] ** 2 + xs[None, :] ** 2) / (2 * var)))
    alpha = np.where(alpha < 1 / 255, 0.0, alpha)
    r = math.ceil(3 * math.sqrt(var))
    lo = max(0, math.floor((64 - r) / 16)) * 16
    hi = min(128, (math.floor((64 + r) / 16) + 1) * 16)
    mask = np.zeros((128, 128), bool)
    mask[lo:hi, lo:hi] = True
    rgb = np.float32([0.9, -0.3, 0.2]).astype(np.float64) * (0.5 / math.sqrt(math.pi)) + 0.5
    img = res["views"][0]["image"]
    for c in range(3):
        assert np.max(np.abs(img[c] - rgb[c] * np.where(mask, alpha, 0.0))) < 2e-6
    pf = proj_fields(res["views"][0]["proj"])
    assert pf["radius"][0] == r


@pytest.mark.parametrize("case", ["mid_cut", "capacity_cut", "ring_18"])
def test_preprocess_views_matches_per_view(case):
    """gs_preprocess_views (the training step's preprocess of a batch's
    views, one pass over the parameters per 16 views) against gs_preprocess
    of each view: records, visible lists and counts bit for bit, the same
    union flags; and each view's visible set, rectangles, tile counts and
    depths against the oracle's preprocess.  18 ring views take two calls
    (16 + 2); the 10-view case runs on a grid of 3 workgroups."""
    import differentiable_gaussian_splatting_dgs_amd as gs
    if case == "ring_18":
        work = synth.plane_scene(4, 8000, 160, 96, [2 * math.pi * j / 18 for j in range(18)], 4, name="ring")
    else:
        work = workload_case(case)
    step = gs.from_workload(work)
    n, nv = step.n, len(work.cameras)
    # (a capped grid on one case: each workgroup walks the Gaussians with a stride)
    step.preprocess_workgroups = 3 if case == "capacity_cut" else 0
    step.union_flags.zero_()
    step.preprocess_views(range(nv))
    torch.cuda.synchronize()
    multi = []
    for k in range(nv):
        V = int(step.vis_count[k].item())
        multi.append((step.vproj[k][:n].cpu().numpy().copy(), step.vis_idx[k][:V].cpu().numpy().copy()))
        assert np.array_equal(step.vbin[k][:n].cpu().numpy().view(np.uint32),
                              multi[k][0][:, 12:16].view(np.uint32)), f"v{k} dense copy"
    uf_multi = step.union_flags[:n].cpu().numpy().copy()
    step.union_flags.zero_()
    proj = torch.empty_like(step.vproj[0])
    pbin = torch.empty_like(step.vbin[0])
    vis = torch.empty_like(step.vis_idx[0])
    cnt = torch.zeros(1, dtype=torch.int64, device=proj.device)
    for k, cam in enumerate(work.cameras):
        gs.gs_preprocess(step.params, n, step.ld, step.views[k].cam, proj, vis, cnt, step.union_flags, step.ws_pre,
                         proj_bin=pbin)
        torch.cuda.synchronize()
        V = int(cnt.item())
        one = proj[:n].cpu().numpy()
        assert np.array_equal(pbin[:n].cpu().numpy().view(np.uint32), one[:, 12:16].view(np.uint32))
        assert np.array_equal(one.view(np.uint32), multi[k][0].view(np.uint32)), f"v{k} records"
        assert np.array_equal(vis[:V].cpu().numpy(), multi[k][1]), f"v{k} visible list"
        pre = oracle.preprocess(work.params, cam)
        assert np.array_equal(multi[k][1], np.flatnonzero(pre["visible"]).astype(np.int32)), f"v{k} oracle list"
        pf = proj_fields(multi[k][0])
        sel = pre["visible"]
        assert np.array_equal(pf["tiles"], pre["tiles"]), f"v{k} tiles"
        assert np.array_equal(pf["rect"][sel], pre["rect"][sel]), f"v{k} rect"
        assert np.array_equal(pf["depth"][sel].view(np.uint32), pre["depth"][sel].view(np.uint32)), f"v{k} depth"
    assert np.array_equal(step.union_flags[:n].cpu().numpy(), uf_multi), "union flags"
    say(f"  {case}: {nv} views, visible {[len(m[1]) for m in multi]}")
