"""Parity of the HIP path at the full sizes of the two largest workloads.

* aerial (3,000,000 Gaussians, one 3840x2160 view with empty sky rows):
  the whole training step against the oracle, exactly as the cut-down
  cases in test_gpu_parity (every key, value, range, pixel and gradient).
* capacity (12,000,000 Gaussians, 16 views of 1920x1080 per step), run as
  bench.py runs a step (views overlapped on three streams): for the last two
  views, which the step leaves in its last buffer sets, the projection and
  visible list against the oracle's preprocess, the sorted pair array
  checked against its definition from those projections (every visible
  Gaussian's rectangle tiles exactly once, ordered by tile, depth bits,
  index; ranges delimit the tiles), and sampled pixels (random ones plus
  every pixel of the longest tile) composited by the oracle against that
  pair array, bit for bit; then Adam on sampled rows against its closed
  form at t = 1 from the step's own gradients.
* mid (1,000,000 Gaussians, four 1920x1080 views), run exactly as bench.py
  times it (TrainStep.step(): views pipelined on three streams, the split
  raster backward at its 1080p segment length, every view's projection
  backward fused into the Adam pass together with the next step's first
  preprocess): every view's visible list, tile ranges, launch order, pair
  values, image, final transmittance, `last` and per-tile processed counts
  against the oracle, exactly; the loss and dL/dI; the Adam update and both
  moments of all 59 x 1M entries against the oracle's accumulated
  gradients; and view 0's screen-space gradients from the same kernels.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import check_grad, keys_from_pairs, proj_fields, run_gpu_step, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module")
def capacity_work():
    return synth.workload(4)


@pytest.mark.timeout(900)
def test_aerial_full_size_training_step():
    from test_gpu_parity import DL_TOL, check_adam, check_loss_grad
    from gpu_helpers import check_forward
    work = synth.workload(3)
    say(f"[aerial full] n={work.n} {work.cameras[0].width}x{work.cameras[0].height}")
    p0 = work.params.copy()
    res, _ = run_gpu_step(work, record_tiles=True)
    ref = oracle.step(work, dl_tol=DL_TOL)
    cam = work.cameras[0]
    gv, ov = res["views"][0], ref["views"][0]
    pre = oracle.preprocess(work.params, cam)
    okeys, ovals, oranges = oracle.bin_sort(work.params, cam)
    say(f"[aerial full] M={gv['M']}")
    check_forward(gv, pre, okeys, ovals, oranges, ov["image"], ov["T_final"], ov["last"], ov["tile_processed"],
                  tag="aerial_full")
    check_loss_grad(gv, ov, work.w_ssim)
    vis = pre["visible"]
    check_grad("aerial_full grad2d", gv["grad2d"][vis], ov["g2d"][vis], ov["m2d"][vis], ov["m2d_dl"][vis])
    check_grad("aerial_full grads", res["grads"], ref["grads"], ref["mags"], ref["mags_dl"])
    tol_g = 1e-3 * np.abs(ref["grads"]) + 1e-4 * ref["mags"] + ref["mags_dl"]
    check_adam(res, ref, work, p0, tol_g)


def check_pairs_against_definition(pf, vis_idx, keys, vals, ranges, TX, tag):
    """The sorted pair array from its definition, given the projections:
    each visible Gaussian's rectangle tiles exactly once; ascending
    (tile, depth bits, index); ranges delimit the tiles."""
    rect = pf["rect"]
    depth_bits = pf["depth"].view(np.uint32)
    M = keys.shape[0]
    assert M == int(pf["tiles"][vis_idx].astype(np.int64).sum()), f"{tag} M"
    tile = (keys >> np.uint64(32)).astype(np.int64)
    assert np.array_equal((keys & np.uint64(0xFFFFFFFF)).astype(np.uint32), depth_bits[vals]), f"{tag} depth bits"
    tx, ty = tile % TX, tile // TX
    r = rect[vals]
    assert np.all((tx >= r[:, 0]) & (tx < r[:, 2]) & (ty >= r[:, 1]) & (ty < r[:, 3])), f"{tag} tile outside rect"
    visible = np.zeros(rect.shape[0], bool)
    visible[vis_idx] = True
    assert visible[vals].all(), f"{tag} value not visible"
    # strictly ascending (key, value): no pair twice; with the count above,
    # every (Gaussian, tile of its rectangle) exactly once
    same = keys[1:] == keys[:-1]
    assert np.all(keys[1:] >= keys[:-1]), f"{tag} keys not sorted"
    assert np.all(vals[1:][same] > vals[:-1][same]), f"{tag} ties not in index order"
    T = ranges.shape[0]
    counts = np.bincount(tile, minlength=T)
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]])
    expect = np.stack([np.where(counts > 0, starts, 0), np.where(counts > 0, starts + counts, 0)], 1)
    assert np.array_equal(ranges.astype(np.int64), expect), f"{tag} ranges"


@pytest.mark.timeout(900)
def test_capacity_full_size_pipelined_step_sampled(capacity_work):
    import differentiable_gaussian_splatting_dgs_amd as gs
    work = capacity_work
    nv = len(work.cameras)
    say(f"[capacity full] n={work.n} views={nv}")
    step = gs.from_workload(work, record_tiles=True)
    step.run_views()
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    for k in (nv - 2, nv - 1):
        cam = work.cameras[k]
        ps, vw = step.sets[k % step.nsets], step.views[k]
        M = vw.num_pairs
        V = int(step.vis_count[k].item())
        say(f"[capacity full] view {k}: V={V} M={M}")
        pre = oracle.preprocess(work.params, cam)
        pf = proj_fields(step.vproj[k][: work.n].cpu().numpy())
        vis_idx = step.vis_idx[k][:V].cpu().numpy()
        vis = pre["visible"]
        assert np.array_equal(vis_idx, np.flatnonzero(vis).astype(np.int32)), f"v{k} visible list"
        assert np.array_equal(pf["tiles"], pre["tiles"]), f"v{k} tiles"
        assert np.array_equal(pf["rect"][vis], pre["rect"][vis]), f"v{k} rect"
        assert np.array_equal(pf["depth"][vis].view(np.uint32), pre["depth"][vis].view(np.uint32)), f"v{k} depth"
        for nm in ("mean2d", "conic", "opacity", "rgb"):
            a, b = pf[nm][vis], pre[nm][vis]
            d = np.abs(a.astype(np.float64) - b) / np.maximum(np.abs(b.astype(np.float64)), 1e-30)
            assert d.max() <= 1e-6, f"v{k} {nm}"
        vals = ps.vals[:M].cpu().numpy()
        ranges = vw.ranges.cpu().numpy().view(np.uint32)
        # the step leaves the keys unwritten: rebuilt from values, ranges and
        # records, then held to their definition
        assert ps.keys is None
        keys = keys_from_pairs(vals, ranges, step.vproj[k][: work.n].cpu().numpy())
        TX = (cam.width + 15) // 16
        check_pairs_against_definition(pf, vis_idx, keys, vals, ranges, TX, f"v{k}")
        del keys
        # sampled pixels: random ones and every pixel of the longest tile
        heavy = int(np.argmax(ranges[:, 1].astype(np.int64) - ranges[:, 0]))
        hy, hx = np.mgrid[0:16, 0:16]
        px = np.concatenate([rng.integers(0, cam.width, 4096), (heavy % TX) * 16 + hx.ravel()]).astype(np.int32)
        py = np.concatenate([rng.integers(0, cam.height, 4096), (heavy // TX) * 16 + hy.ravel()]).astype(np.int32)
        keep = (px < cam.width) & (py < cam.height)
        px, py = px[keep], py[keep]
        rgb, Tf, last = oracle.composite_pixels(work.params, cam, vals, ranges, px, py)
        img = vw.image.cpu().numpy()
        assert np.array_equal(img[:, py, px].T, rgb), f"v{k} sampled image"
        assert np.array_equal(vw.T_final.cpu().numpy()[py, px], Tf), f"v{k} sampled T_final"
        assert np.array_equal(vw.last.cpu().numpy().view(np.uint32)[py, px], last), f"v{k} sampled last"
        say(f"  v{k}: {px.size} sampled pixels bit-identical (heaviest tile {heavy}, "
            f"{int(ranges[heavy, 1] - ranges[heavy, 0])} entries)")
    # Adam at t = 1 on sampled rows, from the step's own gradients
    rows = np.sort(rng.choice(work.n, 20000, replace=False))
    rows_t = torch.as_tensor(rows, device=step.device)
    g = step.grads[:, rows_t].cpu().numpy().astype(np.float64)
    p = step.params[:, rows_t].cpu().numpy().astype(np.float64)
    assert np.isfinite(g).all()
    step.adam()
    torch.cuda.synchronize()
    U = int(step.union_count.item())
    union = np.unique(np.concatenate([step.vis_idx[k][: int(step.vis_count[k].item())].cpu().numpy()
                                      for k in range(nv)]))
    assert np.array_equal(step.union_idx[:U].cpu().numpy(), union), "union list"
    listed = np.isin(rows, union)
    b1, b2 = work.beta1, work.beta2
    m_ref = (1 - b1) * g
    v_ref = (1 - b2) * g * g
    p_ref = p - work.lr * (m_ref / (1 - b1)) / (np.sqrt(v_ref / (1 - b2)) + work.eps)
    p_ref[:, ~listed] = p[:, ~listed]
    pg = step.params[:, rows_t].cpu().numpy().astype(np.float64)
    mg = step.m[:, rows_t].cpu().numpy().astype(np.float64)
    vg = step.v[:, rows_t].cpu().numpy().astype(np.float64)
    # fp32 evaluation of the update: a few roundings of p and of lr * ratio
    tol_p = 4 * np.spacing(np.abs(p).astype(np.float32)).astype(np.float64) + 1e-5 * work.lr
    assert np.all(np.abs(pg - p_ref) <= tol_p), "adam params"
    assert np.all(np.abs(mg[:, listed] - m_ref[:, listed]) <= 1e-6 * np.abs(m_ref[:, listed]) + 1e-38), "adam m"
    assert np.all(np.abs(vg[:, listed] - v_ref[:, listed]) <= 1e-5 * v_ref[:, listed] + 1e-38), "adam v"
    assert not step.grads[:, rows_t].any().item(), "consumed gradients not zeroed"


def test_view_coupling_full_size_sampled():
    """The coupling graph of 1,024 flight views (1920x1080) over the aerial
    scene's 3,000,000 Gaussians, as bench.py times it: for 5 sampled views
    the visible lists against the oracle's, their 5 x 5 block of counts
    exactly and of weights and priorities bit for bit against the oracle
    on the oracle's lists; over the whole matrix the properties any
    intersection matrix has (symmetric, diagonal = list lengths, entries
    within [0, min of the two lengths], weights in [0, 1])."""
    import differentiable_gaussian_splatting_dgs_amd as gs
    work = synth.workload(3)
    cams = synth.flight_cameras(1920, 1080, 1024)
    say(f"[coupling full] n={work.n} views={len(cams)}")
    vc = gs.ViewCoupling(work.n, len(cams), "cuda")
    dp = torch.from_numpy(work.params).cuda()
    vc.visible_lists(dp, work.n, cams)
    inter, w = vc.overlap()
    sample = [0, 1, 417, 800, 1023]
    prev = torch.tensor(sample[:3], dtype=torch.int32, device="cuda")
    s = vc.priority(prev)
    torch.cuda.synchronize()
    inter, w, s = inter.cpu().numpy(), w.cpu().numpy(), s.cpu().numpy()
    counts = vc.counts.cpu().numpy()
    olists = []
    for v in sample:
        ol = oracle.visible_list(work.params, cams[v])
        row = vc.lists[v, :ol.size].cpu().numpy()
        assert counts[v] == ol.size and np.array_equal(row, ol), f"view {v} visible list"
        olists.append(ol)
    oi = oracle.view_overlap(olists)
    ow = oracle.view_coupling(oi)
    sub = np.ix_(sample, sample)
    assert np.array_equal(inter[sub], oi)
    assert np.array_equal(w[sub].view(np.uint64), ow.view(np.uint64))
    os_ = oracle.view_priority(ow, [0, 1, 2])
    assert np.array_equal(s[sample].view(np.uint64), os_.view(np.uint64))
    assert np.array_equal(inter, inter.T)
    assert np.array_equal(np.diag(inter), counts)
    lo = np.minimum(counts[:, None], counts[None, :])
    assert (inter >= 0).all() and (inter <= lo).all()
    assert (w >= 0).all() and (w <= 1).all()
    say(f"[coupling full] sampled block exact; mean off-diagonal weight "
        f"{(w.sum() - np.trace(w)) / (len(cams) * (len(cams) - 1)):.3f}")


@pytest.mark.timeout(900)
def test_mid_full_size_step():
    import differentiable_gaussian_splatting_dgs_amd as gs
    from gpu_helpers import check_forward
    from test_gpu_parity import DL_TOL, check_adam, check_loss_grad
    work = synth.workload(2)
    nv = len(work.cameras)
    say(f"[mid full] n={work.n} views={nv} {work.cameras[0].width}x{work.cameras[0].height}")
    p0 = work.params.copy()
    step = gs.from_workload(work, record_tiles=True)
    assert step.seg == [gs.auto_segment_len(1920, 1080)] * nv == [512] * nv
    assert step.fuse_next_preprocess and step.ndefer == nv
    # view 0's pair array as the step's first binning makes it (its buffer
    # set is reused by view 3 within the step)
    step.prepare_view(0)
    torch.cuda.synchronize()
    M0 = step.views[0].num_pairs
    v0 = dict(vals=step.sets[0].vals[:M0].cpu().numpy(), proj=step.vproj[0][: work.n].cpu().numpy())
    say("[mid full] step()")
    step.step()
    torch.cuda.synchronize()
    res = dict(params=step.params.cpu().numpy(), m=step.m.cpu().numpy(), v=step.v.cpu().numpy(),
               union=step.union_idx[: int(step.union_count.item())].cpu().numpy().copy(),
               grads_after=step.grads.cpu().numpy(), union_flags=step.union_flags[: step.n].cpu().numpy().copy())
    views = []
    for k, vw in enumerate(step.views):
        M = vw.num_pairs
        V = int(step.vis_count[k].item())
        ps = step.sets[k % step.nsets]
        gv = dict(vis=step.vis_idx[k][:V].cpu().numpy().copy(), M=M,
                  ranges=vw.ranges.cpu().numpy().view(np.uint32).copy(),
                  order=vw.order.cpu().numpy().view(np.uint32).copy(), image=vw.image.cpu().numpy(),
                  T_final=vw.T_final.cpu().numpy(), last=vw.last.cpu().numpy().view(np.uint32).copy(),
                  tile_processed=vw.tile_processed.cpu().numpy().view(np.uint32).copy(),
                  loss=float(vw.loss.item()), dL=vw.dL.cpu().numpy())
        if k == 0:
            assert M == M0
            gv["vals"], gv["proj"] = v0["vals"], v0["proj"]
        else:
            gv["vals"] = ps.vals[:M].cpu().numpy()
            # (view 0's records are now the next step's: the Adam pass wrote them)
            gv["proj"] = step.vproj[k][: work.n].cpu().numpy()
        views.append(gv)
    say("[mid full] oracle step")
    ref = oracle.step(work, dl_tol=DL_TOL)
    for k, (cam, gv, ov) in enumerate(zip(work.cameras, views, ref["views"])):
        pre = oracle.preprocess(work.params, cam)
        okeys, ovals, oranges = oracle.bin_sort(work.params, cam)
        tag = f"mid_full/v{k}"
        if gv["proj"] is not None:
            gv["keys"] = keys_from_pairs(gv["vals"], gv["ranges"], gv["proj"])
            check_forward(gv, pre, okeys, ovals, oranges, ov["image"], ov["T_final"], ov["last"],
                          ov["tile_processed"], tag=tag)
        else:
            # the records of this view's set were replaced by the next step's
            # view 0 (the projection itself is checked on views 0-2): keys
            # rebuilt with the oracle's depth bits, everything else as
            # check_forward
            rec = np.zeros((work.n, 16), np.float32)
            rec[:, 12] = pre["depth"]
            gv["keys"] = keys_from_pairs(gv["vals"], gv["ranges"], rec)
            assert np.array_equal(gv["vis"], np.flatnonzero(pre["visible"]).astype(np.int32)), f"{tag} visible"
            assert gv["M"] == len(okeys) and np.array_equal(gv["vals"], ovals), f"{tag} values"
            assert np.array_equal(gv["keys"], okeys), f"{tag} keys"
            assert np.array_equal(gv["ranges"], oranges), f"{tag} ranges"
            assert float(np.max(np.abs(gv["T_final"] - ov["T_final"]))) <= 1e-6, f"{tag} T_final"
            assert np.array_equal(gv["last"], ov["last"]), f"{tag} last"
            assert np.array_equal(gv["tile_processed"], ov["tile_processed"]), f"{tag} tile_processed"
        n_img = int((gv["image"].view(np.uint32) != ov["image"].view(np.uint32)).sum())
        say(f"  {tag}: V={gv['vis'].size} M={gv['M']} image values not bit-identical: {n_img}")
        assert n_img == 0, f"{tag}: {n_img} image values not bit-identical"
        check_loss_grad(gv, ov, work.w_ssim)
    # the fused optimiser pass: union flags now hold the next step's view 0
    nxt = oracle.preprocess(res["params"], work.cameras[0])["visible"]
    assert np.array_equal(res["union_flags"], nxt.astype(np.uint8)), "union flags of the next step's view 0"
    res["union_flags"] = np.zeros_like(res["union_flags"])
    tol_g = 1e-3 * np.abs(ref["grads"]) + 1e-4 * ref["mags"] + ref["mags_dl"]
    check_adam(res, ref, work, p0, tol_g)
    for g2 in step.g2d:
        assert not g2.any().item(), "screen-space gradients not re-zeroed"
    # view 0's screen-space gradients from the split backward at 512 entries
    del step
    torch.cuda.empty_cache()
    one = synth.Workload(work.config, "mid_v0", work.params, work.cameras[:1], work.targets[:1], work.w_l1,
                         work.w_ssim, work.lr, work.beta1, work.beta2, work.eps)
    r1, s1 = run_gpu_step(one)
    assert s1.seg == [512]
    vis = oracle.preprocess(work.params, work.cameras[0])["visible"]
    ov = ref["views"][0]
    check_grad("mid_full/v0 grad2d (split 512)", r1["views"][0]["grad2d"][vis], ov["g2d"][vis], ov["m2d"][vis],
               ov["m2d_dl"][vis])


@pytest.mark.timeout(900)
def test_capacity_full_size_view_gradients(capacity_work):
    """One whole 1920x1080 view of the 12,000,000-Gaussian capacity scene
    (the last of its batch) through the HIP path with the oracle's image
    gradient fed to the backward: image, final transmittance, `last` and
    per-tile processed counts exactly; the library's own loss and dL/dI
    against the oracle's; the screen-space gradients of every visible
    Gaussian (split backward at 512 entries), the 59 gradient planes of all
    12M Gaussians, and the sparse Adam update of the view's visible rows
    against the oracle's gradients."""
    from test_gpu_parity import check_adam, check_loss_grad
    work = capacity_work
    k = len(work.cameras) - 1
    cam, tgt = work.cameras[k], work.targets[k]
    one = synth.Workload(work.config, "capacity_v15", work.params, [cam], [tgt], work.w_l1, work.w_ssim, work.lr,
                         work.beta1, work.beta2, work.eps)
    say(f"[capacity view] n={work.n} view {k}: oracle forward and loss")
    img, Tf, last, proc = oracle.render(work.params, cam)
    L, dL, _, _ = oracle.loss(img, tgt, work.w_l1, work.w_ssim)
    say("[capacity view] GPU step on the oracle's image gradient")
    res, step = run_gpu_step(one, record_tiles=True, dL_override=[dL])
    assert step.seg == [512]
    gv = res["views"][0]
    del step
    torch.cuda.empty_cache()
    say(f"[capacity view] M={gv['M']}")
    assert np.array_equal(gv["image"].view(np.uint32), img.view(np.uint32)), "image not bit-identical"
    assert np.array_equal(gv["T_final"].view(np.uint32), Tf.view(np.uint32)), "T_final"
    assert np.array_equal(gv["last"], last) and np.array_equal(gv["tile_processed"], proc), "last / processed"
    check_loss_grad(gv, dict(loss=L, dL_dimage=dL), work.w_ssim)
    say("[capacity view] oracle backward")
    g2d, m2d, grads, mags = oracle.backward(work.params, cam, dL, at_fp32=True)
    pre = oracle.preprocess(work.params, cam)
    vis = pre["visible"]
    assert np.array_equal(gv["vis"], np.flatnonzero(vis).astype(np.int32)), "visible list"
    check_grad("capacity_full/v15 grad2d", gv["grad2d"][vis], g2d[vis], m2d[vis])
    check_grad("capacity_full/v15 grads", res["grads"], grads, mags)
    ref = dict(union=np.flatnonzero(vis).astype(np.int32), grads=grads)
    check_adam(res, ref, one, work.params, 1e-3 * np.abs(grads) + 1e-4 * mags)
