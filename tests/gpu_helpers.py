"""Shared helpers of the GPU parity tests: run the HIP path through the
C ABI and collect its outputs as numpy arrays; tolerance checks against the
oracle.  Imported by the gpu-marked tests only."""
from __future__ import annotations

import sys

import numpy as np


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu_step(work, t=1, record_tiles=True, pair_capacity=None, device="cuda:0", dL_override=None,
                 segment_len=None):
    """One training step of the HIP path; per-view snapshots.  With
    ``dL_override`` (one [3][H][W] array per view) the backward is fed that
    image gradient instead of the library's loss output (to test the
    backward stages in isolation)."""
    import torch

    import differentiable_gaussian_splatting_dgs_amd as gs

    kw = {} if segment_len is None else {"segment_len": segment_len}
    step = gs.from_workload(work, device=device, record_tiles=record_tiles, pair_capacity=pair_capacity, **kw)
    views = []
    for k, vw in enumerate(step.views):
        step.forward_view(k)
        torch.cuda.synchronize()
        M = vw.num_pairs
        V = int(step.vis_count[k].item())
        out = dict(
            proj=step.proj[: step.n].cpu().numpy().copy(),
            vis=step.vis_idx[k][:V].cpu().numpy().copy(),
            M=M,
            keys=step_keys(step, vw, M),
            vals=step.vals[:M].cpu().numpy().copy(),
            ranges=vw.ranges.cpu().numpy().view(np.uint32).copy(),
            order=vw.order.cpu().numpy().view(np.uint32).copy(),
            image=vw.image.cpu().numpy().copy(),
            T_final=vw.T_final.cpu().numpy().copy(),
            last=vw.last.cpu().numpy().view(np.uint32).copy(),
            tile_processed=vw.tile_processed.cpu().numpy().view(np.uint32).copy(),
            loss=float(vw.loss.item()),
            dL=vw.dL.cpu().numpy().copy(),
        )
        if dL_override is not None:
            vw.dL.copy_(torch.as_tensor(np.asarray(dL_override[k], np.float32)))
        step.backward_view(k, keep_grad2d=True)
        torch.cuda.synchronize()
        out["grad2d"] = step.grad2d[: step.n, :9].cpu().numpy().copy()
        step.project_view(k)
        torch.cuda.synchronize()
        out["grad2d_after"] = step.grad2d[: step.n].cpu().numpy().copy()
        views.append(out)
    grads = step.grads.cpu().numpy().copy()
    step.t = t - 1
    step.adam()
    torch.cuda.synchronize()
    U = int(step.union_count.item())
    res = dict(views=views, grads=grads, params=step.params.cpu().numpy(), m=step.m.cpu().numpy(),
               v=step.v.cpu().numpy(), union=step.union_idx[:U].cpu().numpy().copy(),
               union_flags=step.union_flags[: step.n].cpu().numpy().copy(),
               grads_after=step.grads.cpu().numpy())
    return res, step


def keys_from_pairs(vals, ranges, proj):
    """The 64-bit sort keys (tile << 32 | depth bits) of a pair array, from
    its values, the tile ranges and the projected records: every position
    inside tile t's range gets tile t; a position no range covers keeps an
    all-ones tile, so gaps or ranges past the end never pass as a match."""
    M = vals.shape[0]
    r = ranges.astype(np.int64).reshape(-1, 2)
    tiles = np.full(M, 0xFFFFFFFF, np.uint64)
    nz = np.flatnonzero(r[:, 1] > r[:, 0])
    lens = r[nz, 1] - r[nz, 0]
    pos = np.arange(int(lens.sum()), dtype=np.int64) - np.repeat(np.cumsum(lens) - lens, lens) + np.repeat(r[nz, 0], lens)
    assert pos.size == 0 or (pos.min() >= 0 and pos.max() < M), "tile range outside the pair array"
    tiles[pos] = np.repeat(nz.astype(np.uint64), lens)
    depth = np.ascontiguousarray(proj[:, 12]).view(np.uint32).astype(np.uint64)
    return (tiles << np.uint64(32)) | depth[vals]


def step_keys(step, vw, M):
    """The keys of the view last prepared: as written by the binning when the
    step keeps them, else rebuilt from its values, ranges and records."""
    if step.keys is not None:
        return step.keys[:M].cpu().numpy().view(np.uint64).copy()
    return keys_from_pairs(step.vals[:M].cpu().numpy(), vw.ranges.cpu().numpy().view(np.uint32),
                           step.proj[: step.n].cpu().numpy())


def proj_fields(proj):
    """Split the [n][16] record buffer into named arrays."""
    u32 = proj.view(np.uint32)
    rx, ry = u32[:, 13], u32[:, 14]
    return dict(
        mean2d=proj[:, 0:2], conic=proj[:, 2:5], opacity=proj[:, 5], rgb=proj[:, 6:9],
        radius=proj.view(np.int32)[:, 11], depth=proj[:, 12],
        rect=np.stack([rx & 0xFFFF, ry & 0xFFFF, rx >> 16, ry >> 16], 1).astype(np.int32),
        tiles=u32[:, 15],
    )


def check_grad(name, gpu, ref, mag, extra=0.0, rel=1e-3, mtol=1e-4):
    """|gpu - ref| <= rel |ref| + mtol * mag + extra, elementwise, where mag
    bounds the sum of |terms| behind ref (so fp32 summation order can move
    the result by a few ulps of mag) and extra is an input tolerance
    propagated through the same terms.  Returns the worst ratio."""
    gpu = np.asarray(gpu, np.float64)
    err = np.abs(gpu - ref)
    tol = rel * np.abs(ref) + mtol * mag + extra + 1e-30
    ratio = err / tol
    ratio[~np.isfinite(gpu) & np.isfinite(ref)] = np.inf   # a NaN or inf is outside every tolerance
    worst = float(np.nanmax(ratio)) if ratio.size else 0.0
    nbad = int((~(ratio <= 1)).sum())
    say(f"  {name}: max|err|={err.max() if err.size else 0:.3g} worst err/tol={worst:.3g} bad={nbad}/{err.size}")
    if nbad:
        for idx in np.argsort(ratio, axis=None)[::-1][:8]:
            at = np.unravel_index(idx, ratio.shape)
            say(f"    at {tuple(int(x) for x in at)}: gpu={gpu[at]:.6e} ref={ref[at]:.6e} "
                f"mag={np.broadcast_to(mag, ratio.shape)[at]:.3e} ratio={ratio[at]:.3g}")
    assert nbad == 0, f"{name}: {nbad} entries outside tolerance (worst ratio {worst:.3g})"
    return worst


def check_forward(gv, ov_pre, okeys, ovals, oranges, oimg, oT, olast, oproc, tag=""):
    """Forward parity of one view: exact integers, fp32 floats."""
    pf = proj_fields(gv["proj"])
    vis = ov_pre["visible"]
    assert np.array_equal(gv["vis"], np.flatnonzero(vis).astype(np.int32)), f"{tag} visible list"
    assert np.array_equal(pf["tiles"], ov_pre["tiles"]), f"{tag} tiles_touched"
    assert np.array_equal(pf["rect"][vis], ov_pre["rect"][vis]), f"{tag} rect"
    assert np.array_equal(pf["radius"][vis], ov_pre["radius"][vis]), f"{tag} radius"
    assert np.array_equal(pf["depth"][vis].view(np.uint32), ov_pre["depth"][vis].view(np.uint32)), f"{tag} depth bits"
    for nm, a, b in [("mean2d", pf["mean2d"][vis], ov_pre["mean2d"][vis]),
                     ("conic", pf["conic"][vis], ov_pre["conic"][vis]),
                     ("opacity", pf["opacity"][vis], ov_pre["opacity"][vis]),
                     ("rgb", pf["rgb"][vis], ov_pre["rgb"][vis])]:
        inexact = int((a.view(np.uint32) != b.view(np.uint32)).sum())
        d = np.abs(a.astype(np.float64) - b) / np.maximum(np.abs(b.astype(np.float64)), 1e-30)
        say(f"  {tag} {nm}: not bit-identical {inexact}/{a.size}, max rel {d.max() if d.size else 0:.3g}")
        assert d.size == 0 or d.max() <= 1e-6, f"{tag} {nm}"
    assert gv["M"] == len(okeys), f"{tag} M {gv['M']} vs {len(okeys)}"
    assert np.array_equal(gv["keys"], okeys), f"{tag} keys"
    assert np.array_equal(gv["vals"], ovals), f"{tag} values"
    assert np.array_equal(gv["ranges"], oranges), f"{tag} tile ranges"
    if "order" in gv:
        # launch order: tiles stably sorted by descending bit length of the pair count
        n_pairs = (oranges[:, 1] - oranges[:, 0]).astype(np.int64)
        bits = np.where(n_pairs > 0, np.floor(np.log2(np.maximum(n_pairs, 1))).astype(np.int64) + 1, 0)
        expect = np.argsort(-bits, kind="stable").astype(np.uint32)
        assert np.array_equal(gv["order"], expect), f"{tag} tile order"
    if oimg is None:       # preprocess and binning only
        return
    d_img = float(np.max(np.abs(gv["image"] - oimg))) if oimg.size else 0.0
    n_img = int((gv["image"].view(np.uint32) != oimg.view(np.uint32)).sum())
    say(f"  {tag} image max|diff|={d_img:.3g} not bit-identical {n_img}/{oimg.size}")
    assert d_img <= 1e-4, f"{tag} image"
    assert float(np.max(np.abs(gv["T_final"] - oT))) <= 1e-6, f"{tag} T_final"
    assert np.array_equal(gv["last"], olast), f"{tag} last"
    if oproc is not None:
        assert np.array_equal(gv["tile_processed"], oproc), f"{tag} tile_processed"
