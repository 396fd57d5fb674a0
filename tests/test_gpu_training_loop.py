"""The training step inside a loop (Grendel-GS notes, "training pipeline":
steps repeat, and densification -- clone, split, prune -- runs between
them), through the C ABI:

* two steps with the densification statistic tracked, then densify, then
  one more step, each stage held to the oracle on the state the GPU reached
  (the trajectories may part by the ±lr sign ambiguity of Adam at tiny
  gradients, so the oracle replays each stage from the GPU's own inputs):
  the statistic's counts exactly and its sums within the gradient
  tolerance, the rebuild exactly as the oracle's densify of the same
  statistic, and the step after it (new Gaussian count) against the
  oracle: integers exact, gradients and the Adam update (now with non-zero
  moments) within the stated tolerances;
* checkpoint and resume: k steps, save, a fresh TrainStep loads the file,
  then one step each: the resumed run renders bit-identical images and
  losses and ends within the Adam tolerance of the run that never stopped.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import check_grad, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _work():
    return synth.cut_down(synth.workload(2), 320, 180, n=30000)


def _with_params(work, params):
    return synth.Workload(work.config, work.name, params, work.cameras, work.targets, work.w_l1, work.w_ssim,
                          work.lr, work.beta1, work.beta2, work.eps)


def test_densify_in_the_training_loop():
    import differentiable_gaussian_splatting_dgs_amd as gs
    from test_gpu_parity import DL_TOL
    work = _work()
    nv = len(work.cameras)
    step = gs.from_workload(work, record_tiles=True)
    step.track_densify()
    acc_ref = np.zeros(work.n)
    acc_tol = np.zeros(work.n)
    den_ref = np.zeros(work.n, np.int64)
    for s in range(2):
        p_before = step.params.cpu().numpy().copy()
        step.step()
        torch.cuda.synchronize()
        # the statistic of this step: every view's |dL/d(u, v)| of its visible
        # rows, from the oracle's screen-space gradients at the same parameters
        ref = oracle.step(_with_params(work, p_before), dl_tol=DL_TOL)
        for vw in ref["views"]:
            vis = np.zeros(work.n, bool)
            vis[vw["visible"]] = True
            g = vw["g2d"][:, :2]
            acc_ref[vis] += np.hypot(g[vis, 0], g[vis, 1])
            tol = 1e-3 * np.abs(g) + 1e-4 * vw["m2d"][:, :2] + vw["m2d_dl"][:, :2]
            acc_tol[vis] += np.hypot(tol[vis, 0], tol[vis, 1]) + 1e-6 * np.hypot(g[vis, 0], g[vis, 1])
            den_ref[vis] += 1
        say(f"  step {s + 1}: union {int(step.union_count.item())}")
    acc = step.dens_accum.cpu().numpy().astype(np.float64)
    den = step.dens_denom.cpu().numpy()
    assert np.array_equal(den, den_ref), "densification counts"
    bad = np.abs(acc - acc_ref) > acc_tol + 1e-30
    say(f"  statistic: max|err| {np.abs(acc - acc_ref).max():.3g}, outside tolerance {int(bad.sum())}")
    assert not bad.any(), "densification sums"
    # densify: thresholds at quantiles of the GPU's statistic, the rebuild
    # against the oracle's densify of exactly that statistic
    a32, d32 = step.dens_accum.cpu().numpy(), den
    g = np.where(d32 > 0, a32 / np.maximum(d32, 1).astype(np.float32), 0).astype(np.float32)
    thr = float(np.quantile(g[d32 > 0], 0.7))
    p0, m0, v0 = step.params.cpu().numpy(), step.m.cpu().numpy(), step.v.cpu().numpy()
    lst = float(np.quantile(p0[3:6].max(0), 0.5))
    lgt = float(np.quantile(p0[10], 0.1))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    normals = torch.randn((2, 3, work.n), generator=gen, device="cuda")
    n_new = step.densify(thr, lst, lgt, normals=normals)
    out, om, ov = oracle.densify(p0, m0, v0, a32, d32, thr, lst, lgt, normals.cpu().numpy(), np.log(1.6))
    say(f"  densify: {work.n} -> {n_new} Gaussians (oracle {out.shape[1]})")
    assert n_new == out.shape[1] and n_new != work.n
    pg = step.params.cpu().numpy()
    n_kept_clone = n_new - 2 * int(((g >= thr) & (p0[3:6].max(0) > lst) & (p0[10] >= lgt)).sum())
    assert np.array_equal(pg[:, :n_kept_clone], out[:, :n_kept_clone].astype(np.float32))
    assert np.array_equal(pg[3:, n_kept_clone:], out[3:, n_kept_clone:].astype(np.float32))
    mean_tol = 1e-6 * (np.abs(out[0:3, n_kept_clone:]) + 10.0)
    assert np.all(np.abs(pg[0:3, n_kept_clone:] - out[0:3, n_kept_clone:]) <= mean_tol)
    assert np.array_equal(step.m.cpu().numpy(), om.astype(np.float32))
    assert np.array_equal(step.v.cpu().numpy(), ov.astype(np.float32))
    assert step.n == n_new and not step.dens_accum.any().item() and step.t == 2
    # one more step at the new count: views and gradients against the oracle,
    # then Adam with the moments the densify kept
    p3, m3, v3 = pg.copy(), step.m.cpu().numpy().copy(), step.v.cpu().numpy().copy()
    step.run_views()
    torch.cuda.synchronize()
    work3 = _with_params(work, p3)
    ref = oracle.step(work3, dl_tol=DL_TOL)
    for k, (vw, ovw) in enumerate(zip(step.views, ref["views"])):
        V = int(step.vis_count[k].item())
        assert np.array_equal(step.vis_idx[k][:V].cpu().numpy(), ovw["visible"]), f"v{k} visible list"
        assert np.array_equal(vw.last.cpu().numpy().view(np.uint32), ovw["last"]), f"v{k} last"
        assert float(np.max(np.abs(vw.image.cpu().numpy() - ovw["image"]))) <= 1e-4, f"v{k} image"
    grads = step.grads.cpu().numpy().copy()
    tol_g = 1e-3 * np.abs(ref["grads"]) + 1e-4 * ref["mags"] + ref["mags_dl"]
    check_grad("after densify: grads", grads, ref["grads"], ref["mags"], ref["mags_dl"])
    step.adam()
    torch.cuda.synchronize()
    U = int(step.union_count.item())
    assert np.array_equal(step.union_idx[:U].cpu().numpy(), ref["union"]), "union after densify"
    rows = ref["union"]
    b1, b2, lr, eps = work.beta1, work.beta2, work.lr, work.eps
    t = 3
    gr, tg = ref["grads"][:, rows], tol_g[:, rows]
    m_new = step.m.cpu().numpy()[:, rows].astype(np.float64)
    v_new = step.v.cpu().numpy()[:, rows].astype(np.float64)
    mb, vb = m3[:, rows].astype(np.float64), v3[:, rows].astype(np.float64)
    assert np.all(np.abs(m_new - (b1 * mb + (1 - b1) * gr)) <= (1 - b1) * tg + 1e-6 * np.abs(m_new) + 1e-30), "m"
    lo = b2 * vb + (1 - b2) * np.maximum(np.abs(gr) - tg, 0) ** 2
    hi = b2 * vb + (1 - b2) * (np.abs(gr) + tg) ** 2
    assert np.all((v_new >= lo * (1 - 2e-6) - 1e-30) & (v_new <= hi * (1 + 2e-6) + 1e-30)), "v"
    # the update from the moments the GPU holds, in fp64
    p_new = step.params.cpu().numpy()[:, rows].astype(np.float64)
    bc1, bc2 = 1 - b1 ** t, 1 - b2 ** t
    p_ref = p3[:, rows] - lr * (m_new / bc1) / (np.sqrt(v_new / bc2) + eps)
    tol_p = 4 * np.spacing(np.abs(p3[:, rows]).astype(np.float32)).astype(np.float64) + 1e-5 * lr
    assert np.all(np.abs(p_new - p_ref) <= tol_p), "params after densify"
    outside = np.ones(step.n, bool)
    outside[rows] = False
    assert np.array_equal(step.params.cpu().numpy()[:, outside], p3[:, outside]), "unlisted rows touched"


def test_checkpoint_and_resume(tmp_path):
    import differentiable_gaussian_splatting_dgs_amd as gs
    work = _work()
    a = gs.from_workload(work, record_tiles=True)
    for _ in range(2):
        a.step()
    path = str(tmp_path / "state.pt")
    a.save_checkpoint(path)
    st = {k: (v.cpu().numpy().copy() if torch.is_tensor(v) else v) for k, v in a.state().items()}
    b = gs.from_workload(work, record_tiles=True)
    b.load_checkpoint(path)
    assert b.t == 2
    for k in ("params", "m", "v"):
        assert np.array_equal(getattr(b, k).cpu().numpy(), st[k]), k
    a.step()
    b.step()
    torch.cuda.synchronize()
    for k, (va, vb) in enumerate(zip(a.views, b.views)):
        assert torch.equal(va.image, vb.image), f"v{k} image"
        assert torch.equal(va.last, vb.last), f"v{k} last"
        assert float(va.loss.item()) == float(vb.loss.item()), f"v{k} loss"
    # gradients differ only by the order of float atomics: the updates agree
    # to within fp32 rounding of the gradients, except where a gradient is
    # so small that its sign (and so Adam's step) is not determined
    pa, pb = a.params.cpu().numpy().astype(np.float64), b.params.cpu().numpy().astype(np.float64)
    d = np.abs(pa - pb)
    lr = work.lr
    assert np.all(d <= 2 * lr + 1e-7), "resumed parameters beyond the Adam step bound"
    frac = float((d > 1e-3 * lr).mean())
    say(f"  resume: max |dp| {d.max():.3g}, fraction differing by > 1e-3 lr: {frac:.2e}")
    assert frac < 1e-2
