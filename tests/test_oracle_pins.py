"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these re-types the oracle's own formulas: each compares it with a
closed form, an invariant, brute force, a library routine (numpy sort /
union, scipy Gaussian filter, torch Adam) or central differences.  CPU only.
"""
import math

import numpy as np
import pytest

import oracle
import synth


def camera(width=128, height=128, z=4.0):
    """cfg-0 style camera at (0, 0, -z) looking along +z (R = I)."""
    return synth.ring_camera(width, height, 0.0, radius=z)


def gaussians(n):
    """n Gaussians, identity rotation, zero SH, logit 0."""
    p = np.zeros((59, n), np.float32)
    p[6] = 1.0
    return p


# ---------------------------------------------------------------------------
# the written exponential
# ---------------------------------------------------------------------------

def test_pexp_accuracy_and_specials():
    xs = np.concatenate([np.linspace(-87.0, 88.0, 200001, dtype=np.float32),
                         np.float32([0.0, -0.0, 1e-30, -1e-30, -5.5413, -4.5, 1.0])])
    got = oracle.pexp(xs).astype(np.float64)
    ref = np.exp(xs.astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    assert np.max(np.abs(got - ref) / ulp) <= 1.0          # within one fp32 ulp
    assert oracle.pexp([0.0])[0] == 1.0
    assert oracle.pexp([-88.0])[0] == 0.0
    assert math.isinf(oracle.pexp([89.0])[0])
    assert math.isnan(oracle.pexp([float("nan")])[0])
    assert np.all(got[:-7] >= np.finfo(np.float32).tiny)  # never subnormal


def test_aexp_accuracy_and_range():
    """The compositing weight's exponential on [-5.6, 0]: within 6e-7
    relative of e^x (the polynomial's 9.2e-8 on [-1/2, 1/2], the rounding
    of x log2 e -- at most 2^-21, a relative 3.3e-7 of 2^t -- and the fp32
    evaluation), exactly 1 at 0, nondecreasing, and below 1/255 at -5.6, so
    skipping power < -5.6 drops no entry the rule would composite (o <= 1).
    A wrong coefficient, sign or scaling breaks the bound."""
    xs = np.linspace(-5.6, 0.0, 200001, dtype=np.float32)
    got = oracle.aexp(xs).astype(np.float64)
    ref = np.exp(xs.astype(np.float64))
    assert np.max(np.abs(got - ref) / ref) <= 6e-7
    assert np.all(np.diff(got) >= 0.0)
    assert oracle.aexp([0.0])[0] == 1.0 and oracle.aexp([-0.0])[0] == 1.0
    assert oracle.aexp([-5.6])[0] < 1.0 / 255.0
    # integer powers of e^(ln 2) land on powers of two up to the fit's error
    for k in range(0, 9):
        x = np.float32(-k * math.log(2.0))
        assert abs(float(oracle.aexp([x])[0]) - math.exp(float(x))) <= 6e-7 * math.exp(float(x))


# ---------------------------------------------------------------------------
# spherical harmonics (view-dependent colour of the 48 coefficients)
# ---------------------------------------------------------------------------

def test_sh_orthonormal_by_quadrature():
    # Gauss-Legendre in cos(theta) x uniform in phi: exact for these degrees
    ct, wt = np.polynomial.legendre.leggauss(16)
    phi = (np.arange(32) + 0.5) * 2 * np.pi / 32
    C, P = np.meshgrid(ct, phi, indexing="ij")
    st = np.sqrt(1 - C * C)
    d = np.stack([st * np.cos(P), st * np.sin(P), C], -1).reshape(-1, 3)
    w = (wt[:, None] * np.full(32, 2 * np.pi / 32)[None, :]).reshape(-1)
    Y = oracle.sh_basis(d)
    G = (Y * w[:, None]).T @ Y
    assert np.allclose(G, np.eye(16), atol=1e-12)


def test_sh_values_on_axes():
    c0 = 0.5 / math.sqrt(math.pi)
    c1 = math.sqrt(3 / (4 * math.pi))
    c2c = math.sqrt(15 / (16 * math.pi))
    c2b = math.sqrt(5 / (16 * math.pi))
    c3a = math.sqrt(35 / (32 * math.pi))
    c3c = math.sqrt(21 / (32 * math.pi))
    c3d = math.sqrt(7 / (16 * math.pi))
    Y = oracle.sh_basis(np.eye(3))
    ex, ey, ez = Y
    exp_x = np.zeros(16); exp_y = np.zeros(16); exp_z = np.zeros(16)
    for e in (exp_x, exp_y, exp_z):
        e[0] = c0
        e[6] = -c2b
    exp_x[3] = c1; exp_x[8] = c2c; exp_x[13] = -c3c; exp_x[15] = c3a
    exp_y[1] = c1; exp_y[8] = -c2c; exp_y[9] = -c3a; exp_y[11] = -c3c
    exp_z[2] = c1; exp_z[6] = 2 * c2b; exp_z[12] = 2 * c3d
    assert np.allclose(ex, exp_x, atol=1e-15)
    assert np.allclose(ey, exp_y, atol=1e-15)
    assert np.allclose(ez, exp_z, atol=1e-15)
    d = np.random.default_rng(0).normal(size=(1000, 3))
    d /= np.linalg.norm(d, axis=1, keepdims=True)
    assert np.allclose(oracle.sh_basis(d, np.float32), oracle.sh_basis(d), atol=3e-6)


# ---------------------------------------------------------------------------
# one isotropic Gaussian on the optical axis: closed forms
# ---------------------------------------------------------------------------

def _single(s=0.03, z=3.0, logit=0.7, dc=(0.9, -0.3, 0.2)):
    cam = camera()
    p = gaussians(1)
    p[2, 0] = z - 4.0                    # camera at z = -4
    p[3:6, 0] = math.log(s)
    p[10, 0] = logit
    p[11:14, 0] = dc
    return p, cam


def _single_closed_form(s, z, logit, dc, cam):
    # the parameters as the oracle sees them: stored in fp32
    s = math.exp(float(np.float32(math.log(s))))
    logit = float(np.float32(logit))
    dc = np.float32(dc).astype(np.float64)
    fx = np.float64(np.float32(cam.fx))
    var = (fx * s / z) ** 2 + 0.3
    o = 1 / (1 + math.exp(-logit))
    c0 = 0.5 / math.sqrt(math.pi)
    rgb = np.maximum(np.array(dc) * c0 + 0.5, 0.0)
    xs = np.arange(cam.width) + 0.5 - cam.cx
    ys = np.arange(cam.height) + 0.5 - cam.cy
    rho2 = ys[:, None] ** 2 + xs[None, :] ** 2
    alpha = np.minimum(0.99, o * np.exp(-rho2 / (2 * var)))
    alpha = np.where(alpha < 1 / 255, 0.0, alpha)
    return var, o, rgb, rho2, alpha


def test_single_gaussian_projection_closed_form():
    s, z, logit, dc = 0.03, 3.0, 0.7, (0.9, -0.3, 0.2)
    p, cam = _single(s, z, logit, dc)
    var, o, rgb, _, _ = _single_closed_form(s, z, logit, dc, cam)
    pre = oracle.preprocess(p, cam)
    assert pre["visible"][0]
    assert np.allclose(pre["mean2d"][0], [cam.cx, cam.cy], atol=1e-5)
    assert np.allclose(pre["cov2d"][0], [var, 0.0, var], rtol=1e-5, atol=1e-7)
    assert np.allclose(pre["conic"][0], [1 / var, 0.0, 1 / var], rtol=1e-5, atol=1e-7)
    r = math.ceil(3 * math.sqrt(var))
    assert pre["radius"][0] == r
    x0 = max(0, math.floor((cam.cx - r) / 16)); x1 = min(8, math.floor((cam.cx + r) / 16) + 1)
    assert list(pre["rect"][0]) == [x0, x0, x1, x1]
    assert pre["tiles"][0] == (x1 - x0) ** 2
    assert np.isclose(pre["opacity"][0], o, rtol=1e-6)
    assert np.allclose(pre["rgb"][0], rgb, rtol=1e-6)
    assert pre["depth"][0] == np.float32(z)


def test_single_gaussian_image_closed_form():
    s, z, logit, dc = 0.03, 3.0, 0.7, (0.9, -0.3, 0.2)
    p, cam = _single(s, z, logit, dc)
    var, o, rgb, rho2, alpha = _single_closed_form(s, z, logit, dc, cam)
    img, Tf, last, _ = oracle.render(p, cam)
    r = math.ceil(3 * math.sqrt(var))
    # outside the tile rectangle nothing is drawn
    x0 = max(0, math.floor((cam.cx - r) / 16)) * 16; x1 = min(128, (math.floor((cam.cx + r) / 16) + 1) * 16)
    inside = np.zeros((128, 128), bool)
    inside[x0:x1, x0:x1] = True
    expect = np.where(inside, alpha, 0.0)
    for c in range(3):
        assert np.max(np.abs(img[c] - rgb[c] * expect)) < 2e-6
    assert np.max(np.abs(Tf - (1 - expect))) < 2e-6
    assert np.array_equal(last, (expect > 0).astype(np.uint32))


def test_single_gaussian_gradients_closed_form():
    s, z, logit, dc = 0.03, 3.0, 0.7, (0.9, -0.3, 0.2)
    p, cam = _single(s, z, logit, dc)
    var, o, rgb, rho2, alpha = _single_closed_form(s, z, logit, dc, cam)
    G = np.random.default_rng(5).normal(size=(3, 128, 128))
    _, _, grads, _ = oracle.backward(p, cam, G)
    c0 = 0.5 / math.sqrt(math.pi)
    e = alpha / o
    live = alpha > 0
    # dL/d(SH DC_c) = sum_p G_c alpha_p Y0
    for c in range(3):
        assert np.isclose(grads[11 + c, 0], c0 * np.sum(G[c] * alpha), rtol=1e-9)
    # dL/dlogit = sum_p (G . rgb) e_p * o (1 - o)
    Grgb = np.tensordot(rgb, G, axes=1)
    assert np.isclose(grads[10, 0], np.sum(Grgb * e * live) * o * (1 - o), rtol=1e-9)
    # dL/dlogscale_x: power = -dx^2/(2a) - dy^2/(2c), a = fx^2 s_x^2/z^2 + 0.3
    fx = np.float64(np.float32(cam.fx))
    xs = np.arange(128) + 0.5 - cam.cx
    dx2 = np.broadcast_to(xs[None, :] ** 2, (128, 128))
    dy2 = np.broadcast_to(xs[:, None] ** 2, (128, 128))
    s = math.exp(float(np.float32(math.log(s))))
    da = 2 * fx ** 2 * s ** 2 / z ** 2
    g_lsx = np.sum(Grgb * alpha * dx2 / (2 * var ** 2)) * da
    g_lsy = np.sum(Grgb * alpha * dy2 / (2 * var ** 2)) * da
    assert np.isclose(grads[3, 0], g_lsx, rtol=1e-8)
    assert np.isclose(grads[4, 0], g_lsy, rtol=1e-8)
    assert abs(grads[5, 0]) < 1e-12 * abs(g_lsx)       # no depth extent on the axis


# ---------------------------------------------------------------------------
# compositing order: stacked Gaussians on the axis
# ---------------------------------------------------------------------------

def test_stacked_gaussians_front_to_back():
    cam = camera()
    p = gaussians(2)
    p[2] = [-1.0, 0.5]                      # depths 3 and 4.5
    p[3:6] = math.log(0.05)
    p[10] = [0.3, 1.2]
    p[11:14, 0] = [1.0, 0.0, -0.5]
    p[11:14, 1] = [-0.5, 0.8, 0.4]
    img, Tf, _, _ = oracle.render(p, cam)
    pre = oracle.preprocess(p, cam)
    # closed form at the centre pixels (both Gaussians cover them fully)
    c = (63, 64)
    for px, py in [(63, 63), (64, 64), (60, 66)]:
        al = []
        for i in range(2):
            u, v = pre["mean2d"][i]
            A, B, C = pre["conic"][i].astype(np.float64)
            dx, dy = px + 0.5 - u, py + 0.5 - v
            pw = -0.5 * (A * dx * dx + C * dy * dy) - B * dx * dy
            al.append(min(0.99, pre["opacity"][i] * math.exp(pw)))
        a1, a2 = al
        expect = pre["rgb"][0] * a1 + pre["rgb"][1] * a2 * (1 - a1)
        assert np.allclose(img[:, py, px], expect, atol=1e-6)
        assert abs(Tf[py, px] - (1 - a1) * (1 - a2)) < 1e-6
    # swapping the depths swaps the order
    q = p.copy()
    q[2] = [0.5, -1.0]
    img2, _, _, _ = oracle.render(q, cam)
    pre2 = oracle.preprocess(q, cam)
    px, py = c
    al = []
    for i in range(2):
        u, v = pre2["mean2d"][i]
        A, B, C = pre2["conic"][i].astype(np.float64)
        dx, dy = px + 0.5 - u, py + 0.5 - v
        al.append(min(0.99, pre2["opacity"][i] * math.exp(-0.5 * (A * dx * dx + C * dy * dy) - B * dx * dy)))
    expect = pre2["rgb"][1] * al[1] + pre2["rgb"][0] * al[0] * (1 - al[1])
    assert np.allclose(img2[:, py, px], expect, atol=1e-6)


# ---------------------------------------------------------------------------
# invariants and brute force on the seeded scenes
# ---------------------------------------------------------------------------

def test_composited_counts_against_the_weights():
    """A pixel's composited count is the number of non-zero compositing
    weights (alpha T >= 1/255 * 1e-4 > 0): with one colour c for every
    Gaussian, C / c = sum of weights, and each composited Gaussian adds at
    least 1/255 of T >= 1e-4; the count never exceeds `last`."""
    w = synth.workload(0)
    cam = w.cameras[0]
    cnt = oracle.composited_counts(w.params, cam)
    _, _, last, _ = oracle.render(w.params, cam)
    assert np.all(cnt <= last) and np.array_equal(cnt > 0, last > 0)
    p = w.params.copy()
    p[11:59] = 0.0
    p[11:14] = 0.7
    img, Tf, _, _ = oracle.render(p, cam)
    rgb = oracle.preprocess(p, cam)["rgb"][0]
    wsum = img[0] / rgb[0]
    assert np.all(wsum >= cnt * (1e-4 / 255) * (1 - 1e-5))
    assert cnt.sum() > 5 * cnt.size


def test_weights_plus_transmittance_is_one():
    w = synth.workload(0)
    p = w.params.copy()
    p[11:59] = 0.0
    p[11:14] = 0.7                         # one colour for every Gaussian
    img, Tf, _, _ = oracle.render(p, w.cameras[0])
    rgb = oracle.preprocess(p, w.cameras[0])["rgb"][0]
    for c in range(3):
        assert np.max(np.abs(img[c] / rgb[c] + Tf - 1.0)) < 1e-6


@pytest.mark.parametrize("case", ["cfg0", "cfg1_cut"])
def test_brute_force_equals_tiled_bitwise(case):
    if case == "cfg0":
        w = synth.workload(0)
    else:
        w = synth.cut_down(synth.workload(1), 200, 136, n=6000)
    cam = w.cameras[0]
    a = oracle.render(w.params, cam)
    b = oracle.render_brute(w.params, cam)
    for x, y in zip(a[:3], b):
        assert np.array_equal(x, y)


def test_sampled_pixel_compositing_equals_tiled_render():
    """Compositing single pixels against given tile lists reproduces the
    tiled render bit for bit (the lists here are the oracle's own sort)."""
    w = synth.cut_down(synth.workload(1), 160, 96, n=3000)
    cam = w.cameras[0]
    img, Tf, last, _ = oracle.render(w.params, cam)
    _, vals, ranges = oracle.bin_sort(w.params, cam)
    py, px = np.mgrid[0:cam.height, 0:cam.width]
    rgb, T1, l1 = oracle.composite_pixels(w.params, cam, vals, ranges, px.ravel(), py.ravel())
    assert np.array_equal(rgb.T.reshape(3, cam.height, cam.width), img)
    assert np.array_equal(T1.reshape(cam.height, cam.width), Tf)
    assert np.array_equal(l1.reshape(cam.height, cam.width), last)
    assert (last > 0).mean() > 0.1


def test_binning_matches_numpy_stable_sort():
    w = synth.cut_down(synth.workload(1), 200, 136, n=6000)
    cam = w.cameras[0]
    pre = oracle.preprocess(w.params, cam)
    TX, TY = oracle.tiles_of(cam)
    k_list, v_list = [], []
    depth_bits = pre["depth"].view(np.uint32).astype(np.uint64)
    for i in np.flatnonzero(pre["visible"]):
        x0, y0, x1, y1 = pre["rect"][i]
        for ty in range(y0, y1):
            for tx in range(x0, x1):
                k_list.append((np.uint64(ty * TX + tx) << np.uint64(32)) | depth_bits[i])
                v_list.append(i)
    k = np.array(k_list, np.uint64)
    v = np.array(v_list, np.int32)
    order = np.argsort(k, kind="stable")
    keys, vals, ranges = oracle.bin_sort(w.params, cam)
    assert len(keys) == int(pre["tiles"].sum())
    assert np.array_equal(keys, k[order]) and np.array_equal(vals, v[order])
    # ranges partition [0, M) in tile order, empty tiles [0, 0)
    tile = (keys >> np.uint64(32)).astype(np.int64)
    for t in range(TX * TY):
        s, e = ranges[t]
        idx = np.flatnonzero(tile == t)
        if idx.size == 0:
            assert s == 0 and e == 0
        else:
            assert s == idx[0] and e == idx[-1] + 1 and e - s == idx.size


def test_visible_set_semantics():
    cam = camera()
    p = gaussians(6)
    p[3:6] = math.log(0.05)
    p[2] = [0.0, -4.1, 0.0, 0.0, 0.0, 0.0]      # #1 behind the camera
    p[0, 2] = 50.0                               # #2 far off-screen
    p[7, 3] = np.nan                             # #3 NaN quaternion
    p[6:10, 4] = 0.0                             # #4 zero quaternion
    p[20, 5] = np.inf                            # #5 infinite SH coefficient
    pre = oracle.preprocess(p, cam)
    assert list(pre["visible"]) == [True, False, False, False, False, False]
    assert list(oracle.visible_list(p, cam)) == [0]
    assert np.all(pre["tiles"][1:] == 0)


# ---------------------------------------------------------------------------
# loss: L1 + SSIM with an 11x11 Gaussian window (sigma 1.5)
# ---------------------------------------------------------------------------

def test_l1_of_constants():
    a = np.full((3, 20, 30), 0.25, np.float32)
    b = np.full((3, 20, 30), 0.75, np.float32)
    L, dL, l1, _ = oracle.loss(a, b, 1.0, 0.0)
    assert L == pytest.approx(0.5) and l1 == pytest.approx(0.5)
    assert np.allclose(dL, -1.0 / (3 * 20 * 30))
    L, dL, _, _ = oracle.loss(a, a, 1.0, 0.0)
    assert L == 0.0 and np.all(dL == 0.0)       # subgradient 0 at 0


def test_ssim_identity_and_constants():
    x = np.random.default_rng(1).uniform(size=(3, 24, 40)).astype(np.float32)
    L, dL, l1, ss = oracle.loss(x, x, 0.8, 0.2)
    assert ss == pytest.approx(1.0, abs=1e-12) and L == pytest.approx(0.0, abs=1e-12)
    assert np.max(np.abs(dL)) < 1e-14
    a, b = 0.3, 0.6
    A = np.full((1, 40, 40), a, np.float32)
    B = np.full((1, 40, 40), b, np.float32)
    A3, B3 = np.repeat(A, 3, 0), np.repeat(B, 3, 0)
    # interior pixels (>= 5 from the border) see the full window
    fa, fb = np.float64(np.float32(a)), np.float64(np.float32(b))
    C1 = 0.01 ** 2
    ssim_in = (2 * fa * fb + C1) / (fa * fa + fb * fb + C1)
    from scipy.ndimage import gaussian_filter
    ref = _scipy_ssim_map(A3[0].astype(np.float64), B3[0].astype(np.float64), gaussian_filter)
    assert np.allclose(ref[5:-5, 5:-5], ssim_in, rtol=1e-12)


def _scipy_ssim_map(x, y, gaussian_filter):
    f = lambda z: gaussian_filter(z, 1.5, mode="constant", cval=0.0, truncate=5.0 / 1.5)
    C1, C2 = 0.01 ** 2, 0.03 ** 2
    mx, my = f(x), f(y)
    vx = f(x * x) - mx * mx
    vy = f(y * y) - my * my
    cxy = f(x * y) - mx * my
    return (2 * mx * my + C1) * (2 * cxy + C2) / ((mx * mx + my * my + C1) * (vx + vy + C2))


def test_ssim_matches_scipy_gaussian_filter():
    from scipy.ndimage import gaussian_filter
    rng = np.random.default_rng(2)
    x = rng.uniform(size=(3, 33, 47)).astype(np.float32)
    y = np.clip(x + rng.normal(0, 0.2, x.shape), 0, 1).astype(np.float32)
    _, _, l1, ss = oracle.loss(x, y, 0.8, 0.2)
    ref = np.mean([_scipy_ssim_map(x[c].astype(np.float64), y[c].astype(np.float64), gaussian_filter)
                   for c in range(3)])
    assert ss == pytest.approx(ref, rel=1e-12)
    assert l1 == pytest.approx(np.mean(np.abs(x.astype(np.float64) - y)), rel=1e-12)


def test_loss_gradient_central_differences():
    rng = np.random.default_rng(3)
    x = rng.uniform(size=(3, 18, 21)).astype(np.float32)
    y = rng.uniform(size=(3, 18, 21)).astype(np.float32)
    _, dL, _, _ = oracle.loss(x, y, 0.8, 0.2)
    x64 = x.astype(np.float64)
    for (c, i, j) in [(0, 0, 0), (1, 9, 10), (2, 17, 20), (0, 4, 15), (2, 12, 3)]:
        h = 1e-6
        xp = x64.copy(); xp[c, i, j] += h
        xm = x64.copy(); xm[c, i, j] -= h
        fd = (oracle.loss_frozen_f64(xp, x, y, 0.8, 0.2) - oracle.loss_frozen_f64(xm, x, y, 0.8, 0.2)) / (2 * h)
        assert fd == pytest.approx(dL[c, i, j], rel=1e-6, abs=1e-12)


# ---------------------------------------------------------------------------
# backward: central differences of the fp64 frozen-decision function
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("weights,h,tol", [((1.0, 0.0), 1e-4, 2e-5), ((0.8, 0.2), 1e-3, 2e-4)])
def test_backward_central_differences(weights, h, tol):
    w = synth.cut_down(synth.workload(0), 64, 48, n=300)
    cam = w.cameras[0]
    img, _, _, _ = oracle.render(w.params, cam)
    _, dL, _, _ = oracle.loss(img, w.targets[0], *weights)
    _, _, grads, mags = oracle.backward(w.params, cam, dL)
    vis = np.flatnonzero(oracle.preprocess(w.params, cam)["visible"])
    cand = vis[np.argsort(-np.abs(grads[0, vis]))[:4]]
    p64 = w.params.astype(np.float64)

    def f(p):
        return oracle.loss_frozen_f64(oracle.render_frozen_f64(w.params, p, cam), img, w.targets[0], *weights)

    worst = 0.0
    for i in cand:
        for k in range(59):
            hk = h * max(1.0, abs(p64[k, i]))
            pp = p64.copy(); pp[k, i] += hk
            pm = p64.copy(); pm[k, i] -= hk
            fd = (f(pp) - f(pm)) / (2 * hk)
            worst = max(worst, abs(fd - grads[k, i]) / (mags[k, i] + 1e-30))
    assert worst < tol


def test_projection_backward_central_differences():
    w = synth.cut_down(synth.workload(1), 200, 136, n=400)
    cam = w.cameras[0]
    vis = oracle.preprocess(w.params, cam)["visible"]
    n = w.n
    g2d = np.random.default_rng(4).normal(size=(n, 9))
    g2d[~vis] = 0.0
    an = oracle.project_backward(w.params, cam, g2d)
    p64 = w.params.astype(np.float64)
    for i in np.flatnonzero(vis)[:3]:
        for k in range(59):
            h = 1e-6 * max(1.0, abs(p64[k, i]))
            pp = p64.copy(); pp[k, i] += h
            pm = p64.copy(); pm[k, i] -= h
            op = oracle.project_outputs_f64(w.params, pp, cam)[i]
            om = oracle.project_outputs_f64(w.params, pm, cam)[i]
            fd = np.dot((op - om) / (2 * h), g2d[i])
            scale = np.sum(np.abs((op - om) / (2 * h) * g2d[i]))
            noise = 8 * np.finfo(np.float64).eps * np.sum(np.abs(op * g2d[i])) / h
            assert abs(fd - an[k, i]) <= 1e-6 * scale + noise, (i, k, fd, an[k, i])


def test_batch_of_identical_views_sums():
    w = synth.cut_down(synth.workload(1), 160, 112, n=3000)
    cam, tgt = w.cameras[0], w.targets[0]
    img, _, _, _ = oracle.render(w.params, cam)
    _, dL, _, _ = oracle.loss(img, tgt, 0.8, 0.2)
    _, _, g1, _ = oracle.backward(w.params, cam, dL)
    acc = np.zeros_like(g1)
    mags = np.zeros_like(g1)
    for _ in range(4):
        oracle.backward(w.params, cam, dL, acc, mags)
    assert np.allclose(acc, 4 * g1, rtol=1e-12, atol=0)
    v = oracle.visible_list(w.params, cam)
    assert np.array_equal(oracle.union_list([v, v, v, v]), v)


# ---------------------------------------------------------------------------
# sparse Adam
# ---------------------------------------------------------------------------

def test_adam_first_step_closed_form_and_untouched_rows():
    rng = np.random.default_rng(6)
    n = 50
    p = rng.normal(size=(59, n)).astype(np.float32)
    g = rng.normal(size=(59, n)) * 1e-3
    rows = np.array([1, 4, 5, 17, 49], np.int32)
    lr, b1, b2, eps = 2e-3, 0.9 ** 4, 0.999 ** 4, 1e-15
    pn, mn, vn = oracle.adam(p, g, np.zeros((59, n)), np.zeros((59, n)), rows, lr, b1, b2, eps)
    mask = np.zeros(n, bool)
    mask[rows] = True
    expect = p.astype(np.float64) - lr * g / (np.abs(g) + eps)
    assert np.allclose(pn[:, mask], expect[:, mask], rtol=1e-14, atol=1e-16)
    assert np.array_equal(pn[:, ~mask], p[:, ~mask].astype(np.float64))
    assert np.all(mn[:, ~mask] == 0) and np.all(vn[:, ~mask] == 0)


def test_adam_matches_torch_on_gathered_rows():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    n = 40
    p = rng.normal(size=(59, n)).astype(np.float32)
    rows = np.array([0, 3, 9, 10, 33], np.int32)
    lr, b1, b2, eps = 1e-3, 0.9, 0.999, 1e-15
    tp = torch.tensor(p[:, rows].astype(np.float64), requires_grad=True)
    opt = torch.optim.Adam([tp], lr=lr, betas=(b1, b2), eps=eps)
    P, M, V = p.astype(np.float64), np.zeros((59, n)), np.zeros((59, n))
    for t in range(1, 4):
        g = rng.normal(size=(59, n))
        opt.zero_grad()
        tp.grad = torch.tensor(g[:, rows])
        opt.step()
        P, M, V = oracle.adam(P, g, M, V, rows, lr, b1, b2, eps, step=t)
    assert np.allclose(P[:, rows], tp.detach().numpy(), rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------------------
# view coupling (Odin summary page: Jaccard edge weight, priority score)
# ---------------------------------------------------------------------------

def test_view_coupling_closed_forms():
    """Identical sets weigh 1, disjoint 0, an empty union 0 (the page's
    rule); a hand-worked example: {1,2,3,4} and {3,4,5} share 2 of 5."""
    a = np.array([1, 2, 3, 4], np.int32)
    b = np.array([3, 4, 5], np.int32)
    c = np.array([7, 9], np.int32)
    e = np.zeros(0, np.int32)
    inter = oracle.view_overlap([a, b, a, c, e])
    assert inter.tolist() == [[4, 2, 4, 0, 0], [2, 3, 2, 0, 0], [4, 2, 4, 0, 0], [0, 0, 0, 2, 0],
                              [0, 0, 0, 0, 0]]
    w = oracle.view_coupling(inter)
    assert w[0, 1] == 2 / 5 and w[1, 0] == 2 / 5
    assert w[0, 2] == 1.0 and w[0, 3] == 0.0 and w[4, 4] == 0.0 and w[4, 0] == 0.0
    assert w[3, 3] == 1.0
    # s(v | {0, 3}) = w_0v + w_3v
    s = oracle.view_priority(w, [0, 3])
    assert s.tolist() == [1.0, 2 / 5, 1.0, 1.0, 0.0]


def test_view_coupling_against_python_sets():
    """Random subsets of 0..999: intersections and Jaccard weights against
    Python set arithmetic (a different route to the same definition);
    the matrix is symmetric with the set sizes on its diagonal."""
    rng = np.random.default_rng(11)
    lists = []
    for k in range(7):
        p = rng.uniform(0.05, 0.9)
        lists.append(np.flatnonzero(rng.uniform(size=1000) < p).astype(np.int32))
    lists.append(np.zeros(0, np.int32))
    inter = oracle.view_overlap(lists)
    w = oracle.view_coupling(inter)
    sets = [set(x.tolist()) for x in lists]
    for i in range(len(sets)):
        for j in range(len(sets)):
            assert inter[i, j] == len(sets[i] & sets[j])
            u = len(sets[i] | sets[j])
            assert w[i, j] == (len(sets[i] & sets[j]) / u if u else 0.0)
    prev = [2, 5, 0]
    s = oracle.view_priority(w, prev)
    for v in range(len(sets)):
        assert s[v] == (w[2, v] + w[5, v]) + w[0, v]


# --- tile partition and the sparse all-to-all's two ends ---------------------

def test_tile_partition_closed_forms():
    # equal costs split into equal runs; a single costly tile closes the
    # block whose share it completes; no cost at all puts every tile in the
    # last block
    assert list(oracle.tile_partition([1] * 12, 4)) == [0, 3, 6, 9, 12]
    assert list(oracle.tile_partition([5] * 10, 5)) == [0, 2, 4, 6, 8, 10]
    assert list(oracle.tile_partition([0, 0, 100, 0], 3)) == [0, 3, 3, 4]
    assert list(oracle.tile_partition([0] * 5, 3)) == [0, 0, 0, 5]
    assert list(oracle.tile_partition([7, 1, 1, 1], 1)) == [0, 4]


def test_tile_partition_is_numpy_searchsorted():
    """bounds[d] = 1 + searchsorted(inclusive cumsum, d * total / K, 'left')
    (the exact rational targets are representable here: totals < 2^40 and
    K a power of two), and each block's cost stays within total / K plus
    one tile of the target."""
    rng = np.random.default_rng(11)
    for T, K in ((1, 1), (50, 4), (333, 8), (8160, 64), (977, 16)):
        cost = rng.integers(0, 5000, T) * (rng.random(T) < 0.7)
        b = oracle.tile_partition(cost, K)
        C = np.cumsum(cost.astype(np.int64))
        total = int(C[-1])
        ref = [0] + [1 + int(np.searchsorted(C, d * total / K, side="left")) if total > 0 else 0
                     for d in range(1, K)] + [T]
        assert list(b) == ref, (T, K)
        assert all(b[d] <= b[d + 1] for d in range(K))
        for d in range(K):
            blk = int(cost[b[d]:b[d + 1]].sum())
            assert blk <= total / K + cost.max() + 1e-9


def test_pack_records_against_the_sort_pairs():
    """With one block per tile the packed lists are the tile lists of the
    binning (the same pairs, ascending index instead of depth order); with
    one block every visible Gaussian is listed once, in order; unpacking
    rows of ones counts each Gaussian's blocks."""
    w = synth.cut_down(synth.workload(1), 160, 96, n=3000)
    cam = w.cameras[0]
    pre = oracle.preprocess(w.params, cam)
    TX, TY = oracle.tiles_of(cam)
    T = TX * TY
    _, vals, ranges = oracle.bin_sort(w.params, cam)
    off, idx = oracle.pack_records(pre["rect"], pre["visible"], np.arange(T + 1), TX)
    for t in range(T):
        a, b = ranges[t]
        assert np.array_equal(idx[off[t]:off[t + 1]], np.sort(vals[a:b])), t
    off1, idx1 = oracle.pack_records(pre["rect"], pre["visible"], [0, T], TX)
    assert list(off1) == [0, int(pre["visible"].sum())]
    assert np.array_equal(idx1, np.flatnonzero(pre["visible"]))
    # rows of ones: each Gaussian's row gains its number of blocks
    g = oracle.unpack_grads(np.zeros((w.n, 12), np.float32), np.ones((idx.size, 12), np.float32), off, idx)
    assert np.array_equal(g[:, 0], pre["tiles"].astype(np.float32))
    # one block: the rows land on their Gaussians unchanged
    rows = np.random.default_rng(3).standard_normal((idx1.size, 12)).astype(np.float32)
    g1 = oracle.unpack_grads(np.zeros((w.n, 12), np.float32), rows, off1, idx1)
    assert np.array_equal(g1[idx1], rows)


def test_tile_blocks_of_rect_by_hand():
    # 4 tiles per row; blocks [0,2) [2,5) [5,8) [8,12)
    b = [0, 2, 5, 8, 12]
    assert list(oracle.tile_blocks_of_rect((1, 0, 3, 2), b, 4)) == [0, 1, 2]
    assert list(oracle.tile_blocks_of_rect((0, 2, 1, 3), b, 4)) == [3]
    assert list(oracle.tile_blocks_of_rect((3, 1, 4, 2), b, 4)) == [2]
    # a block lying in the gap between two rows of a rectangle is skipped
    b2 = [0, 3, 5, 12]          # block 1 = tiles 3, 4: (3, 0) and (0, 1)
    assert list(oracle.tile_blocks_of_rect((1, 0, 3, 3), b2, 4)) == [0, 2]


# --- densification -----------------------------------------------------------

def test_densify_stats_closed_form():
    g = np.zeros((4, 12), np.float32)
    g[1, :2] = (3.0, 4.0)
    g[2, :2] = (-5.0, 12.0)
    g[3, :2] = (1e-30, 0.0)       # u*u = 1e-60 underflows to 0 in fp32 (below the denormals)
    a, d = oracle.densify_stats(g, [1, 2, 3], np.zeros(4, np.float32), np.zeros(4, np.int32))
    assert list(a) == [0.0, 5.0, 13.0, 0.0] and list(d) == [0, 1, 1, 1]
    a, d = oracle.densify_stats(g, [1], a, d)
    assert a[1] == 10.0 and d[1] == 2


def _dens_params(n=6):
    p = np.zeros((59, n), np.float32)
    p[0] = np.arange(n)                     # means along x
    p[6] = 1.0                              # identity rotations
    p[10] = 2.0                             # opaque
    p[11:] = np.arange(48)[:, None] * 0.01 + np.arange(n)[None, :]
    return p


def test_densify_by_hand():
    """Six Gaussians: 0 kept (small gradient), 1 cloned (small), 2 split
    (large), 3 pruned (transparent), 4 never seen (denom 0), 5 split but
    transparent (pruned with its children)."""
    p = _dens_params()
    p[3:6, 1] = -5.0
    p[3:6, 2] = (0.0, -1.0, -2.0)           # largest log-scale 0 -> scale 1
    p[3:6, 5] = (0.5, 0.0, 0.0)
    p[10, 3] = -6.0
    p[10, 5] = -7.0
    accum = np.array([0.1, 5.0, 6.0, 9.0, 0.0, 9.0], np.float32)
    denom = np.array([1, 2, 2, 1, 0, 1], np.int32)
    m = np.arange(59 * 6, dtype=np.float32).reshape(59, 6)
    v = m + 1000
    z = np.zeros((2, 3, 6), np.float32)
    z[0, :, 2] = (1.0, 0.0, 0.0)
    z[1, :, 2] = (0.0, 0.0, -2.0)
    out, om, ov = oracle.densify(p, m, v, accum, denom, 1.0, -3.0, -4.0, z, np.log(1.6))
    # columns: kept 0, 1, 4; clone of 1; child 0 of 2; child 1 of 2
    assert out.shape == (59, 6)
    assert np.array_equal(out[:, 0:3], p[:, [0, 1, 4]])
    assert np.array_equal(out[:, 3], p[:, 1])
    c0, c1 = out[:, 4], out[:, 5]
    assert np.allclose(c0[0:3], (2.0 + 1.0, 0.0, 0.0)) and np.allclose(c1[0:3], (2.0, 0.0, -2.0 * np.exp(-2.0)))
    assert np.array_equal(c0[3:6].astype(np.float32), p[3:6, 2] - np.float32(np.log(1.6)))
    assert np.array_equal(c0[6:], p[6:, 2]) and np.array_equal(c1[6:], p[6:, 2])
    assert np.array_equal(om[:, 0:3], m[:, [0, 1, 4]]) and (om[:, 3:] == 0).all()
    assert np.array_equal(ov[:, 0:3], v[:, [0, 1, 4]]) and (ov[:, 3:] == 0).all()


def test_densify_split_rotates_the_offset():
    """A quarter turn about z maps the child's x offset onto y; the offset
    scales with exp(log-scale) per axis before the rotation."""
    p = _dens_params(1)
    p[3:6, 0] = (np.log(2.0), np.log(3.0), 0.0)
    p[6:10, 0] = (np.cos(np.pi / 4), 0.0, 0.0, np.sin(np.pi / 4))
    z = np.zeros((2, 3, 1), np.float32)
    z[0, 0, 0] = 1.0
    z[1, 1, 0] = 1.0
    out, _, _ = oracle.densify(p, p, p, np.array([1.0], np.float32), np.array([1], np.int32), 0.5, 0.0, -4.0, z,
                               np.log(1.6))
    assert np.allclose(out[0:3, 0], (0.0, 2.0, 0.0), atol=1e-6)     # x offset 2 -> +y
    assert np.allclose(out[0:3, 1], (-3.0, 0.0, 0.0), atol=1e-6)    # y offset 3 -> -x
    # nothing densifies below the threshold, nothing is pruned above it
    out, _, _ = oracle.densify(p, p, p, np.array([0.4], np.float32), np.array([1], np.int32), 0.5, 0.0, -4.0, z,
                               np.log(1.6))
    assert np.array_equal(out, p.astype(np.float64))


@pytest.mark.parametrize("case", ["tiny", "small_cut"])
def test_train_view_equals_the_stages(case):
    """The one-view step the CPU baseline times (projection once, no
    magnitudes) gives the render, loss and backward of the separate stages
    bit for bit."""
    w = synth.workload(0) if case == "tiny" else synth.cut_down(synth.workload(1), 200, 136, n=6000)
    cam, tgt = w.cameras[0], w.targets[0]
    L, img, grads = oracle.train_view(w.params, cam, tgt, w.w_l1, w.w_ssim)
    img2, _, _, _ = oracle.render(w.params, cam)
    L2, dL, _, _ = oracle.loss(img2, tgt, w.w_l1, w.w_ssim)
    _, _, g2, _ = oracle.backward(w.params, cam, dL, at_fp32=True)
    assert np.array_equal(img, img2) and L == L2
    assert np.array_equal(grads, g2)
