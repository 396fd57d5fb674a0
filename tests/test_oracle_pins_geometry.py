"""Pins of the oracle's projection and compositing that the on-axis,
isotropic cases cannot see (CPU only).

* Off-axis mean and anisotropic, rotated covariance: the screen covariance
  is checked against a numerical Jacobian of the pinhole map (numpy central
  differences of world point -> pixel, so the camera rotation, the
  perspective division and the off-axis Jacobian terms enter without
  retyping the oracle's formula) applied to a world covariance built with
  scipy's quaternion rotation.  The oracle's rotation matrix and world
  covariance are checked against scipy and against the invariants any
  rotation and covariance have (orthonormal, det 1; symmetric, eigenvalues
  = the squared scales).
* The transmittance stop rule in closed form: a stack of opaque Gaussians
  covering a one-pixel image, where the rule "stop before the Gaussian whose
  compositing would drop T below 1e-4" decides `last`, `T_final` and the
  entries read.
* dC/dalpha_k by brute force: the product-rule derivative of every term of
  C = sum_i c_i alpha_i prod_{j<i} (1 - alpha_j), summed explicitly (no
  suffix recurrence), against the oracle's backward on a six-deep stack.

Geometry follows the Grendel-GS notes' training pipeline ("Gaussian
transform": 2D position, depth, cover radius, colour; per-pixel depth-sorted
alpha compositing).
"""
import math

import numpy as np
import pytest
from scipy.spatial.transform import Rotation

import oracle
import synth

Y0 = 0.5 / math.sqrt(math.pi)


def f64(x):
    """A camera scalar as the oracle sees it: stored in fp32."""
    return float(np.float32(x))


def pixel_of(cam, x):
    """Pinhole map world point -> pixel (u, v) in fp64 from the camera's
    fp32 fields: x_c = R x + t, u = fx x_c / z_c + cx, v = fy y_c / z_c + cy."""
    R = cam.R.astype(np.float64)
    t = cam.t.astype(np.float64)
    c = R @ np.asarray(x, np.float64) + t
    return np.array([f64(cam.fx) * c[0] / c[2] + f64(cam.cx), f64(cam.fy) * c[1] / c[2] + f64(cam.cy)])


def jacobian_fd(cam, x, h=1e-5):
    """2x3 Jacobian of pixel_of at x by central differences."""
    J = np.empty((2, 3))
    for k in range(3):
        e = np.zeros(3)
        e[k] = h
        J[:, k] = (pixel_of(cam, x + e) - pixel_of(cam, x - e)) / (2 * h)
    return J


def one_gaussian(pos, log_scales, quat_wxyz, logit=1.0):
    p = np.zeros((59, 1), np.float32)
    p[0:3, 0] = pos
    p[3:6, 0] = log_scales
    p[6:10, 0] = quat_wxyz
    p[10, 0] = logit
    p[11:14, 0] = (0.4, -0.2, 0.1)
    return p


def screen_cov_expected(cam, p):
    """J (R_q S^2 R_q^T) J^T with J the numerical Jacobian of the pinhole
    map at the mean and R_q from scipy (scalar-last quaternion)."""
    x = p[0:3, 0].astype(np.float64)
    s = np.exp(p[3:6, 0].astype(np.float64))
    w, qx, qy, qz = p[6:10, 0].astype(np.float64)
    Rq = Rotation.from_quat([qx, qy, qz, w]).as_matrix()
    Sig = Rq @ np.diag(s * s) @ Rq.T
    J = jacobian_fd(cam, x)
    return J @ Sig @ J.T, Rq, Sig


def test_off_axis_anisotropic_axis_aligned_gaussian():
    """R = I (camera and quaternion), scales (0.06, 0.02, 0.10), mean off the
    axis: u = fx t_x / t_z + cx, v = fy t_y / t_z + cy, and
    Sigma_2 = J diag(s^2) J^T + 0.3 I with the off-axis Jacobian."""
    cam = synth.ring_camera(128, 96, 0.0)
    pos = (0.35, -0.25, 0.6)
    p = one_gaussian(pos, np.log([0.06, 0.02, 0.10]), (1.0, 0.0, 0.0, 0.0))
    x = p[0:3, 0].astype(np.float64)
    tz = x[2] + 4.0
    u = f64(cam.fx) * x[0] / tz + f64(cam.cx)
    v = f64(cam.fy) * x[1] / tz + f64(cam.cy)
    cov, _, _ = screen_cov_expected(cam, p)
    # off-axis: the Jacobian's third column is non-zero, so the z scale leaks in
    assert abs(cov[0, 1]) > 1e-3 * cov[0, 0]
    exp_cov = cov + 0.3 * np.eye(2)
    pre64 = oracle.preprocess_f64(p.astype(np.float64), cam)
    assert np.allclose(pre64["mean2d"][0], [u, v], rtol=1e-13, atol=1e-12)
    assert pre64["depth"][0] == pytest.approx(tz, rel=1e-15)
    a, b, c = pre64["cov2d"][0]
    assert np.allclose([a, b, c], [exp_cov[0, 0], exp_cov[0, 1], exp_cov[1, 1]], rtol=1e-8, atol=1e-10)
    inv = np.linalg.inv(exp_cov)
    assert np.allclose(pre64["conic"][0], [inv[0, 0], inv[0, 1], inv[1, 1]], rtol=1e-8)
    # the fp32 canonical run, its radius and rectangle from the eigenvalue
    pre = oracle.preprocess(p, cam)
    assert pre["visible"][0]
    assert np.allclose(pre["mean2d"][0], [u, v], rtol=1e-6)
    assert np.allclose(pre["cov2d"][0], [exp_cov[0, 0], exp_cov[0, 1], exp_cov[1, 1]], rtol=2e-5)
    lam = np.linalg.eigvalsh(exp_cov).max()
    r = math.ceil(3 * math.sqrt(lam))
    assert pre["radius"][0] == r
    TX, TY = oracle.tiles_of(cam)
    clamp = lambda q, hi: min(max(q, 0), hi)
    rect = [clamp(math.floor((u - r) / 16), TX), clamp(math.floor((v - r) / 16), TY),
            clamp(math.floor((u + r) / 16) + 1, TX), clamp(math.floor((v + r) / 16) + 1, TY)]
    assert list(pre["rect"][0]) == rect
    assert pre["tiles"][0] == (rect[2] - rect[0]) * (rect[3] - rect[1])


@pytest.mark.parametrize("cam_kind", ["ring", "orbit"])
def test_rotated_gaussian_against_scipy_rotation(cam_kind):
    """A rotated, anisotropic Gaussian (un-normalised quaternion) seen by a
    rotated camera: the oracle's R_q equals scipy's rotation of the
    normalised quaternion (orthonormal, det 1, the same for -q); Sigma is
    symmetric PSD with the squared scales as eigenvalues and equals
    R_q S^2 R_q^T; Sigma_2 equals J Sigma J^T (+ 0.3 I) with the numerical
    Jacobian of the whole world -> pixel map, so the camera rotation and
    the off-axis terms are in it."""
    cam = synth.ring_camera(160, 120, 0.7) if cam_kind == "ring" else synth.orbit_cameras(160, 120, 9)[2]
    q = 1.7 * np.array([0.8, 0.3, -0.4, 0.2]) / np.linalg.norm([0.8, 0.3, -0.4, 0.2])
    p = one_gaussian((0.2, 0.15, -0.3), np.log([0.09, 0.03, 0.015]), q)
    cov, Rq_ref, Sig_ref = screen_cov_expected(cam, p)
    p64 = p.astype(np.float64)
    Rq, Sig, cov_raw = oracle.projection_internals_f64(p64, cam)
    Rq, Sig = Rq[0], Sig[0]
    assert np.allclose(Rq, Rq_ref, atol=1e-14)
    assert np.allclose(Rq @ Rq.T, np.eye(3), atol=1e-14) and np.linalg.det(Rq) == pytest.approx(1.0, abs=1e-14)
    Rneg, _, _ = oracle.projection_internals_f64(-p64, cam)
    assert np.allclose(Rneg[0], Rq, atol=1e-15)
    assert np.array_equal(Sig, Sig.T)
    s2 = np.exp(2 * p64[3:6, 0])
    assert np.allclose(np.sort(np.linalg.eigvalsh(Sig)), np.sort(s2), rtol=1e-12)
    assert np.allclose(Sig, Sig_ref, rtol=1e-12, atol=1e-17)
    assert np.allclose(cov_raw[0], [cov[0, 0], cov[0, 1], cov[1, 1]], rtol=1e-8, atol=1e-12)
    pre64 = oracle.preprocess_f64(p64, cam)
    assert np.allclose(pre64["mean2d"][0], pixel_of(cam, p64[0:3, 0]), rtol=1e-13)
    pre = oracle.preprocess(p, cam)
    assert pre["visible"][0]
    exp_cov = cov + 0.3 * np.eye(2)
    assert np.allclose(pre["cov2d"][0], [exp_cov[0, 0], exp_cov[0, 1], exp_cov[1, 1]], rtol=2e-5, atol=1e-6)


# ---------------------------------------------------------------------------
# one-pixel image: a stack of Gaussians on the optical axis
# ---------------------------------------------------------------------------

def stack(depths, logits, dcs):
    """Gaussians on the axis of the 1x1 camera at (0, 0, -4): each projects
    exactly onto the pixel centre (u = cx = 1/2), so power = 0 and
    alpha = min(0.99, sigmoid(logit)); unit scales put the one tile in
    every rectangle; colour = Y0 dc + 1/2 (DC band only)."""
    n = len(depths)
    p = np.zeros((59, n), np.float32)
    p[2] = depths
    p[6] = 1.0
    p[10] = logits
    p[11:14] = np.asarray(dcs, np.float32).T
    return p


def closed_form(p, order):
    """alpha, colours of the Gaussians in depth order, in fp64."""
    logit = p[10, order].astype(np.float64)
    alpha = np.minimum(0.99, 1.0 / (1.0 + np.exp(-logit)))
    col = Y0 * p[11:14, order].astype(np.float64).T + 0.5
    return alpha, col


def test_stop_rule_closed_form():
    """Six Gaussians of alpha 0.95 in scrambled index order: T runs 1, 0.05,
    0.0025, 1.25e-4; the fourth would take it to 6.25e-6 < 1e-4, so the
    pixel stops before it: three composited (last = 3), four entries read,
    T_final = 0.05^3, colour = sum of c_k 0.95 T_k over the first three in
    depth order."""
    cam = synth.ring_camera(1, 1, 0.0)
    depths = [0.9, 0.1, 0.5, 0.3, 0.7, 1.1]
    logit = math.log(0.95 / 0.05)
    dcs = [(0.5 * k - 1.0, 0.3 * k - 0.6, 1.0 - 0.25 * k) for k in range(6)]
    p = stack(depths, [logit] * 6, dcs)
    order = np.argsort(depths)
    alpha, col = closed_form(p, order)
    img, Tf, last, proc = oracle.render(p, cam)
    T = 1.0
    C = np.zeros(3)
    for k in range(3):
        C += col[k] * alpha[k] * T
        T *= 1 - alpha[k]
    assert T * (1 - alpha[3]) < 1e-4 < T          # far from the threshold either way
    assert int(last[0, 0]) == 3 and int(proc[0]) == 4
    assert int(oracle.composited_counts(p, cam)[0, 0]) == 3
    assert Tf[0, 0] == pytest.approx(T, rel=1e-5)
    assert np.allclose(img[:, 0, 0], C, rtol=1e-6, atol=1e-7)


def test_stop_rule_with_clamp_and_skip():
    """Alpha clamped at 0.99, a skipped Gaussian (alpha < 1/255) between two
    composited ones, then a stop: depth order 0.99 (T -> 0.01), skip,
    0.5 (T -> 0.005), 0.99 would take T to 5e-5: last = 3 (the position of
    the 0.5 one), four read, colour = 0.99 c0 + 0.5 * 0.01 c2."""
    cam = synth.ring_camera(1, 1, 0.0)
    p = stack([0.1, 0.2, 0.3, 0.4], [10.0, -7.0, 0.0, 10.0],
              [(1.0, 0.0, -1.0), (1.5, 1.5, 1.5), (-0.5, 0.8, 0.2), (0.3, 0.3, 0.3)])
    alpha, col = closed_form(p, np.arange(4))
    assert alpha[0] == 0.99 and alpha[1] < 1 / 255
    img, Tf, last, proc = oracle.render(p, cam)
    assert int(last[0, 0]) == 3 and int(proc[0]) == 4
    assert int(oracle.composited_counts(p, cam)[0, 0]) == 2      # the skipped one is not counted
    assert Tf[0, 0] == pytest.approx(0.01 * 0.5, rel=1e-5)
    assert np.allclose(img[:, 0, 0], 0.99 * col[0] + 0.5 * 0.01 * col[2], rtol=1e-6)


def brute_dC_dalpha(alpha, col):
    """d C_c / d alpha_k of C_c = sum_i col[i, c] alpha_i prod_{j<i}
    (1 - alpha_j), term by term by the product rule."""
    K = alpha.size
    out = np.zeros((K, 3))
    for k in range(K):
        for i in range(K):
            if i < k:
                continue
            if i == k:
                out[k] += col[i] * np.prod(1 - alpha[:i])
            else:
                others = [1 - alpha[j] for j in range(i) if j != k]
                out[k] += col[i] * alpha[i] * (-1.0) * np.prod(others)
    return out


def test_dC_dalpha_brute_force():
    """Six stacked Gaussians (no stop, no clamp) on a one-pixel view, image
    gradient G: the oracle's dL/d(opacity) equals G . dC/dalpha_k by brute
    force (alpha = opacity at power 0), dL/d(logit) that times o (1 - o),
    dL/d(rgb_k) = alpha_k T_k G and dL/d(DC_k) = Y0 alpha_k T_k G."""
    cam = synth.ring_camera(1, 1, 0.0)
    ops = np.array([0.3, 0.55, 0.2, 0.45, 0.6, 0.35])
    depths = [0.6, 0.2, 1.0, 0.4, 0.8, 0.0]
    rng = np.random.default_rng(12)
    dcs = rng.uniform(-1.0, 1.0, size=(6, 3))
    p = stack(depths, np.log(ops / (1 - ops)), dcs)
    order = np.argsort(depths)
    alpha, col = closed_form(p, order)
    G = np.array([0.7, -1.3, 0.4]).reshape(3, 1, 1)
    g2d, _, grads, _ = oracle.backward(p, cam, G)
    dC = brute_dC_dalpha(alpha, col)
    # the brute-force derivative itself against central differences of C
    for k in range(6):
        h = 1e-7
        ap, am = alpha.copy(), alpha.copy()
        ap[k] += h
        am[k] -= h
        Cp = sum(col[i] * ap[i] * np.prod(1 - ap[:i]) for i in range(6))
        Cm = sum(col[i] * am[i] * np.prod(1 - am[:i]) for i in range(6))
        assert np.allclose((Cp - Cm) / (2 * h), dC[k], rtol=1e-6, atol=1e-9)
    T = np.concatenate([[1.0], np.cumprod(1 - alpha)[:-1]])
    Gv = G.ravel()
    for r, i in enumerate(order):
        assert g2d[i, 5] == pytest.approx(float(dC[r] @ Gv), rel=1e-11, abs=1e-15)
        o = alpha[r]
        assert grads[10, i] == pytest.approx(float(dC[r] @ Gv) * o * (1 - o), rel=1e-11, abs=1e-15)
        assert np.allclose(g2d[i, 6:9], alpha[r] * T[r] * Gv, rtol=1e-12)
        assert np.allclose(grads[11:14, i], Y0 * alpha[r] * T[r] * Gv, rtol=1e-12)
