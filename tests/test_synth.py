"""Properties of the seeded synthetic workloads (CPU)."""
import math

import numpy as np

import oracle
import synth


def test_tiny_workload_shape_and_determinism():
    a = synth.workload(0)
    b = synth.workload(0)
    assert a.params.shape == (59, 2048) and a.params.dtype == np.float32
    assert np.array_equal(a.params, b.params)
    assert np.array_equal(a.targets[0], b.targets[0])
    assert a.targets[0].shape == (3, 128, 128)
    assert np.all(np.abs(a.params[0:3]) <= 1.0)
    q = a.params[6:10].astype(np.float64)
    assert np.allclose((q * q).sum(0), 1.0, atol=1e-6)
    cam = a.cameras[0]
    assert np.array_equal(cam.R, np.eye(3, dtype=np.float32))
    assert np.allclose(cam.t, [0, 0, 4]) and np.allclose(cam.campos, [0, 0, -4])
    assert math.isclose(cam.fx, 64 / math.tan(math.radians(30)))
    assert (a.w_l1, a.w_ssim, a.lr, a.beta1, a.beta2, a.eps) == (1.0, 0.0, 1e-3, 0.9, 0.999, 1e-15)


def test_small_scene_radius_statistic():
    # Grendel-GS notes, "Sparse All-to-All communication": ~90% of the
    # Gaussians cover a screen radius below 2% of the image width
    w = synth.workload(1)
    assert w.params.shape == (59, 100_000)
    cam = w.cameras[0]
    assert (cam.width, cam.height) == (1297, 840)
    pre = oracle.preprocess(w.params, cam)
    r = pre["radius"][pre["visible"]]
    assert abs(np.mean(r < 0.02 * cam.width) - 0.90) < 0.015
    assert np.all(w.targets[0] >= 0) and np.all(w.targets[0] <= 1)


def test_batch_scaling_rule():
    # Grendel-GS notes, "Hyper-parameter scaling rule": lr * sqrt(b), beta^b
    lr, b1, b2, eps = synth._adam_for_batch(4)
    assert math.isclose(lr, 2e-3) and math.isclose(b1, 0.6561) and math.isclose(b2, 0.999 ** 4)
    lr, b1, b2, eps = synth._adam_for_batch(16)
    assert math.isclose(lr, 4e-3) and math.isclose(b1, 0.9 ** 16) and math.isclose(b2, 0.999 ** 16)


def test_ring_cameras_look_at_origin():
    for k in range(4):
        cam = synth.ring_camera(1920, 1080, 2 * math.pi * k / 4)
        R = cam.R.astype(np.float64)
        assert np.allclose(R @ R.T, np.eye(3), atol=1e-6)
        assert np.isclose(np.linalg.det(R), 1.0, atol=1e-6)
        # the origin projects to the image centre, 4 units ahead
        tc = cam.t.astype(np.float64)
        assert np.allclose(tc, [0, 0, 4], atol=1e-5)


def test_aerial_sky_rows_empty():
    w = synth.aerial(n=60_000)
    cam = w.cameras[0]
    pre = oracle.preprocess(w.params, cam)
    v = pre["mean2d"][:, 1]
    ok = pre["depth"] > 0.2
    assert ok.mean() > 0.999
    assert np.all(v[ok] >= 0.2 * cam.height)
    # buildings: 15% of the Gaussians off the ground plane
    assert np.mean(np.abs(w.params[1]) > 0.08) > 0.08
