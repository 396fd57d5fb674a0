"""Seeded synthetic inputs for the 3D Gaussian Splatting training step.

This module builds the *inputs* of one training step -- Gaussian parameters,
pinhole cameras, target images and the optimiser hyper-parameters -- for five
workload configurations.  It holds none of the method's arithmetic: no
projection of Gaussians, no covariance, colour, compositing, loss or Adam.
Both the CPU oracle (``oracle/``) and the HIP path consume what it returns.

The workloads stand in for the scenes the pages measure on (a 360-degree
capture, a 1080p city scene, a 4K aerial scene with empty sky); none of those
datasets is used.  The configurations:

  0  tiny reference : 2,048 Gaussians, one 128x128 view, L1 loss
  1  small scene    : 100,000 Gaussians, one 1297x840 view
  2  mid scene      : 1,000,000 Gaussians, 1920x1080, batch of 4 ring views
  3  aerial 4K      : 3,000,000 Gaussians, one 3840x2160 tilted top-down view
  4  capacity       : 12,000,000 Gaussians, 1920x1080, 16 of 64 orbit views

Parameter layout (59 fp32 planes, plane-major ``[59][n]``), following the
primitive table of the Grendel-GS notes ("Background: what is 3D Gaussian
splatting", parameter table): planes 0-2 position xyz; 3-5 log-scale xyz;
6-9 quaternion (w, x, y, z), stored un-normalised; 10 opacity logit; 11-58
spherical-harmonic coefficients, plane 11 + 3k + c for basis k = 0..15 and
colour channel c = R, G, B.

Random draws use numpy's PCG64 (``numpy.random.default_rng(seed)``) with
``seed`` = the configuration index unless given, in the fixed order written
in each builder below.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

N_PARAMS = 59
TILE = 16

# Mean of the per-axis log-scale normal for the plane/sphere scenes and for
# the aerial scene.  Chosen (by bisection with the oracle's projection, see
# tests/golden/calibrate_log_scale.py) so that about 90% of the Gaussians
# visible in view 0 have a screen radius below 2% of the image width -- the
# observation the Grendel-GS notes report in "Sparse All-to-All
# communication".  tests/test_synth.py re-checks the statistic.
LOG_SCALE_MU_SCENE = -4.32
LOG_SCALE_MU_AERIAL = -4.73


@dataclass
class Camera:
    """Pinhole camera, world -> camera ``x_c = R x_w + t``.

    Camera axes: x right, y down, z forward.  Pixel (i, j) covers
    [i, i+1) x [j, j+1) in image coordinates and is sampled at its centre
    (i + 1/2, j + 1/2).  ``R`` is row-major 3x3.
    """
    width: int
    height: int
    fx: float
    fy: float
    cx: float
    cy: float
    R: np.ndarray          # (3, 3) float32
    t: np.ndarray          # (3,) float32
    campos: np.ndarray     # (3,) float32, camera centre in world
    near: float = 0.2


@dataclass
class Workload:
    config: int
    name: str
    params: np.ndarray                 # (59, n) float32
    cameras: list                      # list[Camera], one per view of the step
    targets: list                      # list[(3, H, W) float32]
    w_l1: float
    w_ssim: float
    lr: float
    beta1: float
    beta2: float
    eps: float
    meta: dict = field(default_factory=dict)

    @property
    def n(self) -> int:
        return self.params.shape[1]


# --------------------------------------------------------------------------
# cameras
# --------------------------------------------------------------------------

def _intrinsics(width: int, height: int, hfov_deg: float = 60.0):
    fx = (width / 2.0) / math.tan(math.radians(hfov_deg) / 2.0)
    return fx, fx, width / 2.0, height / 2.0


def look_camera(width, height, eye, forward, down) -> Camera:
    """Camera at ``eye`` with optical axis ``forward`` and image-down ``down``
    (both world vectors; ``down`` is orthogonalised against ``forward``)."""
    eye = np.asarray(eye, np.float64)
    f = np.asarray(forward, np.float64)
    f = f / np.linalg.norm(f)
    d = np.asarray(down, np.float64)
    d = d - f * np.dot(d, f)
    d = d / np.linalg.norm(d)
    r = np.cross(d, f)
    R = np.stack([r, d, f])           # rows: right, down, forward
    t = -R @ eye
    fx, fy, cx, cy = _intrinsics(width, height)
    return Camera(width, height, fx, fy, cx, cy,
                  R.astype(np.float32), t.astype(np.float32),
                  eye.astype(np.float32))


def ring_camera(width, height, theta, radius=4.0) -> Camera:
    """Camera on a horizontal ring of ``radius`` around the origin, looking at
    the origin; image-down is world +y.  theta = 0 puts it at (0, 0, -radius)
    looking along +z."""
    eye = np.array([radius * math.sin(theta), 0.0, -radius * math.cos(theta)])
    return look_camera(width, height, eye, -eye, (0.0, 1.0, 0.0))


def orbit_cameras(width, height, count, radius=4.0, max_elev_deg=35.0):
    """``count`` cameras on a band of the sphere of ``radius`` around the
    origin, all looking at the origin: azimuths step by the golden angle,
    elevations spread evenly in sine up to +-``max_elev_deg`` (a spiral
    that covers the band without repeats, like a capture orbit)."""
    golden = math.pi * (3.0 - math.sqrt(5.0))
    smax = math.sin(math.radians(max_elev_deg))
    cams = []
    for k in range(count):
        th = k * golden
        el = math.asin(smax * (2.0 * (k + 0.5) / count - 1.0)) if count > 1 else 0.0
        eye = np.array([radius * math.cos(el) * math.sin(th), -radius * math.sin(el),
                        -radius * math.cos(el) * math.cos(th)])
        cams.append(look_camera(width, height, eye, -eye, (0.0, 1.0, 0.0)))
    return cams


def random_visible_lists(rng, n, count):
    """``count`` ascending int32 index lists over [0, n) with the shapes
    visible sets take: an empty one, a full one, a single index, then
    random mixes of contiguous runs (a region in view: whole 32-index words
    set) and scattered indices (small, distant Gaussians), at densities
    from 0.1% to 90%."""
    out = [np.zeros(0, np.int32), np.arange(n, dtype=np.int32),
           np.array([n - 1] if n > 0 else [], np.int32)]
    while len(out) < count:
        dens = float(rng.choice([0.001, 0.01, 0.1, 0.3, 0.6, 0.9]))
        mask = rng.random(n) < dens * 0.5
        for _ in range(int(rng.integers(0, 6))):
            a = int(rng.integers(0, max(n, 1)))
            mask[a:a + int(rng.integers(1, max(2, int(dens * n))))] = True
        out.append(np.flatnonzero(mask).astype(np.int32))
    return out[:count]


# --------------------------------------------------------------------------
# targets
# --------------------------------------------------------------------------

def sinusoid_target(rng, width, height, n_waves=32):
    """Per channel: 0.5 + sum of ``n_waves`` random 2-D sinusoids over the
    normalised pixel-centre coordinates, clipped to [0, 1].  Amplitudes
    N(0, 0.1); directions uniform; frequencies U[0, 8] cycles per frame;
    phases U[0, 2 pi).  Draw order per channel: amplitudes, angles, freqs,
    phases."""
    xs = (np.arange(width, dtype=np.float64) + 0.5) / width
    ys = (np.arange(height, dtype=np.float64) + 0.5) / height
    out = np.empty((3, height, width), np.float32)
    for c in range(3):
        a = rng.normal(0.0, 0.1, n_waves)
        ang = rng.uniform(0.0, 2 * math.pi, n_waves)
        mag = rng.uniform(0.0, 8.0, n_waves)
        phi = rng.uniform(0.0, 2 * math.pi, n_waves)
        # sin(p + q) = sin p cos q + cos p sin q, with p over x and q over y
        px = 2 * math.pi * np.outer(mag * np.cos(ang), xs)             # (k, W)
        qy = 2 * math.pi * np.outer(mag * np.sin(ang), ys) + phi[:, None]  # (k, H)
        img = 0.5 + (a[:, None] * np.cos(qy)).T @ np.sin(px) + (a[:, None] * np.sin(qy)).T @ np.cos(px)
        out[c] = np.clip(img, 0.0, 1.0)
    return out


# --------------------------------------------------------------------------
# Gaussian attributes shared by all scenes
# --------------------------------------------------------------------------

def _fill_attributes(rng, params, log_mu, log_sigma, logit_sigma):
    """Draw order, each drawn plane-major: log-scales (3, n); quaternions
    (4, n), normalised per Gaussian; opacity logits (n); SH DC (3, n);
    SH rest (45, n) in plane order 14..58."""
    n = params.shape[1]
    params[3:6] = rng.normal(log_mu, log_sigma, (3, n))
    q = rng.normal(0.0, 1.0, (4, n))
    q /= np.sqrt((q * q).sum(axis=0, keepdims=True))
    params[6:10] = q
    params[10] = rng.normal(0.0, logit_sigma, n)
    # one plane per draw: the same stream as a single (k, n) draw, without
    # the large float64 temporary
    for k in range(11, 14):
        params[k] = rng.normal(0.0, 0.5, n)
    for k in range(14, 59):
        params[k] = rng.normal(0.0, 0.1, n)


def _plane_sphere_points(rng, n):
    """8 random planes + 4 random spheres in [-1, 1]^3, n // 12 points each
    (the remainder goes to the last primitive), then N(0, 0.01) jitter."""
    counts = [n // 12] * 12
    counts[-1] += n - sum(counts)
    pts = []
    for p in range(8):
        nrm = rng.normal(0.0, 1.0, 3)
        nrm /= np.linalg.norm(nrm)
        centre = rng.uniform(-0.6, 0.6, 3)
        half = rng.uniform(0.3, 0.8)
        a = np.eye(3)[np.argmin(np.abs(nrm))]
        e1 = np.cross(nrm, a)
        e1 /= np.linalg.norm(e1)
        e2 = np.cross(nrm, e1)
        uv = rng.uniform(-half, half, (counts[p], 2))
        pts.append(centre + uv[:, :1] * e1 + uv[:, 1:] * e2)
    for s in range(4):
        centre = rng.uniform(-0.5, 0.5, 3)
        rad = rng.uniform(0.15, 0.4)
        d = rng.normal(0.0, 1.0, (counts[8 + s], 3))
        d /= np.linalg.norm(d, axis=1, keepdims=True)
        pts.append(centre + rad * d)
    pts = np.concatenate(pts, axis=0)
    pts += rng.normal(0.0, 0.01, pts.shape)
    return pts


def _adam_for_batch(b):
    """Grendel-GS notes, "Hyper-parameter scaling rule": learning rate times
    sqrt(batch), betas raised to the batch size.  Base lr 1e-3, betas
    (0.9, 0.999), eps 1e-15."""
    return 1e-3 * math.sqrt(b), 0.9 ** b, 0.999 ** b, 1e-15


# --------------------------------------------------------------------------
# the five configurations
# --------------------------------------------------------------------------

def tiny(seed=0, n=2048, width=128, height=128) -> Workload:
    rng = np.random.default_rng(seed)
    p = np.empty((N_PARAMS, n), np.float32)
    p[0:3] = rng.uniform(-1.0, 1.0, (n, 3)).T
    _fill_attributes(rng, p, -3.0, 0.3, 1.0)
    cam = ring_camera(width, height, 0.0)
    target = rng.uniform(0.0, 1.0, (3, height, width)).astype(np.float32)
    lr, b1, b2, eps = _adam_for_batch(1)
    return Workload(0, "tiny", p, [cam], [target], 1.0, 0.0, lr, b1, b2, eps)


def plane_scene(config, n, width, height, thetas, seed, log_mu=LOG_SCALE_MU_SCENE,
                name="scene") -> Workload:
    rng = np.random.default_rng(seed)
    p = np.empty((N_PARAMS, n), np.float32)
    p[0:3] = _plane_sphere_points(rng, n).T
    _fill_attributes(rng, p, log_mu, 0.5, 1.5)
    cams = [ring_camera(width, height, th) for th in thetas]
    targets = [sinusoid_target(rng, width, height) for _ in thetas]
    lr, b1, b2, eps = _adam_for_batch(len(thetas))
    return Workload(config, name, p, cams, targets, 0.8, 0.2, lr, b1, b2, eps,
                    meta={"thetas": list(thetas), "log_mu": log_mu})


def small(seed=1) -> Workload:
    return plane_scene(1, 100_000, 1297, 840, [0.0], seed, name="small")


def mid(seed=2) -> Workload:
    return plane_scene(2, 1_000_000, 1920, 1080,
                       [2 * math.pi * k / 4 for k in range(4)], seed, name="mid")


def capacity(seed=4, n=12_000_000, width=1920, height=1080, views=16) -> Workload:
    """The capacity batch: 16 ring views out of 64 positions; ``views``
    keeps the first few, ``width`` / ``height`` shrink them (parity sizes)."""
    rng = np.random.default_rng(seed + 1000)
    js = np.sort(rng.choice(64, 16, replace=False))[:views]
    return plane_scene(4, n, width, height,
                       [2 * math.pi * int(j) / 64 for j in js], seed, name="capacity")


def aerial_camera(width=3840, height=2160, height_above=4.0, tilt_deg=30.0) -> Camera:
    """Camera ``height_above`` over the ground plane y = 0 (world up is -y),
    optical axis ``tilt_deg`` from nadir toward +z; the far ground is at the
    top of the image."""
    t = math.radians(tilt_deg)
    fwd = (0.0, math.cos(t), math.sin(t))
    down = (0.0, math.sin(t), -math.cos(t))
    return look_camera(width, height, (0.0, -height_above, 0.0), fwd, down)


def flight_cameras(width, height, count, seed=7, height_above=4.0, tilt_deg=30.0,
                   x_range=(-3.0, 3.0), z_range=(-2.5, 0.5), max_yaw_deg=25.0):
    """``count`` aerial cameras over the ground plane of the aerial scene,
    as a survey flight takes them: eyes ``height_above`` the plane at
    uniform random (x, z) in the ranges, each tilted ``tilt_deg`` from nadir
    and turned by a uniform random yaw of up to +-``max_yaw_deg`` from +z.
    Views near one another see overlapping parts of the ground; distant ones
    see disjoint parts."""
    rng = np.random.default_rng(seed)
    xs = rng.uniform(*x_range, count)
    zs = rng.uniform(*z_range, count)
    yaws = np.radians(rng.uniform(-max_yaw_deg, max_yaw_deg, count))
    t = math.radians(tilt_deg)
    cams = []
    for x, z, a in zip(xs, zs, yaws):
        h = (math.sin(a), 0.0, math.cos(a))          # heading on the ground
        fwd = (math.sin(t) * h[0], math.cos(t), math.sin(t) * h[2])
        down = (-math.cos(t) * h[0], math.sin(t), -math.cos(t) * h[2])
        cams.append(look_camera(width, height, (float(x), -height_above, float(z)), fwd, down))
    return cams


def _pixel_rays(cam: Camera, u, v):
    """World directions of rays through image points (u, v) (fp64)."""
    R = cam.R.astype(np.float64)
    xc = (u - cam.cx) / cam.fx
    yc = (v - cam.cy) / cam.fy
    dc = np.stack([xc, yc, np.ones_like(xc)], axis=1)
    return dc @ R            # rows of R are the camera axes in world


def aerial(seed=3, n=3_000_000, width=3840, height=2160,
           log_mu=LOG_SCALE_MU_AERIAL) -> Workload:
    """85% of the Gaussians on a noisy ground plane (height noise N(0, 0.02)),
    15% on the five visible faces of 64 random boxes (footprint U[0.05, 0.3]^2,
    height U[0.1, 1.0]).  No Gaussian centre lies in the top 20% of the rows:
    ground points are cast from image rows [0.2H + 64, H); box points whose
    centre falls on the sky side of the plane through the eye and image row
    0.2H + 8 are redrawn.  Log-scales N(log_mu, 0.8) per axis.

    Draw order: ground (u, v) pixels, ground height noise, box footprint
    rows/cols, box sizes, box heights, box face points (redraws appended),
    then the common attributes and the target.
    """
    rng = np.random.default_rng(seed)
    cam = aerial_camera(width, height)
    eye = cam.campos.astype(np.float64)
    n_ground = int(round(0.85 * n))
    n_box = n - n_ground
    p = np.empty((N_PARAMS, n), np.float32)

    # ground: ray-cast random image points in the non-sky rows onto y = 0
    u = rng.uniform(0.0, width, n_ground)
    v = rng.uniform(0.2 * height + 64.0, height, n_ground)
    d = _pixel_rays(cam, u, v)
    s = -eye[1] / d[:, 1]
    g = eye[None, :] + s[:, None] * d
    g[:, 1] = rng.normal(0.0, 0.02, n_ground)

    # sky half-space: points x with dot(x - eye, nsky) > 0 project above row
    # 0.2H + 8 (the plane holds the eye, the camera right axis and the ray
    # through that row)
    r_axis = cam.R[0].astype(np.float64)
    ray_sky = _pixel_rays(cam, np.array([cam.cx]), np.array([0.2 * height + 8.0]))[0]
    nsky = np.cross(ray_sky, r_axis)
    fwd = cam.R[2].astype(np.float64)
    if np.dot(nsky, _pixel_rays(cam, np.array([cam.cx]), np.array([0.0]))[0]) < 0:
        nsky = -nsky

    # boxes on the ground, footprints cast from rows [0.35H, H)
    nb = 64
    bu = rng.uniform(0.1 * width, 0.9 * width, nb)
    bv = rng.uniform(0.35 * height, height, nb)
    bd = _pixel_rays(cam, bu, bv)
    bc = eye[None, :] + (-eye[1] / bd[:, 1])[:, None] * bd
    size = rng.uniform(0.05, 0.3, (nb, 2))
    bh = rng.uniform(0.1, 1.0, nb)
    per = [n_box // nb] * nb
    per[-1] += n_box - sum(per)
    box_pts = []
    for b in range(nb):
        need = per[b]
        got = []
        while need > 0:
            face = rng.integers(0, 5, need)
            a = rng.uniform(-1.0, 1.0, (need, 2))
            hx, hz = size[b] / 2.0
            x = np.empty((need, 3))
            # face 0: top (y = -h); 1/2: x = -+hx; 3/4: z = -+hz
            y_side = -bh[b] * (a[:, 1] + 1.0) / 2.0
            top = face == 0
            x[top] = np.stack([a[top, 0] * hx, np.full(top.sum(), -bh[b]), a[top, 1] * hz], 1)
            for f, sx in ((1, -1.0), (2, 1.0)):
                m = face == f
                x[m] = np.stack([np.full(m.sum(), sx * hx), y_side[m], a[m, 0] * hz], 1)
            for f, sz in ((3, -1.0), (4, 1.0)):
                m = face == f
                x[m] = np.stack([a[m, 0] * hx, y_side[m], np.full(m.sum(), sz * hz)], 1)
            x += bc[b][None, :] * np.array([1.0, 0.0, 1.0])
            ok = (x - eye[None, :]) @ nsky <= 0.0
            ok &= (x - eye[None, :]) @ fwd > 0.5
            got.append(x[ok])
            need -= int(ok.sum())
        box_pts.append(np.concatenate(got, 0))
    # a ground point pushed onto the sky side by its height noise loses the noise
    g[(g - eye[None, :]) @ nsky > 0.0, 1] = 0.0
    pts = np.concatenate([g] + box_pts, axis=0)
    p[0:3] = pts.T
    _fill_attributes(rng, p, log_mu, 0.8, 1.5)
    target = sinusoid_target(rng, width, height)
    lr, b1, b2, eps = _adam_for_batch(1)
    return Workload(3, "aerial", p, [cam], [target], 0.8, 0.2, lr, b1, b2, eps,
                    meta={"log_mu": log_mu, "sky_rows": int(0.2 * height)})


BUILDERS = {0: tiny, 1: small, 2: mid, 3: aerial, 4: capacity}


def workload(config: int, **kw) -> Workload:
    """The seeded workload of configuration ``config`` (0..4)."""
    return BUILDERS[config](**kw)


def cut_down(w: Workload, width: int, height: int, n: int | None = None,
             views: int | None = None) -> Workload:
    """Same scene, fewer Gaussians (``n`` evenly strided ones) and/or a smaller image
    (intrinsics rescaled so the field of view stays 60 degrees horizontal).
    Used for parity sizes the oracle finishes in seconds."""
    if n is None or n >= w.n:
        params = w.params
    else:
        idx = np.linspace(0, w.n - 1, n).round().astype(np.int64)
        params = np.ascontiguousarray(w.params[:, idx])
    cams = []
    for c in w.cameras[: views or len(w.cameras)]:
        fx, fy, cx, cy = _intrinsics(width, height)
        cams.append(Camera(width, height, fx, fy, cx, cy, c.R, c.t, c.campos, c.near))
    rng = np.random.default_rng(12345 + w.config)
    if w.config == 0:
        targets = [rng.uniform(0.0, 1.0, (3, height, width)).astype(np.float32) for _ in cams]
    else:
        targets = [sinusoid_target(rng, width, height) for _ in cams]
    lr, b1, b2, eps = _adam_for_batch(len(cams))
    return Workload(w.config, w.name + f"_{width}x{height}", params, cams, targets,
                    w.w_l1, w.w_ssim, lr, b1, b2, eps, meta=dict(w.meta))
