"""CPU oracle of the 3D Gaussian Splatting training step (numpy front end).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by
the CPU-baseline leg of ``bench.py``; never by the product path.  The
arithmetic lives in ``gs_oracle.cpp`` (plain C++17, built with g++ by
``build()``); this module only marshals numpy arrays.

Every function returns fresh numpy arrays.  Per-Gaussian outputs are
indexed by Gaussian; images are ``[3][H][W]``; parameter planes are
``[59][n]``.
"""

from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gs_oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")
TILE = 16

# The oracle's arithmetic contract: no FMA contraction, no fast-math, IEEE
# division/sqrt, no flush-to-zero (x86-64 SSE keeps subnormals by default).
CXXFLAGS = ["-O2", "-std=c++17", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
            "-fPIC", "-shared", "-Wall"]


def build(force: bool = True) -> str:
    """Compile ``liboracle.so`` with g++ (a few seconds)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["g++", *CXXFLAGS, "-o", tmp, _SRC], check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Cam(C.Structure):
    _fields_ = [("width", C.c_int32), ("height", C.c_int32),
                ("fx", C.c_float), ("fy", C.c_float), ("cx", C.c_float), ("cy", C.c_float),
                ("R", C.c_float * 9), ("t", C.c_float * 3), ("campos", C.c_float * 3),
                ("near_z", C.c_float)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = C.CDLL(_LIB)
        P = C.c_void_p
        i64, i32, f64 = C.c_int64, C.c_int, C.c_double
        L.or_pexp.restype = C.c_float
        L.or_pexp.argtypes = [C.c_float]
        L.or_aexp.restype = C.c_float
        L.or_aexp.argtypes = [C.c_float]
        L.or_num_threads.restype = C.c_int
        L.or_set_threads.argtypes = [C.c_int]
        L.or_sh_basis_f64.argtypes = [P, i64, P]
        L.or_sh_basis_f32.argtypes = [P, i64, P]
        L.or_preprocess.argtypes = [P, i64, i64, P] + [P] * 11
        L.or_preprocess_f64.argtypes = [P, i64, i64, P] + [P] * 6
        L.or_projection_internals_f64.argtypes = [P, i64, i64, P, P, P, P]
        L.or_bin.restype = i64
        L.or_bin.argtypes = [P, i64, i64, P, P, P, i64, P]
        L.or_render.argtypes = [P, i64, i64, P, P, P, P, P]
        L.or_render_brute.argtypes = [P, i64, i64, P, P, P, P]
        L.or_composited_counts.argtypes = [P, i64, i64, P, P]
        L.or_composite_pixels.argtypes = [P, i64, i64, P, P, P, P, P, i64, P, P, P]
        L.or_loss.restype = f64
        L.or_loss.argtypes = [P, P, i32, i32, f64, f64, P, P, P]
        L.or_render_frozen_f64.argtypes = [P, P, i64, i64, P, P]
        L.or_loss_frozen_f64.restype = f64
        L.or_loss_frozen_f64.argtypes = [P, P, P, i32, i32, f64, f64]
        L.or_backward.argtypes = [P, i64, i64, P, P, P, P, P, P, P, i32]
        L.or_train_view.restype = f64
        L.or_train_view.argtypes = [P, i64, i64, P, P, f64, f64, P, P]
        L.or_project_backward.argtypes = [P, i64, i64, P, P, P]
        L.or_project_outputs_f64.argtypes = [P, P, i64, i64, P, P]
        L.or_adam.argtypes = [P, P, P, P, i64, P, i64, f64, f64, f64, f64, f64, f64]
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(C.c_void_p)


def cam_struct(cam) -> _Cam:
    """ctypes camera from a ``synth.Camera`` (or anything with its fields)."""
    c = _Cam()
    c.width, c.height = int(cam.width), int(cam.height)
    c.fx, c.fy, c.cx, c.cy = float(cam.fx), float(cam.fy), float(cam.cx), float(cam.cy)
    R = np.asarray(cam.R, np.float32).reshape(9)
    for k in range(9):
        c.R[k] = float(R[k])
    for k in range(3):
        c.t[k] = float(np.float32(cam.t[k]))
        c.campos[k] = float(np.float32(cam.campos[k]))
    c.near_z = float(cam.near)
    return c


def tiles_of(cam):
    return (cam.width + TILE - 1) // TILE, (cam.height + TILE - 1) // TILE


def _params(params):
    p = np.ascontiguousarray(params, np.float32)
    assert p.ndim == 2 and p.shape[0] == 59
    return p


def set_threads(n: int):
    lib().or_set_threads(int(n))


def num_threads() -> int:
    return lib().or_num_threads()


def pexp(x):
    f = lib().or_pexp
    return np.array([f(float(v)) for v in np.asarray(x, np.float32).ravel()], np.float32)


def aexp(x):
    """The compositing weight's exponential (x in [-5.6, 0])."""
    f = lib().or_aexp
    return np.array([f(float(v)) for v in np.asarray(x, np.float32).ravel()], np.float32)


def sh_basis(dirs, dtype=np.float64):
    d = np.ascontiguousarray(dirs, dtype).reshape(-1, 3)
    Y = np.empty((d.shape[0], 16), dtype)
    fn = lib().or_sh_basis_f64 if dtype == np.float64 else lib().or_sh_basis_f32
    fn(_p(d), d.shape[0], _p(Y))
    return Y


def preprocess(params, cam):
    """fp32 canonical projection: dict of per-Gaussian arrays."""
    p = _params(params)
    n = p.shape[1]
    out = dict(mean2d=np.empty((n, 2), np.float32), depth=np.empty(n, np.float32),
               cov2d=np.empty((n, 3), np.float32), conic=np.empty((n, 3), np.float32),
               opacity=np.empty(n, np.float32), rgb=np.empty((n, 3), np.float32),
               rgb_pos=np.empty((n, 3), np.uint8), radius=np.empty(n, np.int32),
               rect=np.empty((n, 4), np.int32), tiles=np.empty(n, np.uint32),
               visible=np.empty(n, np.uint8))
    c = cam_struct(cam)
    lib().or_preprocess(_p(p), n, n, C.byref(c), *[_p(out[k]) for k in (
        "mean2d", "depth", "cov2d", "conic", "opacity", "rgb", "rgb_pos", "radius", "rect",
        "tiles", "visible")])
    out["visible"] = out["visible"].astype(bool)
    out["rgb_pos"] = out["rgb_pos"].astype(bool)
    return out


def preprocess_f64(params64, cam):
    p = np.ascontiguousarray(params64, np.float64)
    n = p.shape[1]
    out = dict(mean2d=np.empty((n, 2)), depth=np.empty(n), cov2d=np.empty((n, 3)),
               conic=np.empty((n, 3)), opacity=np.empty(n), rgb=np.empty((n, 3)))
    c = cam_struct(cam)
    lib().or_preprocess_f64(_p(p), n, n, C.byref(c), *[_p(out[k]) for k in (
        "mean2d", "depth", "cov2d", "conic", "opacity", "rgb")])
    return out


def projection_internals_f64(params64, cam):
    """fp64 intermediates of the projection: the normalised quaternion's
    rotation R_q [n][3][3], the world covariance Sigma [n][3][3] and the
    screen covariance before the 0.3 dilation [n][3] (a, b, c)."""
    p = np.ascontiguousarray(params64, np.float64)
    n = p.shape[1]
    Rq = np.empty((n, 3, 3))
    Sig = np.empty((n, 3, 3))
    cov = np.empty((n, 3))
    c = cam_struct(cam)
    lib().or_projection_internals_f64(_p(p), n, n, C.byref(c), _p(Rq), _p(Sig), _p(cov))
    return Rq, Sig, cov


def visible_list(params, cam):
    """Ascending int32 indices of the Gaussians visible in the view."""
    return np.flatnonzero(preprocess(params, cam)["visible"]).astype(np.int32)


def bin_sort(params, cam):
    """Sorted (key, value) pairs and tile ranges: keys (tile << 32 | depth
    bits) uint64 [M], values int32 [M], ranges uint32 [T][2]."""
    p = _params(params)
    n = p.shape[1]
    c = cam_struct(cam)
    M = lib().or_bin(_p(p), n, n, C.byref(c), None, None, 0, None)
    TX, TY = tiles_of(cam)
    keys = np.empty(max(M, 1), np.uint64)
    vals = np.empty(max(M, 1), np.int32)
    ranges = np.empty((TX * TY, 2), np.uint32)
    lib().or_bin(_p(p), n, n, C.byref(c), _p(keys), _p(vals), max(M, 1), _p(ranges))
    return keys[:M], vals[:M], ranges


def render(params, cam):
    """fp32 canonical tiled render: image [3][H][W], T_final [H][W],
    last [H][W] uint32, tile_processed [T] uint32."""
    p = _params(params)
    n = p.shape[1]
    W, H = cam.width, cam.height
    TX, TY = tiles_of(cam)
    img = np.empty((3, H, W), np.float32)
    Tf = np.empty((H, W), np.float32)
    last = np.empty((H, W), np.uint32)
    proc = np.empty(TX * TY, np.uint32)
    c = cam_struct(cam)
    lib().or_render(_p(p), n, n, C.byref(c), _p(img), _p(Tf), _p(last), _p(proc))
    return img, Tf, last, proc


def composited_counts(params, cam):
    """Per pixel the number of Gaussians composited, [H][W] uint32."""
    p = _params(params)
    n = p.shape[1]
    out = np.empty((cam.height, cam.width), np.uint32)
    c = cam_struct(cam)
    lib().or_composited_counts(_p(p), n, n, C.byref(c), _p(out))
    return out


def render_brute(params, cam):
    p = _params(params)
    n = p.shape[1]
    W, H = cam.width, cam.height
    img = np.empty((3, H, W), np.float32)
    Tf = np.empty((H, W), np.float32)
    last = np.empty((H, W), np.uint32)
    c = cam_struct(cam)
    lib().or_render_brute(_p(p), n, n, C.byref(c), _p(img), _p(Tf), _p(last))
    return img, Tf, last


def composite_pixels(params, cam, vals, ranges, px, py):
    """Pixels (px[k], py[k]) composited with the fp32 rule of ``render``
    against the per-tile lists given by (vals, ranges [T][2]): rgb [k][3],
    T_final [k], last [k]."""
    p = _params(params)
    n = p.shape[1]
    v = np.ascontiguousarray(vals, np.int32)
    r = np.ascontiguousarray(ranges, np.uint32).reshape(-1)
    x = np.ascontiguousarray(px, np.int32)
    y = np.ascontiguousarray(py, np.int32)
    k = x.shape[0]
    rgb = np.empty((k, 3), np.float32)
    Tf = np.empty(k, np.float32)
    last = np.empty(k, np.uint32)
    c = cam_struct(cam)
    lib().or_composite_pixels(_p(p), n, n, C.byref(c), _p(v), _p(r), _p(x), _p(y), k, _p(rgb), _p(Tf), _p(last))
    return rgb, Tf, last


def loss(image, target, w_l1, w_ssim):
    """fp64 loss of an fp32 image: (L, dL/dI [3][H][W] f64, mean L1, mean SSIM)."""
    img = np.ascontiguousarray(image, np.float32)
    tgt = np.ascontiguousarray(target, np.float32)
    _, H, W = img.shape
    dL = np.empty((3, H, W), np.float64)
    l1 = C.c_double()
    ss = C.c_double()
    L = lib().or_loss(_p(img), _p(tgt), W, H, float(w_l1), float(w_ssim), _p(dL),
                      C.byref(l1), C.byref(ss))
    return L, dL, l1.value, ss.value


def render_frozen_f64(base_params, params64, cam):
    b = _params(base_params)
    p = np.ascontiguousarray(params64, np.float64)
    n = b.shape[1]
    img = np.empty((3, cam.height, cam.width), np.float64)
    c = cam_struct(cam)
    lib().or_render_frozen_f64(_p(b), _p(p), n, n, C.byref(c), _p(img))
    return img


def loss_frozen_f64(image64, image32, target, w_l1, w_ssim):
    i64 = np.ascontiguousarray(image64, np.float64)
    i32 = np.ascontiguousarray(image32, np.float32)
    t = np.ascontiguousarray(target, np.float32)
    _, H, W = t.shape
    return lib().or_loss_frozen_f64(_p(i64), _p(i32), _p(t), W, H, float(w_l1), float(w_ssim))


def backward(params, cam, dL_dimage, grads=None, mags=None, at_fp32=False, gmag=None):
    """fp64 backward of one view.  Returns (g2d [n][9], m2d [n][9],
    grads [59][n], mags [59][n]); grads/mags accumulate into the given
    arrays when passed (batch accumulation).  With ``at_fp32`` the chain
    rule is evaluated at the fp32 forward's values (screen-space mean,
    conic, opacity, colour, and the projection's intermediates) instead of
    their fp64 recomputation.
    ``gmag`` ([3][H][W], optional) replaces |dL/dI| in the magnitudes."""
    p = _params(params)
    n = p.shape[1]
    dL = np.ascontiguousarray(dL_dimage, np.float64)
    gm = None if gmag is None else np.ascontiguousarray(gmag, np.float64)
    g2d = np.empty((n, 9))
    m2d = np.empty((n, 9))
    if grads is None:
        grads = np.zeros((59, n))
    if mags is None:
        mags = np.zeros((59, n))
    assert grads.dtype == np.float64 and grads.flags.c_contiguous and grads.shape == (59, n)
    assert mags.dtype == np.float64 and mags.flags.c_contiguous and mags.shape == (59, n)
    c = cam_struct(cam)
    lib().or_backward(_p(p), n, n, C.byref(c), _p(dL), None if gm is None else _p(gm), _p(g2d), _p(m2d),
                      _p(grads), _p(mags), int(at_fp32))
    return g2d, m2d, grads, mags


def train_view(params, cam, target, w_l1, w_ssim, grads=None):
    """One view of the step projecting once and without magnitudes (the
    plain step the CPU baseline times): returns (loss, image [3][H][W] f32,
    grads [59][n] f64 with this view's gradients added)."""
    p = _params(params)
    n = p.shape[1]
    t = np.ascontiguousarray(target, np.float32)
    img = np.empty((3, cam.height, cam.width), np.float32)
    if grads is None:
        grads = np.zeros((59, n))
    assert grads.dtype == np.float64 and grads.flags.c_contiguous and grads.shape == (59, n)
    c = cam_struct(cam)
    L = lib().or_train_view(_p(p), n, n, C.byref(c), _p(t), float(w_l1), float(w_ssim), _p(img), _p(grads))
    return L, img, grads


def project_backward(params, cam, g2d):
    p = _params(params)
    n = p.shape[1]
    g = np.ascontiguousarray(g2d, np.float64)
    out = np.zeros((59, n))
    c = cam_struct(cam)
    lib().or_project_backward(_p(p), n, n, C.byref(c), _p(g), _p(out))
    return out


def project_outputs_f64(base_params, params64, cam):
    b = _params(base_params)
    p = np.ascontiguousarray(params64, np.float64)
    n = b.shape[1]
    out = np.empty((n, 9))
    c = cam_struct(cam)
    lib().or_project_outputs_f64(_p(b), _p(p), n, n, C.byref(c), _p(out))
    return out


def adam(params, grads, m, v, rows, lr, b1, b2, eps, step=1):
    """fp64 Adam over the listed rows; returns new (params, m, v).  The
    bias corrections 1 - beta^step are formed here in fp64."""
    p = np.array(params, np.float64, order="C")
    g = np.ascontiguousarray(grads, np.float64)
    mm = np.array(m, np.float64, order="C")
    vv = np.array(v, np.float64, order="C")
    r = np.ascontiguousarray(rows, np.int32)
    ld = p.shape[1]
    bc1 = 1.0 - b1 ** step
    bc2 = 1.0 - b2 ** step
    lib().or_adam(_p(p), _p(g), _p(mm), _p(vv), ld, _p(r), r.shape[0], lr, b1, b2, eps, bc1, bc2)
    return p, mm, vv


def union_list(visible_lists):
    """Ascending union of per-view visible index lists."""
    out = np.zeros(0, np.int32)
    for v in visible_lists:
        out = np.union1d(out, v)
    return out.astype(np.int32)


# ---------------------------------------------------------------------------
# view coupling (Odin summary page, "Relative locality graph" and the
# importance-based edge weight / scheduling priority formulas), over the
# views' visible-index lists as the views' point sets
# ---------------------------------------------------------------------------

def view_overlap(visible_lists):
    """[B][B] int64 matrix of |V_i n V_j| (the diagonal: |V_i|) for B
    ascending visible-index lists, one np.intersect1d per pair."""
    B = len(visible_lists)
    inter = np.zeros((B, B), np.int64)
    for i in range(B):
        for j in range(i, B):
            c = np.intersect1d(visible_lists[i], visible_lists[j], assume_unique=True).size
            inter[i, j] = inter[j, i] = c
    return inter


def view_coupling(inter):
    """Jaccard edge weights w_ij = |V_i n V_j| / |V_i u V_j| in fp64, with
    |V_i u V_j| = |V_i| + |V_j| - |V_i n V_j|; w_ij = 0 when the union is
    empty."""
    inter = np.asarray(inter, np.int64)
    d = np.diag(inter)
    union = d[:, None] + d[None, :] - inter
    w = np.zeros(inter.shape, np.float64)
    nz = union > 0
    w[nz] = inter[nz].astype(np.float64) / union[nz].astype(np.float64)
    return w


def view_priority(w, prev):
    """s(v | U_prev) = sum over u in U_prev of w_uv, for every view v, the
    terms added in the order of ``prev`` (fp64)."""
    w = np.asarray(w, np.float64)
    s = np.zeros(w.shape[0], np.float64)
    for u in prev:
        s = s + w[u]
    return s


def tile_partition(cost, num_blocks):
    """Bounds of ``num_blocks`` contiguous runs of tile ids of about equal
    total cost (Grendel-GS notes, "dynamic load balancing", pixel-wise
    balancing: cumulative sum of the per-tile cost, then a sorted search
    for the multiples of total / K).  P is the exclusive prefix sum of
    ``cost`` (P[0] = 0, P[T] = total); bounds[0] = 0, bounds[K] = T, and
    bounds[d] for 0 < d < K is the first t with P[t] >= d * total / K,
    compared exactly as K * P[t] >= d * total in integers."""
    cost = np.asarray(cost, np.uint64)
    T, K = cost.size, int(num_blocks)
    P = np.zeros(T + 1, dtype=object)
    P[1:] = np.cumsum(cost.astype(object))
    total = P[T]
    bounds = np.zeros(K + 1, np.int64)
    bounds[K] = T
    for d in range(1, K):
        # searchsorted on the exact rational targets d * total / K
        t = 0
        while t < T and K * P[t] < d * total:
            t += 1
        bounds[d] = t
    return bounds


def tile_blocks_of_rect(rect, bounds, TX):
    """Ascending block ids whose tile-id range holds a tile of the half-open
    rectangle rect = (x0, y0, x1, y1): the tiles are enumerated one by one
    and each is looked up in the bounds."""
    x0, y0, x1, y1 = (int(r) for r in rect)
    ids = np.array([ty * TX + tx for ty in range(y0, y1) for tx in range(x0, x1)], np.int64)
    if ids.size == 0:
        return np.zeros(0, np.int64)
    return np.unique(np.searchsorted(np.asarray(bounds, np.int64), ids, side="right") - 1)


def pack_records(rects, visible, bounds, TX):
    """The sending side of the sparse all-to-all from the Gaussian-wise to
    the pixel-wise split (Grendel-GS notes, "hybrid parallel strategy" and
    "sparse all-to-all communication"): for each tile block d, in order,
    the ascending indices of the visible Gaussians whose rectangle holds a
    tile of block d.  Returns (offsets [K + 1] int64, indices int32)."""
    K = len(bounds) - 1
    per = [[] for _ in range(K)]
    for i in np.flatnonzero(np.asarray(visible)):
        for d in tile_blocks_of_rect(rects[i], bounds, TX):
            per[d].append(int(i))
    offsets = np.zeros(K + 1, np.int64)
    offsets[1:] = np.cumsum([len(x) for x in per])
    idx = np.array([i for x in per for i in x], np.int32)
    return offsets, idx


def unpack_grads(grad2d, recv, offsets, idx):
    """The receiving end of the reverse all-to-all: each block's gradient
    rows (``recv`` in the packed order) added into the Gaussians' rows,
    block by block in ascending order, in fp32 (each Gaussian appears at
    most once per block)."""
    g = np.array(grad2d, np.float32, copy=True)
    for d in range(len(offsets) - 1):
        a, b = int(offsets[d]), int(offsets[d + 1])
        g[idx[a:b]] = g[idx[a:b]] + np.asarray(recv[a:b], np.float32)
    return g


def densify_stats(grad2d, rows, accum, denom):
    """One view's contribution to the densification statistic (Grendel-GS
    notes, "training pipeline": densification clones or splits Gaussians
    whose screen position keeps being pulled, prunes transparent ones): for
    every listed (visible) row, accum += |dL/d(u, v)| in pixel units and
    denom += 1.  fp32, one rounding per operation (u*u, v*v, their sum, the
    square root, the accumulation), since the statistic decides."""
    g = np.asarray(grad2d, np.float32)
    r = np.asarray(rows, np.int64)
    a = np.array(accum, np.float32, copy=True)
    d = np.array(denom, np.int32, copy=True)
    gu, gv = g[r, 0], g[r, 1]
    with np.errstate(over="ignore"):      # a huge gradient overflows to +inf, as in fp32 anywhere
        a[r] = a[r] + np.sqrt(gu * gu + gv * gv)
    d[r] = d[r] + 1
    return a, d


def _rot(q):
    """Rotation matrices [n][3][3] of quaternions (w, x, y, z) [4][n], fp64."""
    q = np.asarray(q, np.float64)
    q = q / np.linalg.norm(q, axis=0)
    w, x, y, z = q
    return np.stack([
        np.stack([1 - 2 * (y * y + z * z), 2 * (x * y - w * z), 2 * (x * z + w * y)], -1),
        np.stack([2 * (x * y + w * z), 1 - 2 * (x * x + z * z), 2 * (y * z - w * x)], -1),
        np.stack([2 * (x * z - w * y), 2 * (y * z + w * x), 1 - 2 * (x * x + y * y)], -1)], -2)


def densify(params, m, v, accum, denom, grad_threshold, log_scale_threshold, logit_threshold, normals,
            log_shrink):
    """Clone / split / prune (Grendel-GS notes, "training pipeline",
    densification), on the [59][n] parameter planes:

    * g = accum / denom (fp32; 0 where denom = 0); a Gaussian densifies
      when g >= grad_threshold;
    * a densifying Gaussian whose largest log-scale is <= log_scale_threshold
      is cloned (kept, plus an identical copy); a larger one is split: it is
      replaced by two children at mean + R(q) (exp(log-scale) * z_c) for the
      caller's standard normals z_c = normals[c, :, i], with log-scales
      lowered by log_shrink (fp32) and every other parameter copied;
    * a Gaussian whose opacity logit is not >= logit_threshold is pruned
      with all its copies.

    Output columns: the kept originals in index order, then the clones, then
    every split parent's first child, then every second child.  New
    Gaussians start with zero Adam moments; kept ones keep theirs.  Returns
    (params, m, v) with the children's means in fp64, the rest copied."""
    p = np.asarray(params, np.float32)
    a = np.asarray(accum, np.float32)
    d = np.asarray(denom, np.int32)
    g = np.zeros_like(a)
    nz = d > 0
    g[nz] = a[nz] / d[nz].astype(np.float32)
    dense = g >= np.float32(grad_threshold)
    maxls = p[3:6].max(axis=0)
    small = maxls <= np.float32(log_scale_threshold)
    big = maxls > np.float32(log_scale_threshold)
    low = ~(p[10] >= np.float32(logit_threshold))
    clone = dense & small & ~low
    split = dense & big & ~low
    keep = ~(dense & big) & ~low
    kids = []
    for c in range(2):
        ch = p[:, split].astype(np.float64)
        s = np.exp(p[3:6, split].astype(np.float64))
        off = np.einsum("nij,nj->ni", _rot(p[6:10, split]), (s * np.asarray(normals, np.float64)[c][:, split]).T)
        ch[0:3] = p[0:3, split].astype(np.float64) + off.T
        ch[3:6] = (p[3:6, split] - np.float32(log_shrink)).astype(np.float64)
        kids.append(ch)
    out = np.concatenate([p[:, keep].astype(np.float64), p[:, clone].astype(np.float64)] + kids, axis=1)
    zeros = np.zeros((p.shape[0], int(clone.sum()) + 2 * int(split.sum())), np.float32)
    om = np.concatenate([np.asarray(m, np.float32)[:, keep], zeros], axis=1)
    ov = np.concatenate([np.asarray(v, np.float32)[:, keep], zeros], axis=1)
    return out, om, ov


# ---------------------------------------------------------------------------
# one whole training step, stage by stage
# ---------------------------------------------------------------------------

def step(work, params=None, m=None, v=None, t=1, at_fp32=True, dl_tol=None):
    """One oracle training step over all views of ``work`` (a
    ``synth.Workload``).  Returns a dict with per-view forward results,
    the accumulated fp64 gradients (+ magnitudes), the union list, and the
    Adam-updated fp64 params / m / v.

    The chain rule is evaluated at the fp32 forward's values by default (the
    gradient of the image that was rendered).  With
    ``dl_tol = (a, r)`` the image-gradient tolerance a * max|dL/dI| +
    r * |dL/dI| is also propagated through the backward's magnitudes
    (``mags_dl``, per view ``m2d_dl``)."""
    p32 = _params(work.params if params is None else params)
    n = p32.shape[1]
    grads = np.zeros((59, n))
    mags = np.zeros((59, n))
    mags_dl = np.zeros((59, n))
    views = []
    total_loss = 0.0
    for cam, tgt in zip(work.cameras, work.targets):
        img, Tf, last, proc = render(p32, cam)
        L, dL, l1, ss = loss(img, tgt, work.w_l1, work.w_ssim)
        g2d, m2d, _, _ = backward(p32, cam, dL, grads, mags, at_fp32=at_fp32)
        vw = dict(image=img, T_final=Tf, last=last, tile_processed=proc, loss=L, dL_dimage=dL, g2d=g2d, m2d=m2d)
        if dl_tol is not None:
            gm = dl_tol[0] * np.max(np.abs(dL)) + dl_tol[1] * np.abs(dL)
            _, m2d_dl, _, _ = backward(p32, cam, dL, None, mags_dl, at_fp32=at_fp32, gmag=gm)
            vw["m2d_dl"] = m2d_dl
        vw["visible"] = visible_list(p32, cam)
        views.append(vw)
        total_loss += L
    rows = union_list([vw["visible"] for vw in views])
    m0 = np.zeros((59, n)) if m is None else m
    v0 = np.zeros((59, n)) if v is None else v
    p_new, m_new, v_new = adam(p32, grads, m0, v0, rows, work.lr, work.beta1, work.beta2,
                               work.eps, step=t)
    return dict(views=views, loss=total_loss, grads=grads, mags=mags, mags_dl=mags_dl, union=rows,
                params=p_new, m=m_new, v=v_new)
