"""Python binding of libgs, the HIP (gfx950) library for one 3D Gaussian
Splatting training step.

The functions below carry the names of the C entry points declared in
``include/gs.h`` and only marshal arguments (torch tensors -> device
pointers, the current HIP stream); every step of the computation runs in the
library's kernels.  Importing this module fails loudly if ``libgs.so`` has
not been built: there is no fallback.

``TrainStep`` strings the entry points together for a batch of views and
owns the device buffers (allocated once with torch, reused across steps).
"""
from __future__ import annotations

import contextlib
import ctypes as C
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgs.so")

GS_OK, GS_ERR_INVALID_ARG, GS_ERR_CAPACITY, GS_ERR_HIP = 0, 1, 2, 3
GS_OP_PREPROCESS, GS_OP_BIN_SORT, GS_OP_LOSS, GS_OP_SPARSE_ADAM, GS_OP_RASTER = 0, 1, 2, 3, 4
GS_OP_VIEW_OVERLAP, GS_OP_PACK, GS_OP_DENSIFY, GS_OP_PREPROCESS_VIEWS = 5, 6, 7, 8
GS_PROJ_WORDS = 16
GS_GRAD2D_WORDS = 12
GS_MAX_FUSED_VIEWS = 16
GS_TOUCHED_SLOTS = 16
GS_BIN_ALL, GS_BIN_DEPTH, GS_BIN_PAIRS = 0, 1, 2
GS_MAX_PREPROCESS_VIEWS = 16
GS_MAX_COUPLED_VIEWS = 65536
GS_MAX_TILE_BLOCKS = 64
GS_MAX_PARTITION_TILES = 1 << 21
GS_MAX_PLANE_ROWS = 1 << 30
SEGMENT_LEN = 512    # list entries per segment of the split raster backward
TILE = 16

EXPORTS = ["gs_status_string", "gs_last_error", "gs_version", "gs_workspace_size", "gs_preprocess",
           "gs_bin_sort", "gs_bin_sort_async", "gs_render_fwd", "gs_loss", "gs_render_bwd", "gs_project_bwd",
           "gs_sparse_adam", "gs_project_bwd_adam", "gs_visible_list", "gs_view_overlap", "gs_view_priority",
           "gs_tile_partition", "gs_pack_records", "gs_unpack_grads", "gs_densify_stats", "gs_densify",
           "gs_sparse_adam_noalloc", "gs_preprocess_views"]
GS_NOALLOC_SCRATCH_BYTES = 256 * 1024
GS_NOALLOC_MAX_N = (GS_NOALLOC_SCRATCH_BYTES // 4 - 1) * 4096


class gs_camera(C.Structure):
    _fields_ = [("width", C.c_int32), ("height", C.c_int32),
                ("fx", C.c_float), ("fy", C.c_float), ("cx", C.c_float), ("cy", C.c_float),
                ("R", C.c_float * 9), ("t", C.c_float * 3), ("campos", C.c_float * 3),
                ("near_z", C.c_float)]


class gs_param_grads(C.Structure):
    _fields_ = [("params", C.c_void_p), ("ld", C.c_int64), ("cam", C.POINTER(gs_camera)),
                ("vis_idx", C.c_void_p), ("vis_count", C.c_void_p), ("grads", C.c_void_p)]


_P, _i64, _i32, _f32, _sz = C.c_void_p, C.c_int64, C.c_int32, C.c_float, C.c_size_t
_handle = None


def lib():
    """The loaded libgs.so with argument types set (loaded on first use;
    raises if it has not been built -- there is no fallback)."""
    global _handle
    if _handle is not None:
        return _handle
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python differentiable_gaussian_splatting_dgs_amd/build.py` "
                           "(or __graft_entry__.build()); there is no CPU fallback")
    L = C.CDLL(LIB_PATH)
    L.gs_status_string.restype = C.c_char_p
    L.gs_status_string.argtypes = [C.c_int]
    L.gs_last_error.restype = C.c_char_p
    L.gs_last_error.argtypes = []
    L.gs_version.restype = C.c_int
    L.gs_workspace_size.argtypes = [C.c_int, _i64, _i32, _i32, _i64, C.POINTER(_sz)]
    L.gs_preprocess.argtypes = [_P, _i64, _i64, C.POINTER(gs_camera), _P, _P, _P, _P, _P, _P, _sz, _P]
    L.gs_preprocess_views.argtypes = [_P, _i64, _i64, C.POINTER(gs_camera), _i32, _P, _P, _P, _P, _P, _i32, _P,
                                      _sz, _P]
    L.gs_bin_sort.argtypes = [_P, _P, _i64, _P, _P, _i32, _i32, _P, _P, _i64, C.POINTER(_i64), _P, _P, _P, _sz, _P]
    L.gs_bin_sort_async.argtypes = [_P, _P, _i64, _P, _P, _i32, _i32, _P, _P, _i64, _P, _P, _P, _P, _sz, _i32, _P]
    L.gs_render_fwd.argtypes = [_P, _i64, _P, _P, _P, _i64, _i32, _i32, _P, _P, _P, _P, _P, _sz, _i32, _P]
    L.gs_loss.argtypes = [_P, _P, _i32, _i32, _f32, _f32, _P, _P, _P, _sz, _P]
    L.gs_render_bwd.argtypes = [_P, _i64, _P, _P, _P, _i64, _i32, _i32, _P, _P, _P, _P, _P, _sz, _i32,
                                C.POINTER(gs_param_grads), _P, _P, _i32, _P]
    L.gs_project_bwd.argtypes = [_P, _i64, _i64, C.POINTER(gs_camera), _P, _P, _P, _P, _P]
    L.gs_sparse_adam.argtypes = [_P, _P, _P, _P, _i64, _i64, _P, _P, _P, _f32, _f32, _f32, _f32, _f32, _f32,
                                 _P, _sz, _P]
    L.gs_sparse_adam_noalloc.argtypes = [_P, _P, _P, _P, _i64, _i64, _P, _P, _P, _f32, _f32, _f32, _f32, _f32,
                                         _f32, _P]
    L.gs_project_bwd_adam.argtypes = [_P, _P, _P, _P, _i64, _i64, C.POINTER(gs_camera), _i32,
                                      C.POINTER(C.c_void_p), _P, _P, _P, _P, C.POINTER(gs_camera), _P, _P, _P, _f32, _f32,
                                      _f32, _f32, _f32, _f32, _P, _sz, _P]
    L.gs_visible_list.argtypes = [_P, _i64, _P, _P, _P, _sz, _P]
    L.gs_view_overlap.argtypes = [_P, _i64, _P, _i32, _i64, _P, _P, _P, _sz, _P]
    L.gs_view_priority.argtypes = [_P, _i32, _P, _i32, _P, _P]
    L.gs_tile_partition.argtypes = [_P, _i32, _i32, _P, _P]
    L.gs_pack_records.argtypes = [_P, _i64, _P, _P, _i32, _i32, _P, _i32, _i64, _P, _P, _P, _P, _sz, _P]
    L.gs_unpack_grads.argtypes = [_P, _P, _P, _i32, _i64, _P, _i64, _P]
    L.gs_densify_stats.argtypes = [_P, _P, _P, _i64, _P, _P, _P]
    L.gs_densify.argtypes = [_P, _P, _P, _i64, _i64, _P, _P, _P, _f32, _f32, _f32, _f32, _P, _P, _P, _i64, _P, _P,
                             _sz, _P]
    for name in EXPORTS[3:]:
        getattr(L, name).restype = C.c_int
    _handle = L
    return L


class GSError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().gs_last_error().decode() or lib().gs_status_string(status).decode()
        super().__init__(f"{where}: {lib().gs_status_string(status).decode()} ({msg})")


def _check(status: int, where: str):
    if status != GS_OK:
        raise GSError(status, where)


def _ptr(t):
    if t is None:
        return None
    return C.c_void_p(t.data_ptr())


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def make_camera(cam) -> gs_camera:
    """ctypes camera from anything with the fields of ``gs_camera``
    (width, height, fx, fy, cx, cy, R (3x3), t, campos, near)."""
    c = gs_camera()
    c.width, c.height = int(cam.width), int(cam.height)
    c.fx, c.fy, c.cx, c.cy = float(cam.fx), float(cam.fy), float(cam.cx), float(cam.cy)
    R = [float(x) for row in cam.R for x in row]
    for k in range(9):
        c.R[k] = R[k]
    for k in range(3):
        c.t[k] = float(cam.t[k])
        c.campos[k] = float(cam.campos[k])
    c.near_z = float(getattr(cam, "near", getattr(cam, "near_z", 0.2)))
    return c


# ---------------------------------------------------------------------------
# the C entry points, one wrapper each
# ---------------------------------------------------------------------------

def gs_version() -> int:
    return lib().gs_version()


def gs_status_string(status: int) -> str:
    return lib().gs_status_string(status).decode()


def gs_last_error() -> str:
    return lib().gs_last_error().decode()


def gs_workspace_size(op: int, n: int = 0, width: int = 0, height: int = 0, pair_capacity: int = 0) -> int:
    b = _sz(0)
    _check(lib().gs_workspace_size(op, n, width, height, pair_capacity, C.byref(b)), "gs_workspace_size")
    return b.value


def gs_preprocess(params, n, ld, cam, proj, vis_idx, vis_count, union_flags, workspace, stream=None,
                  proj_bin=None):
    """``proj_bin``: None, or a [n][4] float32 tensor that also receives
    each record's last four words (what the binning reads)."""
    c = cam if isinstance(cam, gs_camera) else make_camera(cam)
    _check(lib().gs_preprocess(_ptr(params), n, ld, C.byref(c), _ptr(proj), _ptr(proj_bin), _ptr(vis_idx),
                              _ptr(vis_count), _ptr(union_flags), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(stream)), "gs_preprocess")


def gs_preprocess_views(params, n, ld, cams, proj, vis_idx, vis_count, union_flags, workspace, stream=None,
                        max_workgroups=0, proj_bin=None):
    """gs_preprocess of several views in one pass over the parameters:
    ``cams``, ``proj`` and ``vis_idx`` hold one entry per view (and
    ``proj_bin``, when given, one tensor or None per view),
    ``vis_count`` is a device int64 tensor with one count per view;
    ``max_workgroups`` > 0 caps the grid (a smaller HBM share)."""
    nv = len(cams)
    assert len(proj) == nv and len(vis_idx) == nv
    carr = (gs_camera * max(nv, 1))(*[c if isinstance(c, gs_camera) else make_camera(c) for c in cams])
    parr = (C.c_void_p * max(nv, 1))(*[t.data_ptr() for t in proj])
    varr = (C.c_void_p * max(nv, 1))(*[t.data_ptr() for t in vis_idx])
    barr = None
    if proj_bin is not None:
        assert len(proj_bin) == nv
        barr = (C.c_void_p * max(nv, 1))(*[None if t is None else t.data_ptr() for t in proj_bin])
    _check(lib().gs_preprocess_views(_ptr(params), n, ld, carr, nv, parr, barr, varr, _ptr(vis_count),
                                     _ptr(union_flags), int(max_workgroups), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(stream)),
           "gs_preprocess_views")


def gs_bin_sort(proj, n, vis_idx, vis_count, width, height, keys, vals, pair_capacity, tile_ranges, workspace,
                tile_order=None, stream=None, proj_bin=None) -> int:
    """Returns M (the pair count); raises GSError(GS_ERR_CAPACITY) with
    ``.num_pairs`` set when M > pair_capacity.  ``proj_bin``: None or the
    view's dense copy from gs_preprocess."""
    m = _i64(0)
    st = lib().gs_bin_sort(_ptr(proj), _ptr(proj_bin), n, _ptr(vis_idx), _ptr(vis_count), width, height, _ptr(keys), _ptr(vals),
                          pair_capacity, C.byref(m), _ptr(tile_ranges), _ptr(tile_order), _ptr(workspace),
                          workspace.numel() * workspace.element_size(), _stream(stream))
    if st != GS_OK:
        err = GSError(st, "gs_bin_sort")
        err.num_pairs = m.value
        raise err
    return m.value


def gs_bin_sort_async(proj, n, vis_idx, vis_count, width, height, keys, vals, pair_capacity, num_pairs_dev,
                      tile_ranges, workspace, tile_order=None, stream=None, proj_bin=None, part=0):
    """As gs_bin_sort without blocking: M lands in num_pairs_dev (a device
    int64); M > pair_capacity leaves empty ranges (checked by the caller)."""
    _check(lib().gs_bin_sort_async(_ptr(proj), _ptr(proj_bin), n, _ptr(vis_idx), _ptr(vis_count), width, height,
                                   _ptr(keys), _ptr(vals), pair_capacity, _ptr(num_pairs_dev), _ptr(tile_ranges),
                                   _ptr(tile_order), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   int(part), _stream(stream)), "gs_bin_sort_async")


def gs_render_fwd(proj, n, vals, tile_ranges, num_pairs, width, height, image, T_final, last,
                  tile_processed=None, tile_order=None, split_ws=None, segment_len=SEGMENT_LEN, stream=None):
    _check(lib().gs_render_fwd(_ptr(proj), n, _ptr(vals), _ptr(tile_ranges), _ptr(tile_order), num_pairs, width,
                               height, _ptr(image), _ptr(T_final), _ptr(last), _ptr(tile_processed),
                               _ptr(split_ws), _nbytes(split_ws), segment_len, _stream(stream)),
           "gs_render_fwd")


def gs_loss(image, target, width, height, w_l1, w_ssim, loss, dL_dimage, workspace, stream=None):
    _check(lib().gs_loss(_ptr(image), _ptr(target), width, height, float(w_l1), float(w_ssim), _ptr(loss),
                        _ptr(dL_dimage), _ptr(workspace), workspace.numel() * workspace.element_size(),
                        _stream(stream)), "gs_loss")


def gs_render_bwd(proj, n, vals, tile_ranges, num_pairs, width, height, T_final, last, dL_dimage, grad2d,
                  tile_order=None, split_ws=None, segment_len=SEGMENT_LEN, param_grads=None, visits=None,
                  stream=None, touched=None, touched_slot=0):
    """``param_grads``: None, or (params, ld, cam, vis_idx, vis_count,
    grads) to chain the view's projection backward into the [59][ld]
    gradient planes in the same call; ``visits``: None or a device int64
    scalar the number of back-propagated (pixel, entry) pairs is added to."""
    pg = None
    if param_grads is not None:
        params, ld, cam, vis_idx, vis_count, grads = param_grads
        c = cam if isinstance(cam, gs_camera) else make_camera(cam)
        pg = gs_param_grads(params.data_ptr(), int(ld), C.pointer(c), vis_idx.data_ptr(), vis_count.data_ptr(),
                            grads.data_ptr())
    _check(lib().gs_render_bwd(_ptr(proj), n, _ptr(vals), _ptr(tile_ranges), _ptr(tile_order), num_pairs, width,
                               height, _ptr(T_final), _ptr(last), _ptr(dL_dimage), _ptr(grad2d),
                               _ptr(split_ws), _nbytes(split_ws), segment_len,
                               None if pg is None else C.byref(pg), _ptr(visits), _ptr(touched),
                               int(touched_slot), _stream(stream)),
           "gs_render_bwd")


def gs_project_bwd(params, n, ld, cam, vis_idx, vis_count, grad2d, grads, stream=None):
    c = cam if isinstance(cam, gs_camera) else make_camera(cam)
    _check(lib().gs_project_bwd(_ptr(params), n, ld, C.byref(c), _ptr(vis_idx), _ptr(vis_count), _ptr(grad2d),
                               _ptr(grads), _stream(stream)), "gs_project_bwd")


def gs_sparse_adam(params, grads, m, v, n, ld, union_flags, union_idx, union_count, lr, beta1, beta2, eps,
                   bias_c1, bias_c2, workspace, stream=None):
    _check(lib().gs_sparse_adam(_ptr(params), _ptr(grads), _ptr(m), _ptr(v), n, ld, _ptr(union_flags),
                               _ptr(union_idx), _ptr(union_count), float(lr), float(beta1), float(beta2),
                               float(eps), float(bias_c1), float(bias_c2), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream)), "gs_sparse_adam")


def gs_sparse_adam_noalloc(params, grads, m, v, n, ld, union_flags, union_idx, union_count, lr, beta1, beta2,
                           eps, bias_c1, bias_c2, stream=None):
    _check(lib().gs_sparse_adam_noalloc(_ptr(params), _ptr(grads), _ptr(m), _ptr(v), n, ld, _ptr(union_flags),
                                        _ptr(union_idx), _ptr(union_count), float(lr), float(beta1), float(beta2),
                                        float(eps), float(bias_c1), float(bias_c2), _stream(stream)),
           "gs_sparse_adam_noalloc")


def gs_project_bwd_adam(params, grads, m, v, n, ld, cams, grad2d, union_flags, union_idx, union_count, lr,
                        beta1, beta2, eps, bias_c1, bias_c2, workspace, next_cam=None, next_proj=None,
                        next_flags=None, stream=None, next_proj_bin=None, touched=None):
    """``cams`` / ``grad2d``: one camera and one screen-gradient buffer per
    fused view; ``grads`` None when no other view contributed; ``next_*``:
    the preprocess of the view rendered next, on the updated rows."""
    nv = len(cams)
    assert len(grad2d) == nv
    carr = (gs_camera * max(nv, 1))(*[c if isinstance(c, gs_camera) else make_camera(c) for c in cams])
    parr = (C.c_void_p * max(nv, 1))(*[g.data_ptr() for g in grad2d])
    nc = None
    if next_cam is not None:
        nc = C.byref(next_cam if isinstance(next_cam, gs_camera) else make_camera(next_cam))
    _check(lib().gs_project_bwd_adam(_ptr(params), _ptr(grads), _ptr(m), _ptr(v), n, ld, carr, nv, parr,
                                     _ptr(touched), _ptr(union_flags), _ptr(union_idx), _ptr(union_count), nc, _ptr(next_proj),
                                     _ptr(next_proj_bin), _ptr(next_flags), lr, beta1, beta2, eps, bias_c1, bias_c2, _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(stream)),
           "gs_project_bwd_adam")


def gs_visible_list(flags, n, vis_idx, vis_count, workspace, stream=None):
    _check(lib().gs_visible_list(_ptr(flags), n, _ptr(vis_idx), _ptr(vis_count), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)), "gs_visible_list")


def gs_view_overlap(lists, ld, counts, num_views, n, inter, weights, workspace, stream=None):
    _check(lib().gs_view_overlap(_ptr(lists), ld, _ptr(counts), num_views, n, _ptr(inter), _ptr(weights),
                                 _ptr(workspace), _nbytes(workspace), _stream(stream)), "gs_view_overlap")


def gs_view_priority(weights, num_views, prev, num_prev, score, stream=None):
    _check(lib().gs_view_priority(_ptr(weights), num_views, _ptr(prev), num_prev, _ptr(score), _stream(stream)),
           "gs_view_priority")


def gs_tile_partition(cost, num_tiles, num_blocks, bounds, stream=None):
    _check(lib().gs_tile_partition(_ptr(cost), num_tiles, num_blocks, _ptr(bounds), _stream(stream)),
           "gs_tile_partition")


def gs_pack_records(proj, n, vis_idx, vis_count, width, height, bounds, num_blocks, capacity, send_offsets,
                    send_idx, send_rec, workspace, stream=None):
    _check(lib().gs_pack_records(_ptr(proj), n, _ptr(vis_idx), _ptr(vis_count), width, height, _ptr(bounds),
                                 num_blocks, capacity, _ptr(send_offsets), _ptr(send_idx), _ptr(send_rec),
                                 _ptr(workspace), _nbytes(workspace), _stream(stream)), "gs_pack_records")


def gs_unpack_grads(recv_grad, send_offsets, send_idx, num_blocks, capacity, grad2d, n, stream=None):
    _check(lib().gs_unpack_grads(_ptr(recv_grad), _ptr(send_offsets), _ptr(send_idx), num_blocks, capacity,
                                 _ptr(grad2d), n, _stream(stream)), "gs_unpack_grads")


def gs_densify_stats(grad2d, vis_idx, vis_count, n, accum, denom, stream=None):
    _check(lib().gs_densify_stats(_ptr(grad2d), _ptr(vis_idx), _ptr(vis_count), n, _ptr(accum), _ptr(denom),
                                  _stream(stream)), "gs_densify_stats")


def gs_densify(params, m, v, n, ld, accum, denom, normals, grad_threshold, log_scale_threshold, logit_threshold,
               log_shrink, out_params, out_m, out_v, ld_out, out_n, workspace, stream=None):
    _check(lib().gs_densify(_ptr(params), _ptr(m), _ptr(v), n, ld, _ptr(accum), _ptr(denom), _ptr(normals),
                            grad_threshold, log_scale_threshold, logit_threshold, log_shrink, _ptr(out_params),
                            _ptr(out_m), _ptr(out_v), ld_out, _ptr(out_n), _ptr(workspace), _nbytes(workspace),
                            _stream(stream)), "gs_densify")


def auto_segment_len(width: int, height: int) -> int:
    """Segment length of the split raster backward for a width x height
    view, from its count of 8x8 quarter-tiles (one wave each): splitting
    pays while the few longest lists set the raster time and the rest of
    the chip has run dry; measured on MI355X, 256 is best near 17k
    quarters (1297x840), 512 near 33k (1920x1080), and with 130k (3840x2160)
    the chip stays full to the end and the split only adds the records'
    traffic (0: unsplit)."""
    q = ((width + TILE - 1) // TILE) * ((height + TILE - 1) // TILE) * 4
    return 256 if q < 24_000 else (512 if q < 64_000 else 0)


class ViewCoupling:
    """Visible lists of a set of views over one scene and their coupling
    graph (gs_preprocess per view into row v of ``lists``, then
    gs_view_overlap).  Buffers are allocated once for ``num_views`` views
    of ``n`` Gaussians."""

    def __init__(self, n: int, num_views: int, device="cuda"):
        self.n, self.B, self.device = int(n), int(num_views), torch.device(device)
        self.ld = max(self.n, 1)
        self.lists = torch.empty((self.B, self.ld), dtype=torch.int32, device=self.device)
        self.counts = torch.zeros(self.B, dtype=torch.int64, device=self.device)
        self.inter = torch.empty((self.B, self.B), dtype=torch.int64, device=self.device)
        self.weights = torch.empty((self.B, self.B), dtype=torch.float64, device=self.device)
        self.ws = _bytes(gs_workspace_size(GS_OP_VIEW_OVERLAP, self.n, self.B), self.device)
        self.ws_pre = _bytes(gs_workspace_size(GS_OP_PREPROCESS, self.n), self.device)
        self.proj = torch.empty((max(self.n, 1), GS_PROJ_WORDS), dtype=torch.float32, device=self.device)

    def visible_lists(self, params, ld, cams, stream=None):
        """Row v of ``lists`` and counts[v] = the visible list of cams[v]."""
        assert len(cams) == self.B
        for v, cam in enumerate(cams):
            gs_preprocess(params, self.n, ld, cam, self.proj, self.lists[v], self.counts[v:v + 1], None,
                          self.ws_pre, stream)

    def overlap(self, weights=True, stream=None):
        gs_view_overlap(self.lists, self.ld, self.counts, self.B, self.n, self.inter,
                        self.weights if weights else None, self.ws, stream)
        return self.inter, (self.weights if weights else None)

    def priority(self, prev, stream=None):
        """s(v | prev) for every view, prev an int32 device tensor."""
        score = torch.empty(self.B, dtype=torch.float64, device=self.device)
        gs_view_priority(self.weights, self.B, prev, int(prev.numel()), score, stream)
        return score


# ---------------------------------------------------------------------------
# a training step over a batch of views
# ---------------------------------------------------------------------------

def _bytes(nbytes, device):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


class View:
    """Per-view device buffers (image-sized ones and the pair arrays)."""

    def __init__(self, cam, target, n, pair_capacity, device):
        self.cam = make_camera(cam)
        W, H = self.cam.width, self.cam.height
        self.W, self.H = W, H
        self.T = ((W + TILE - 1) // TILE) * ((H + TILE - 1) // TILE)
        self.target = torch.as_tensor(target, dtype=torch.float32).to(device).contiguous()
        self.image = torch.empty((3, H, W), dtype=torch.float32, device=device)
        self.T_final = torch.empty((H, W), dtype=torch.float32, device=device)
        self.last = torch.empty((H, W), dtype=torch.int32, device=device)
        self.dL = torch.empty((3, H, W), dtype=torch.float32, device=device)
        self.loss = torch.zeros(1, dtype=torch.float32, device=device)
        self.ranges = torch.empty((self.T, 2), dtype=torch.int32, device=device)
        self.order = torch.empty(self.T, dtype=torch.int32, device=device)
        self.tile_processed = torch.empty(self.T, dtype=torch.int32, device=device)
        self.num_pairs = 0


class _PairSet:
    """Buffers of one view's binning that its rasterisation reads: sorted
    pairs and the binning workspace.  A step cycles through several sets so
    that later views' binning can run while the current view renders and
    back-propagates."""

    def __init__(self, n, cap, device, with_keys):
        self.n, self.device, self.with_keys = n, device, with_keys
        self.alloc(cap)

    def alloc(self, cap):
        self.capacity = cap
        # the 64-bit sort keys are an output the rasterisers never read; the
        # binning needs them only for images over 256 tiles on a side
        self.keys = torch.empty(max(cap, 1), dtype=torch.int64, device=self.device) if self.with_keys else None
        self.vals = torch.empty(max(cap, 1), dtype=torch.int32, device=self.device)
        self.ws_sort = _bytes(gs_workspace_size(GS_OP_BIN_SORT, self.n, 0, 0, cap), self.device)


class TrainStep:
    """Owns parameters, Adam state and scratch; ``step()`` runs one training
    step (all views of the batch, then sparse Adam).

    Views cycle through three buffer sets (two for a batch of two).  The
    last ndefer = min(views, max_fused_views) views (at most
    GS_MAX_FUSED_VIEWS) own a screen-gradient buffer each; the earlier ones
    alternate between two more.
    In ``step()`` the first view is binned on the caller's stream (its
    records come from the previous step's Adam pass) while the other views'
    preprocess runs in one pass over the parameters on a side stream; view
    k + 1's binning is then issued on a side stream (two alternating ones
    for batches of more than 8 views, ``bin_streams``) while view k renders,
    takes its loss and runs the raster backward on the caller's stream; the
    projection backward of an early view runs on another stream, that of the
    last ndefer views in the Adam pass (one read of the parameters for all
    of them); events order every reuse of a set or buffer and every
    hand-over.  ``forward_view`` / ``backward_view`` run
    one view's stages in order on the current stream."""

    # every projection also writes a dense [n][4] copy of the records' last
    # four words per view, which the binning reads (16 bytes per Gaussian
    # instead of a 64-byte record)
    dense_bin = True
    # the fused views' raster backward marks the rows it reaches, and the
    # Adam pass reads only those rows' screen-space gradients: "auto" turns
    # it on for more than 8 fused views, where those buffers outgrow the
    # caches (at 16 views of 12 M Gaussians: the pass 8.9 -> 8.2 ms, the
    # marking +45 us per raster backward; at 4 views of 1 M the pass gains
    # nothing and the marking costs ~10 us per view)
    use_touched = "auto"

    def __init__(self, params, cameras, targets, w_l1, w_ssim, lr, beta1, beta2, eps, device="cuda",
                 pair_capacity=None, record_tiles=False, segment_len="auto", fuse_next_preprocess=True,
                 max_fused_views=GS_MAX_FUSED_VIEWS, bin_streams="auto"):
        p = torch.as_tensor(params, dtype=torch.float32)
        assert p.ndim == 2 and p.shape[0] == 59
        self.device = torch.device(device)
        n = int(p.shape[1])
        self.w_l1, self.w_ssim = float(w_l1), float(w_ssim)
        self.lr, self.beta1, self.beta2, self.eps = float(lr), float(beta1), float(beta2), float(eps)
        self.t = 0
        self.record_tiles = record_tiles
        self.timer = None        # optional: name -> list of (start, end) torch.cuda.Event pairs
        self.timer_stages = None  # optional: the stage names to time (None: all)
        self.timer_views = None   # optional: the views whose raster backward is timed (None: all)
        self.visits = None       # optional: device int64 [views]: view k's raster backward adds its
                                 # back-propagated (pixel, entry) count to visits[k]
        # densification statistic (track_densify): per Gaussian the summed
        # |dL/d(u, v)| and the number of views it was visible in
        self.dens_accum = None
        self.dens_denom = None
        # screen-gradient buffers: one per view whose projection backward
        # step() fuses into Adam (the last ndefer views), two alternating
        # for the earlier views
        nv = len(cameras)
        assert 1 <= max_fused_views <= GS_MAX_FUSED_VIEWS
        self.ndefer = min(nv, int(max_fused_views))
        self.nfirst = nv - self.ndefer
        self.vis_count = torch.zeros(len(cameras), dtype=torch.int64, device=self.device)
        self.union_count = torch.zeros(1, dtype=torch.int64, device=self.device)
        if pair_capacity is None:
            pair_capacity = max(1 << 20, 24 * n)       # grown on demand
        self.pair_capacity = int(min(pair_capacity, (1 << 31) - 1))
        self.views = [View(c, tg, n, self.pair_capacity, self.device) for c, tg in zip(cameras, targets)]
        # binnings in flight beside the rendered view: with few views a
        # view's render chain outlasts the next binning and a second binning
        # beside it gains nothing (4 views of 1080p: 3.680 ms per step with
        # one, 3.689 with two); with many, the binnings bound the step (16
        # views: 57.2 ms with one, 52.9 with two, 54.1 with three, 57.4 with
        # four)
        self.bin_streams = (2 if len(cameras) > 8 else 1) if bin_streams == "auto" else int(bin_streams)
        assert 1 <= self.bin_streams <= 4
        # a set per binning in flight, one for the rendered view and one spare
        self.nsets = min(self.bin_streams + 2, max(2, len(self.views)))
        self._with_keys = any(v.W > 4096 or v.H > 4096 for v in self.views)
        self._cur = 0                       # set of the view last prepared
        self._curv = 0                      # the view last prepared
        self._free = [None] * self.nsets    # per set: event after its last reader
        self._gcur = 0
        self._alloc_rows(p.to(self.device).contiguous(), None, None)
        self.M_dev = torch.zeros(len(self.views), dtype=torch.int64, device=self.device)
        self.M_host = torch.zeros(len(self.views), dtype=torch.int64, pin_memory=True)
        self._set_cap = [0] * len(self.views)       # capacity of the set each view was binned into
        # preprocess + binning of the next views, and further binning streams
        self.side = torch.cuda.Stream(device=self.device)
        self.sides = [self.side] + [torch.cuda.Stream(device=self.device) for _ in range(self.bin_streams - 1)]
        self.gstream = torch.cuda.Stream(device=self.device)   # projection backward
        self.ws_loss = _bytes(max(gs_workspace_size(GS_OP_LOSS, 0, v.W, v.H) for v in self.views), self.device)
        # step()'s Adam pass also runs the next step's first preprocess on the
        # rows it updates (the views are the same every step, so a row
        # outside the union was invisible in view 0 and keeps its record);
        # its visibility bytes wait in next_flags, zero between uses
        self.fuse_next_preprocess = fuse_next_preprocess
        self._pre0 = False       # view 0's records and flags come from the last Adam pass
        self.preprocess_after_first = False   # the other views' preprocess waits for view 0's binning
        # ... for view 0's depth sort (batches of up to 8 views: at 4 views
        # 3.597 -> 3.588 ms per step; at 16 the long preprocess then delays
        # view 1's binning, 51.76 -> 52.37 ms)
        self.preprocess_after_depth = len(self.views) <= 8
        self.preprocess_workgroups = 0        # grid cap of that preprocess (0: full)
        # the forward's checkpoints and segment list, read by the split raster
        # backward of the same view (both on the current stream, the view's
        # backward before the next view's forward); segment_len None: unsplit
        if segment_len == "auto":
            self.seg = [auto_segment_len(v.W, v.H) for v in self.views]
        else:
            self.seg = [int(segment_len or 0)] * len(self.views)
        split_views = [v for v, sg in zip(self.views, self.seg) if sg]
        self.split_ws = (_bytes(max(gs_workspace_size(GS_OP_RASTER, 0, v.W, v.H) for v in split_views), self.device)
                         if split_views else None)

    def _touched_on(self):
        if self.use_touched == "auto":
            return self.ndefer > 8
        return bool(self.use_touched)

    def _split(self, k):
        """View k's split workspace (None when its backward runs unsplit)."""
        return self.split_ws if self.seg[k] else None

    def _alloc_rows(self, params, m, v):
        """Every buffer with a row per Gaussian, for the n = params.shape[1]
        Gaussians of `params` (device, [59][n], kept); Adam moments from m, v
        or zero; gradients, screen-space gradients and flags zero."""
        self.n = n = int(params.shape[1])
        self.ld = n
        rows = max(n, 1)
        self.params = params
        self.grads = torch.zeros_like(params)
        self.m = m if m is not None else torch.zeros_like(params)
        self.v = v if v is not None else torch.zeros_like(params)
        self.g2d = [torch.zeros((rows, GS_GRAD2D_WORDS), dtype=torch.float32, device=self.device)
                    for _ in range(self.ndefer + (2 if self.nfirst > 0 else 0))]
        self.vis_idx = [torch.empty(rows, dtype=torch.int32, device=self.device) for _ in self.views]
        # every view's projected records (the views' preprocess runs in one
        # pass over the parameters at the start of a step)
        self.vproj = [torch.empty((rows, GS_PROJ_WORDS), dtype=torch.float32, device=self.device)
                      for _ in self.views]
        self.vbin = [torch.empty((rows, 4), dtype=torch.float32, device=self.device) if self.dense_bin else None
                     for _ in self.views]
        self.union_flags = torch.zeros(((rows + 15) // 16) * 16, dtype=torch.uint8, device=self.device)
        self.union_idx = torch.empty(rows, dtype=torch.int32, device=self.device)
        self.next_flags = torch.zeros(((rows + 15) // 16) * 16, dtype=torch.uint8, device=self.device)
        # which fused view's raster backward reached each row (byte w: fused
        # view w), so the Adam pass reads only those screen-space rows; zero
        # between steps (the pass clears what it reads)
        self.touched = torch.zeros((rows, GS_TOUCHED_SLOTS), dtype=torch.uint8, device=self.device)
        self.sets = [_PairSet(n, self.pair_capacity, self.device, self._with_keys) for _ in range(self.nsets)]
        self._free = [None] * self.nsets
        self.ws_pre = _bytes(gs_workspace_size(GS_OP_PREPROCESS, n), self.device)
        npv = min(len(self.views), GS_MAX_PREPROCESS_VIEWS)
        self.ws_pre_views = _bytes(gs_workspace_size(GS_OP_PREPROCESS_VIEWS, n, npv), self.device)
        self.ws_adam = _bytes(gs_workspace_size(GS_OP_SPARSE_ADAM, n), self.device)
        if self.dens_accum is not None:
            self.track_densify()

    # the records of the view last prepared (what tests read back)
    @property
    def proj(self):
        return self.vproj[self._curv]

    @property
    def keys(self):
        """The sorted keys of the view last prepared, or None when the
        binning left them unwritten (images of at most 256 x 256 tiles)."""
        return self.sets[self._cur].keys

    @property
    def vals(self):
        return self.sets[self._cur].vals

    # the screen-gradient buffer of the view last back-propagated
    @property
    def grad2d(self):
        return self.g2d[self._gcur]

    def _gbuf(self, k):
        """Index of view k's screen-gradient buffer."""
        return k - self.nfirst if k >= self.nfirst else self.ndefer + k % 2

    @contextlib.contextmanager
    def _stage(self, name, view=None):
        """Bracket the enclosed launches with events on the current stream
        (the stream the library launches on) when timing is enabled."""
        if self.timer is None or (self.timer_stages is not None and name not in self.timer_stages) or \
                (view is not None and self.timer_views is not None and view not in self.timer_views):
            yield
            return
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        yield
        b.record()
        self.timer.setdefault(name, []).append((a, b))

    # -- one view ---------------------------------------------------------
    def prepare_view(self, k, sync=True, preprocess=True, between=None):
        """Preprocess view k (unless preprocess is False: its records and
        visible list are there already) and bin/sort it into buffer set
        k % nsets.  With sync, the pair count is read (blocking) and the set
        grown if it overflowed; without, it stays on the device in M_dev[k].
        ``between``: None, or a function called (to issue work on the
        stream) between the binning's depth sort and its pairs."""
        vw = self.views[k]
        ps = self.sets[k % self.nsets]
        self._cur = k % self.nsets
        self._curv = k
        if preprocess:
            with self._stage("preprocess"):
                if k == 0 and self._pre0:
                    # records and flags from the last Adam pass
                    gs_visible_list(self.next_flags, self.n, self.vis_idx[0], self.vis_count[0:1], self.ws_pre)
                    self._pre0 = False
                else:
                    gs_preprocess(self.params, self.n, self.ld, vw.cam, self.vproj[k], self.vis_idx[k],
                                  self.vis_count[k:k + 1], self.union_flags, self.ws_pre, proj_bin=self.vbin[k])
        with self._stage("bin_sort"):
            self._bin_sort(k, ps, between)
        if sync:
            M = int(self.M_dev[k].item())
            if M > ps.capacity:
                # grow (once per new high-water mark) and redo the sort
                ps.alloc(int(min(M * 5 // 4 + 1024, (1 << 31) - 1)))
                self.pair_capacity = max(self.pair_capacity, ps.capacity)
                self._bin_sort(k, ps)
            vw.num_pairs = M

    def _bin_sort(self, k, ps, between=None):
        vw = self.views[k]
        vw.num_pairs = None
        self._set_cap[k] = ps.capacity
        args = (self.vproj[k], self.n, self.vis_idx[k], self.vis_count[k:k + 1], vw.W, vw.H, ps.keys, ps.vals,
                ps.capacity, self.M_dev[k:k + 1], vw.ranges, ps.ws_sort, vw.order)
        if between is None:
            gs_bin_sort_async(*args, proj_bin=self.vbin[k])
        else:
            gs_bin_sort_async(*args, proj_bin=self.vbin[k], part=GS_BIN_DEPTH)
            between()
            gs_bin_sort_async(*args, proj_bin=self.vbin[k], part=GS_BIN_PAIRS)

    def _pair_bound(self, k):
        vw = self.views[k]
        return vw.num_pairs if vw.num_pairs is not None else self.sets[k % self.nsets].capacity

    def render_view(self, k):
        """Forward raster and loss of a prepared view."""
        self.render_fwd_view(k)
        self.loss_view(k)

    def render_fwd_view(self, k):
        vw = self.views[k]
        ps = self.sets[k % self.nsets]
        with self._stage("render_fwd"):
            gs_render_fwd(self.vproj[k], self.n, ps.vals, vw.ranges, self._pair_bound(k), vw.W, vw.H, vw.image, vw.T_final,
                          vw.last, vw.tile_processed if self.record_tiles else None, vw.order, self._split(k),
                          self.seg[k])

    def loss_view(self, k):
        vw = self.views[k]
        with self._stage("loss"):
            gs_loss(vw.image, vw.target, vw.W, vw.H, self.w_l1, self.w_ssim, vw.loss, vw.dL, self.ws_loss)

    def forward_view(self, k):
        self.prepare_view(k)
        self.render_view(k)

    def backward_view(self, k, keep_grad2d=False):
        """Raster backward; unless keep_grad2d, the projection backward is
        chained on in the same call (the view's parameter gradients added
        to the gradient planes, the screen-space buffer left zero)."""
        vw = self.views[k]
        ps = self.sets[k % self.nsets]
        self._gcur = self._gbuf(k)
        # (the densification statistic reads the screen-space gradients
        # before the projection backward re-zeroes them)
        chain = not keep_grad2d and self.dens_accum is None
        pg = (self.params, self.ld, vw.cam, self.vis_idx[k], self.vis_count[k:k + 1], self.grads) if chain else None
        # a view whose screen-space rows go to the fused Adam pass marks
        # the rows it reaches in its slot of the touched map
        fused = keep_grad2d and k >= self.nfirst and self._touched_on()
        with self._stage("render_bwd+project_bwd" if chain else "render_bwd", k):
            gs_render_bwd(self.vproj[k], self.n, ps.vals, vw.ranges, self._pair_bound(k), vw.W, vw.H, vw.T_final, vw.last,
                          vw.dL, self.g2d[self._gcur], vw.order, self._split(k), self.seg[k], param_grads=pg,
                          visits=None if self.visits is None else self.visits[k:k + 1],
                          touched=self.touched if fused else None, touched_slot=k - self.nfirst if fused else 0)
        if self.dens_accum is not None:
            gs_densify_stats(self.g2d[self._gcur], self.vis_idx[k], self.vis_count[k:k + 1], self.n,
                             self.dens_accum, self.dens_denom)
            if not keep_grad2d:
                self.project_view(k)

    def project_view(self, k):
        vw = self.views[k]
        with self._stage("project_bwd"):
            gs_project_bwd(self.params, self.n, self.ld, vw.cam, self.vis_idx[k], self.vis_count[k:k + 1],
                           self.g2d[self._gbuf(k)], self.grads)

    def run_views(self, defer_projection=False):
        """Every view of the batch, gradients accumulated: view k + 1 is
        prepared on the side stream and view k's projection backward runs on
        the gradient stream while the current stream renders and
        back-propagates through the rasteriser.  Nothing blocks until every
        view is issued; then the pair counts are read, and a view that
        overflowed its buffer set makes the whole batch run again with the
        set grown.  With defer_projection the screen-space gradients of the
        last ndefer views are left for adam(fused=True)."""
        stat0 = None
        if self.dens_accum is not None:
            stat0 = (self.dens_accum.clone(), self.dens_denom.clone())
        while True:
            self._issue_views(defer_projection)
            self._counts_read.synchronize()
            M = self.M_host.tolist()
            over = [k for k in range(len(self.views)) if M[k] > self._set_cap[k]]
            for k, vw in enumerate(self.views):
                vw.num_pairs = M[k]
            if not over:
                return
            for k in over:
                ps = self.sets[k % self.nsets]
                if M[k] > ps.capacity:
                    ps.alloc(int(min(M[k] * 5 // 4 + 1024, (1 << 31) - 1)))
                    self.pair_capacity = max(self.pair_capacity, ps.capacity)
            torch.cuda.current_stream(self.device).synchronize()
            self.grads.zero_()
            for g2 in self.g2d:
                g2.zero_()
            self.touched.zero_()
            if stat0 is not None:
                self.dens_accum.copy_(stat0[0])
                self.dens_denom.copy_(stat0[1])

    def preprocess_views(self, ks):
        """The preprocess of views ``ks`` in one pass over the parameters per
        GS_MAX_PREPROCESS_VIEWS of them (records, visible lists, counts, the
        union flags) on the current stream."""
        ks = list(ks)
        with self._stage("preprocess_views"):
            for i in range(0, len(ks), GS_MAX_PREPROCESS_VIEWS):
                grp = ks[i:i + GS_MAX_PREPROCESS_VIEWS]
                k0 = grp[0]
                assert grp == list(range(k0, k0 + len(grp))), "consecutive views"
                gs_preprocess_views(self.params, self.n, self.ld, [self.views[k].cam for k in grp],
                                    [self.vproj[k] for k in grp], [self.vis_idx[k] for k in grp],
                                    self.vis_count[k0:k0 + len(grp)], self.union_flags, self.ws_pre_views,
                                    max_workgroups=self.preprocess_workgroups,
                                    proj_bin=[self.vbin[k] for k in grp])

    def _issue_views(self, defer):
        main = torch.cuda.current_stream(self.device)
        nv = len(self.views)
        proj_done = [None, None]
        start = torch.cuda.Event()
        start.record(main)
        # (the batch preprocess waits for the first view's depth sort: the
        # sort's latency-bound kernels run at full speed first, and the
        # preprocess then streams beside the pairs' generation)
        depth_done = torch.cuda.Event()
        after_depth = self.preprocess_after_depth and nv > 1 and not self.preprocess_after_first
        self.prepare_view(0, sync=False, between=(lambda: depth_done.record(main)) if after_depth else None)
        first_done = torch.cuda.Event()
        first_done.record(main)
        pre_done = None
        if nv > 1:
            # the other views' preprocess, one pass over the parameters, on
            # the side stream beside the first view's binning
            with torch.cuda.stream(self.side):
                self.side.wait_event(first_done if self.preprocess_after_first else
                                     (depth_done if after_depth else start))
                self.preprocess_views(range(1, nv))
                pre_done = torch.cuda.Event()
                pre_done.record(self.side)
        # views 1, 2, 3, ... are binned on the side streams in turn, so two
        # binnings (sets k + 1 and k + 2) can run beside view k
        sides = self.sides[:max(1, min(len(self.sides), self.nsets - 1))]
        bin_done = [None] * len(sides)
        for k in range(nv):
            self.render_view(k)
            if k < self.nfirst and proj_done[k % 2] is not None:
                main.wait_event(proj_done[k % 2])          # buffer re-zeroed by view k - 2's projection
            self.backward_view(k, keep_grad2d=True)
            project = not (defer and k >= self.nfirst)
            # the set's last reader is this raster backward (the projection
            # backward reads params, not the set); an event marks it only
            # when a later view of this batch takes the set (a later batch's
            # side-stream work starts behind this batch's optimiser pass)
            raster_done = None
            if project or k + self.nsets < nv:
                raster_done = torch.cuda.Event()
                raster_done.record(main)
            if project:
                with torch.cuda.stream(self.gstream):
                    self.gstream.wait_event(raster_done)
                    self.project_view(k)
                    done = torch.cuda.Event()
                    done.record(self.gstream)
                proj_done[k % 2] = done
            self._free[k % self.nsets] = raster_done if k + self.nsets < nv else None
            if k + 1 < nv:
                sd = sides[k % len(sides)]
                with torch.cuda.stream(sd):
                    if k < len(sides):
                        sd.wait_event(first_done)              # the first view's binning goes first
                        if sd is not self.side:
                            sd.wait_event(pre_done)
                    prev = self._free[(k + 1) % self.nsets]
                    if prev is not None:
                        sd.wait_event(prev)
                    self.prepare_view(k + 1, sync=False, preprocess=False)
                    ready = torch.cuda.Event()
                    ready.record(sd)
                    bin_done[k % len(sides)] = ready
                main.wait_event(ready)
        # pair counts to the host, after the last binning
        with torch.cuda.stream(self.side):
            self.side.wait_event(first_done)
            for ev in bin_done[1:]:
                if ev is not None:
                    self.side.wait_event(ev)
            self.M_host.copy_(self.M_dev, non_blocking=True)
            self._counts_read = torch.cuda.Event()
            self._counts_read.record(self.side)
        # every projection backward issued is done before the optimiser
        for ev in proj_done:
            if ev is not None:
                main.wait_event(ev)

    def adam(self, fused=False):
        """Sparse Adam over the union; with fused, the projection backward
        of the last ndefer views (left by run_views(defer_projection=True))
        runs in the same pass."""
        self.t += 1
        bc1 = 1.0 - self.beta1 ** self.t
        bc2 = 1.0 - self.beta2 ** self.t
        with self._stage("sparse_adam"):
            if fused:
                ks = range(self.nfirst, len(self.views))
                nxt = {}
                if self.fuse_next_preprocess:
                    # (view 0's records hold a preprocess of this batch's
                    # parameters: rows outside the union are invisible
                    # there, tiles 0)
                    if self._pre0:
                        self.next_flags.zero_()
                    nxt = dict(next_cam=self.views[0].cam, next_proj=self.vproj[0], next_flags=self.next_flags,
                               next_proj_bin=self.vbin[0])
                gs_project_bwd_adam(self.params, self.grads if self.nfirst > 0 else None, self.m, self.v, self.n,
                                    self.ld, [self.views[k].cam for k in ks], [self.g2d[self._gbuf(k)] for k in ks],
                                    self.union_flags, self.union_idx, self.union_count, self.lr, self.beta1,
                                    self.beta2, self.eps, bc1, bc2, self.ws_adam,
                                    touched=self.touched if self._touched_on() else None, **nxt)
                self._pre0 = bool(nxt)
            else:
                gs_sparse_adam(self.params, self.grads, self.m, self.v, self.n, self.ld, self.union_flags,
                               self.union_idx, self.union_count, self.lr, self.beta1, self.beta2, self.eps, bc1,
                               bc2, self.ws_adam)

    def step(self):
        """One training step: for each view preprocess, bin/sort, render,
        loss, backward (gradients accumulate); then sparse Adam, fused with
        the projection backward of the last ndefer views."""
        self.run_views(defer_projection=True)
        self.adam(fused=True)

    # -- training state ------------------------------------------------------
    def state(self):
        """Device copies of the training state: parameters, both Adam
        moments and the step count (what a checkpoint holds)."""
        return dict(params=self.params.clone(), m=self.m.clone(), v=self.v.clone(), t=self.t)

    def save_checkpoint(self, path):
        """Write the training state (parameters, Adam moments, step count)
        to `path` (tensors only, loadable without unpickling code)."""
        torch.cuda.current_stream(self.device).synchronize()
        torch.save({"params": self.params.cpu(), "m": self.m.cpu(), "v": self.v.cpu(),
                    "t": torch.tensor(self.t, dtype=torch.int64)}, path)

    def load_checkpoint(self, path):
        """Continue from save_checkpoint's file (the same Gaussian count)."""
        ck = torch.load(path, map_location="cpu", weights_only=True)
        assert ck["params"].shape == self.params.shape, "checkpoint of another Gaussian count"
        self.load_state({"params": ck["params"].to(self.device), "m": ck["m"].to(self.device),
                         "v": ck["v"].to(self.device), "t": int(ck["t"])})

    # -- densification ------------------------------------------------------
    def track_densify(self):
        """Start (or restart from zero) the densification statistic: every
        raster backward from now on adds its visible rows' |dL/d(u, v)| and a
        count (gs_densify_stats), before the projection backward consumes
        the screen-space gradients."""
        rows = max(self.n, 1)
        self.dens_accum = torch.zeros(rows, dtype=torch.float32, device=self.device)
        self.dens_denom = torch.zeros(rows, dtype=torch.int32, device=self.device)

    def densify(self, grad_threshold, log_scale_threshold, logit_threshold, normals=None, seed=0,
                log_shrink=math.log(1.6)):
        """Clone / split / prune from the statistic gathered since
        track_densify (gs_densify), then continue with the new Gaussians:
        every per-Gaussian buffer is rebuilt for the new count, kept
        Gaussians keep their Adam moments, new ones start from zero, the
        statistic restarts from zero and the step count carries on.
        `normals` ([2][3][n] device fp32 standard normals) are the split
        children's random offsets; drawn from `seed` when not given.
        Returns the new Gaussian count."""
        assert self.dens_accum is not None, "track_densify() first"
        n = self.n
        if normals is None:
            gen = torch.Generator(device=self.device)
            gen.manual_seed(int(seed))
            normals = torch.randn((2, 3, max(n, 1)), generator=gen, device=self.device, dtype=torch.float32)
        ld_out = max(2 * n, 1)
        out = [torch.empty((59, ld_out), dtype=torch.float32, device=self.device) for _ in range(3)]
        out_n = torch.zeros(1, dtype=torch.int64, device=self.device)
        ws = _bytes(gs_workspace_size(GS_OP_DENSIFY, n), self.device)
        gs_densify(self.params, self.m, self.v, n, self.ld, self.dens_accum, self.dens_denom, normals,
                   float(grad_threshold), float(log_scale_threshold), float(logit_threshold), float(log_shrink),
                   out[0], out[1], out[2], ld_out, out_n, ws)
        n_new = int(out_n.item())
        p, m, v = (o[:, :n_new].contiguous() for o in out)
        del out
        self._alloc_rows(p, m, v)
        self._pre0 = False
        return n_new

    def load_state(self, st):
        """Continue from a state(): parameters and moments copied in, the
        step count restored; what the last Adam pass left for the next
        step's first view (records, visibility bytes, union flags) is
        dropped, so that view is projected afresh."""
        torch.cuda.current_stream(self.device).synchronize()
        self.params.copy_(st["params"])
        self.m.copy_(st["m"])
        self.v.copy_(st["v"])
        self.t = int(st["t"])
        self.grads.zero_()
        for g2 in self.g2d:
            g2.zero_()
        self.touched.zero_()
        self.union_flags.zero_()
        self.next_flags.zero_()
        self._pre0 = False


def from_workload(work, device="cuda", **kw) -> TrainStep:
    """TrainStep for a ``synth.Workload``."""
    return TrainStep(work.params, work.cameras, work.targets, work.w_l1, work.w_ssim, work.lr, work.beta1,
                     work.beta2, work.eps, device=device, **kw)
