// C-ABI layer of libgs: argument checks, workspace carving, stream plumbing
// and the status/error strings.  Every check runs on the host before any
// work is enqueued, so a GS_ERR_INVALID_ARG call has launched nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/gs.h"
#include "gs_internal.h"

static_assert(GS_MAX_FUSED_VIEWS == gs::kMaxFusedViews, "fused view limit");
static_assert(GS_MAX_PREPROCESS_VIEWS == gs::kMaxPreprocessViews, "preprocess view limit");
static_assert(GS_MAX_COUPLED_VIEWS == gs::kMaxCoupledViews, "coupled view limit");
static_assert(GS_MAX_TILE_BLOCKS == gs::kMaxTileBlocks, "tile block limit");
static_assert(GS_MAX_PARTITION_TILES == gs::kMaxPartitionTiles, "partition tile limit");

namespace {

thread_local char g_err[512] = "";

gs_status fail(gs_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

gs_status ok() {
  g_err[0] = '\0';
  return GS_OK;
}

gs_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return ok();
  return fail(GS_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int32_t kMaxDim = 65535 * 16;   // tile coordinates are stored in 16 bits

gs_status check_camera(const gs_camera* cam, gs::CamArgs& out) {
  if (cam == nullptr) return fail(GS_ERR_INVALID_ARG, "camera is NULL");
  if (cam->width <= 0 || cam->height <= 0 || cam->width > kMaxDim || cam->height > kMaxDim)
    return fail(GS_ERR_INVALID_ARG, "camera size %dx%d out of range", cam->width, cam->height);
  const float fs[] = {cam->fx, cam->fy, cam->cx, cam->cy, cam->near_z};
  for (float f : fs)
    if (!std::isfinite(f)) return fail(GS_ERR_INVALID_ARG, "camera intrinsics not finite");
  for (int k = 0; k < 9; ++k) out.R[k] = cam->R[k];
  for (int k = 0; k < 3; ++k) {
    out.t[k] = cam->t[k];
    out.campos[k] = cam->campos[k];
  }
  out.fx = cam->fx;
  out.fy = cam->fy;
  out.cx = cam->cx;
  out.cy = cam->cy;
  out.near_z = cam->near_z;
  out.width = cam->width;
  out.height = cam->height;
  out.tiles_x = (cam->width + 15) / 16;
  out.tiles_y = (cam->height + 15) / 16;
  return GS_OK;
}

gs_status check_size(int32_t width, int32_t height) {
  if (width <= 0 || height <= 0 || width > kMaxDim || height > kMaxDim)
    return fail(GS_ERR_INVALID_ARG, "image size %dx%d out of range", width, height);
  return GS_OK;
}

// The split backward's workspace (its size for the image) and segment
// length (a power of two, 64 ... 65536); both ignored without a workspace.
gs_status check_split(const void* ws, size_t ws_bytes, int32_t width, int32_t height, int32_t segment_len,
                      int& seg_shift) {
  seg_shift = 6;
  if (ws == nullptr) return GS_OK;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(GS_ERR_INVALID_ARG, "split_ws not 256-byte aligned");
  const size_t need = gs::raster_split_bytes(width, height);
  if (ws_bytes < need)
    return fail(GS_ERR_INVALID_ARG, "split_ws_bytes = %zu < %zu needed for %dx%d", ws_bytes, need, width, height);
  if (segment_len < 64 || segment_len > 65536 || (segment_len & (segment_len - 1)) != 0)
    return fail(GS_ERR_INVALID_ARG, "segment_len = %d: not a power of two in [64, 65536]", int(segment_len));
  seg_shift = __builtin_ctz(uint32_t(segment_len));
  return GS_OK;
}

#define REQUIRE(cond, ...)                                   \
  do {                                                       \
    if (!(cond)) return fail(GS_ERR_INVALID_ARG, __VA_ARGS__); \
  } while (0)

#define CHECK(expr)                          \
  do {                                       \
    const gs_status s_ = (expr);             \
    if (s_ != GS_OK) return s_;              \
  } while (0)

gs::SsimWindow make_window() {
  gs::SsimWindow w;
  double g[11], s = 0.0;
  for (int k = 0; k < 11; ++k) {
    g[k] = std::exp(-double((k - 5) * (k - 5)) / (2.0 * 1.5 * 1.5));
    s += g[k];
  }
  for (int k = 0; k < 11; ++k) w.g[k] = float(g[k] / s);
  return w;
}

size_t adam_ws_bytes(int64_t n) { return gs::compact_ws_bytes(n); }

}  // namespace

// The scratch of gs_sparse_adam_noalloc.  In host code `scratch` names a
// host-side stand-in, not device memory: kernels get the address that
// hipGetSymbolAddress returns for the current device (each device holds its
// own copy), taken once per device and kept in g_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[GS_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// The device address of `scratch` on the current device (looked up on the
// first call on that device).
gs_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "gs_sparse_adam_noalloc (hipGetDevice)");
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(GS_ERR_HIP, "gs_sparse_adam_noalloc: device %d beyond the %d the library tracks", dev,
                kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "gs_sparse_adam_noalloc (hipGetSymbolAddress)");
    if (p == nullptr) return fail(GS_ERR_HIP, "gs_sparse_adam_noalloc: NULL scratch address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GS_OK;
}

}  // namespace

extern "C" {

const char* gs_status_string(int status) {
  switch (status) {
    case GS_OK: return "GS_OK";
    case GS_ERR_INVALID_ARG: return "GS_ERR_INVALID_ARG: invalid argument";
    case GS_ERR_CAPACITY: return "GS_ERR_CAPACITY: pair capacity exceeded";
    case GS_ERR_HIP: return "GS_ERR_HIP: HIP runtime error";
    default: return "unknown gs_status";
  }
}

const char* gs_last_error(void) { return g_err; }

int gs_version(void) { return 1; }

gs_status gs_workspace_size(gs_op op, int64_t n, int32_t width, int32_t height, int64_t pair_capacity,
                            size_t* bytes) {
  REQUIRE(bytes != nullptr, "bytes is NULL");
  switch (op) {
    case GS_OP_PREPROCESS:
      REQUIRE(n >= 0 && n < (int64_t(1) << 31), "n = %lld out of range", (long long)n);
      *bytes = gs::preprocess_ws_bytes(n);
      return ok();
    case GS_OP_BIN_SORT:
      REQUIRE(n >= 0 && n < (int64_t(1) << 31), "n = %lld out of range", (long long)n);
      REQUIRE(pair_capacity >= 0 && pair_capacity < (int64_t(1) << 31), "pair_capacity out of range");
      *bytes = gs::binsort_ws_bytes(n, pair_capacity);
      return ok();
    case GS_OP_LOSS:
      CHECK(check_size(width, height));
      *bytes = gs::loss_ws_bytes(width, height);
      return ok();
    case GS_OP_SPARSE_ADAM:
      REQUIRE(n >= 0 && n < (int64_t(1) << 31), "n = %lld out of range", (long long)n);
      *bytes = adam_ws_bytes(n);
      return ok();
    case GS_OP_RASTER:
      CHECK(check_size(width, height));
      *bytes = gs::raster_split_bytes(width, height);
      return ok();
    case GS_OP_PREPROCESS_VIEWS:
      REQUIRE(n >= 0 && n < (int64_t(1) << 31), "n = %lld out of range", (long long)n);
      REQUIRE(width >= 1 && width <= GS_MAX_PREPROCESS_VIEWS, "num_views = %d out of range", width);
      *bytes = gs::preprocess_views_ws_bytes(n, width);
      return ok();
    case GS_OP_DENSIFY:
      REQUIRE(n >= 0 && n < (int64_t(1) << 30), "n = %lld out of range", (long long)n);
      *bytes = gs::densify_ws_bytes(n);
      return ok();
    case GS_OP_PACK:
      REQUIRE(n >= 0 && n < (int64_t(1) << 31), "n = %lld out of range", (long long)n);
      REQUIRE(width >= 1 && width <= GS_MAX_TILE_BLOCKS, "num_blocks = %d out of range", width);
      *bytes = gs::pack_ws_bytes(n, width);
      return ok();
    case GS_OP_VIEW_OVERLAP:
      REQUIRE(n >= 0 && n < (int64_t(1) << 31), "n = %lld out of range", (long long)n);
      REQUIRE(width >= 0 && width <= GS_MAX_COUPLED_VIEWS, "num_views = %d out of range", width);
      *bytes = gs::coupling_ws_bytes(n, width);
      return ok();
  }
  return fail(GS_ERR_INVALID_ARG, "unknown op %d", int(op));
}

gs_status gs_preprocess(const float* params, int64_t n, int64_t ld, const gs_camera* cam, float* proj,
                        float* proj_bin, int32_t* vis_idx, int64_t* vis_count, uint8_t* union_flags, void* workspace,
                        size_t workspace_bytes, void* stream) {
  gs::CamArgs c;
  CHECK(check_camera(cam, c));
  REQUIRE(n >= 0 && n < GS_MAX_PLANE_ROWS, "n = %lld out of range", (long long)n);
  REQUIRE(ld >= n, "ld < n");
  REQUIRE(vis_count != nullptr, "vis_count is NULL");
  if (n > 0) {
    REQUIRE(params && proj && vis_idx, "NULL array");
    REQUIRE(aligned(proj, 16) && aligned(params, 4) && aligned(vis_idx, 4), "misaligned array");
  }
  REQUIRE(proj_bin == nullptr || aligned(proj_bin, 16), "proj_bin not 16-byte aligned");
  REQUIRE(union_flags == nullptr || aligned(union_flags, 16), "union_flags not 16-byte aligned");
  REQUIRE(workspace != nullptr && aligned(workspace, 256), "workspace NULL or not 256-byte aligned");
  REQUIRE(workspace_bytes >= gs::preprocess_ws_bytes(n), "workspace too small");
  return hip_status(gs::launch_preprocess(params, n, ld, c, proj, proj_bin, vis_idx, vis_count, union_flags,
                                          workspace, static_cast<hipStream_t>(stream)),
                    "gs_preprocess");
}

gs_status gs_preprocess_views(const float* params, int64_t n, int64_t ld, const gs_camera* cams, int32_t num_views,
                              float* const* proj, float* const* proj_bin, int32_t* const* vis_idx,
                              int64_t* vis_count, uint8_t* union_flags, int32_t max_workgroups, void* workspace,
                              size_t workspace_bytes, void* stream) {
  REQUIRE(num_views >= 1 && num_views <= GS_MAX_PREPROCESS_VIEWS, "num_views = %d outside [1, %d]", int(num_views),
          GS_MAX_PREPROCESS_VIEWS);
  REQUIRE(cams != nullptr && proj != nullptr && vis_idx != nullptr, "cams / proj / vis_idx NULL");
  gs::CamArgs c[gs::kMaxPreprocessViews];
  for (int32_t w = 0; w < num_views; ++w) CHECK(check_camera(cams + w, c[w]));
  REQUIRE(n >= 0 && n < GS_MAX_PLANE_ROWS, "n = %lld out of range", (long long)n);
  REQUIRE(ld >= n, "ld < n");
  REQUIRE(vis_count != nullptr && aligned(vis_count, 8), "vis_count NULL or misaligned");
  if (n > 0) {
    REQUIRE(params != nullptr && aligned(params, 4), "params NULL or misaligned");
    for (int32_t w = 0; w < num_views; ++w) {
      REQUIRE(proj[w] != nullptr && aligned(proj[w], 16), "proj[%d] NULL or not 16-byte aligned", int(w));
      REQUIRE(vis_idx[w] != nullptr && aligned(vis_idx[w], 4), "vis_idx[%d] NULL or misaligned", int(w));
    }
  }
  if (proj_bin != nullptr)
    for (int32_t w = 0; w < num_views; ++w)
      REQUIRE(proj_bin[w] == nullptr || aligned(proj_bin[w], 16), "proj_bin[%d] not 16-byte aligned", int(w));
  REQUIRE(union_flags == nullptr || aligned(union_flags, 16), "union_flags not 16-byte aligned");
  REQUIRE(max_workgroups >= 0, "max_workgroups = %d < 0", int(max_workgroups));
  REQUIRE(workspace != nullptr && aligned(workspace, 256), "workspace NULL or not 256-byte aligned");
  REQUIRE(workspace_bytes >= gs::preprocess_views_ws_bytes(n, num_views), "workspace too small");
  return hip_status(gs::launch_preprocess_views(params, n, ld, c, num_views, proj, proj_bin, vis_idx, vis_count,
                                                union_flags, max_workgroups, workspace,
                                                static_cast<hipStream_t>(stream)),
                    "gs_preprocess_views");
}

gs_status gs_bin_sort(const float* proj, const float* proj_bin, int64_t n, const int32_t* vis_idx,
                      const int64_t* vis_count,
                      int32_t width, int32_t height, uint64_t* keys, int32_t* vals, int64_t pair_capacity,
                      int64_t* num_pairs, uint32_t* tile_ranges, uint32_t* tile_order, void* workspace,
                      size_t workspace_bytes, void* stream) {
  CHECK(check_size(width, height));
  REQUIRE(n >= 0 && n < (int64_t(1) << 31), "n = %lld out of range", (long long)n);
  REQUIRE(pair_capacity >= 0 && pair_capacity < (int64_t(1) << 31), "pair_capacity out of range");
  REQUIRE(vis_count != nullptr && num_pairs != nullptr && tile_ranges != nullptr, "NULL argument");
  if (n > 0) REQUIRE(proj && vis_idx && aligned(proj, 16), "NULL or misaligned proj / vis_idx");
  REQUIRE(proj_bin == nullptr || aligned(proj_bin, 16), "proj_bin not 16-byte aligned");
  if (pair_capacity > 0)
    REQUIRE(vals && (keys ? aligned(keys, 8) : gs::binsort_keys_optional((width + 15) / 16, (height + 15) / 16)),
            "NULL or misaligned keys / vals (keys may be NULL only up to 256 x 256 tiles)");
  REQUIRE(workspace != nullptr && aligned(workspace, 256), "workspace NULL or not 256-byte aligned");
  REQUIRE(workspace_bytes >= gs::binsort_ws_bytes(n, pair_capacity), "workspace too small");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int32_t TX = (width + 15) / 16, TY = (height + 15) / 16;
  hipError_t e =
      gs::launch_binsort_stage1(proj, proj_bin, n, vis_idx, vis_count, TX, TY, nullptr, workspace, pair_capacity,
                                st);
  if (e != hipSuccess) return hip_status(e, "gs_bin_sort (depth sort)");
  int64_t M = 0;
  e = hipMemcpyAsync(&M, gs::binsort_count_ptr(workspace, n, pair_capacity), sizeof(int64_t), hipMemcpyDeviceToHost,
                     st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_status(e, "gs_bin_sort (pair count)");
  *num_pairs = M;
  if (M > pair_capacity)
    return fail(GS_ERR_CAPACITY, "%lld pairs > capacity %lld", (long long)M, (long long)pair_capacity);
  e = gs::launch_binsort_stage2(proj, n, vis_idx, vis_count, M, TX, TY, keys, vals, tile_ranges, tile_order,
                                workspace, pair_capacity, st);
  return hip_status(e, "gs_bin_sort");
}

gs_status gs_bin_sort_async(const float* proj, const float* proj_bin, int64_t n, const int32_t* vis_idx,
                            const int64_t* vis_count,
                            int32_t width, int32_t height, uint64_t* keys, int32_t* vals, int64_t pair_capacity,
                            int64_t* num_pairs_dev, uint32_t* tile_ranges, uint32_t* tile_order, void* workspace,
                            size_t workspace_bytes, int32_t part, void* stream) {
  CHECK(check_size(width, height));
  REQUIRE(part == GS_BIN_ALL || part == GS_BIN_DEPTH || part == GS_BIN_PAIRS, "part = %d is not a binning part",
          int(part));
  REQUIRE(n >= 0 && n < (int64_t(1) << 31), "n = %lld out of range", (long long)n);
  REQUIRE(pair_capacity >= 0 && pair_capacity < (int64_t(1) << 31), "pair_capacity out of range");
  REQUIRE(vis_count != nullptr && num_pairs_dev != nullptr && tile_ranges != nullptr, "NULL argument");
  REQUIRE(aligned(num_pairs_dev, 8), "misaligned num_pairs_dev");
  if (n > 0) REQUIRE(proj && vis_idx && aligned(proj, 16), "NULL or misaligned proj / vis_idx");
  REQUIRE(proj_bin == nullptr || aligned(proj_bin, 16), "proj_bin not 16-byte aligned");
  if (pair_capacity > 0)
    REQUIRE(vals && (keys ? aligned(keys, 8) : gs::binsort_keys_optional((width + 15) / 16, (height + 15) / 16)),
            "NULL or misaligned keys / vals (keys may be NULL only up to 256 x 256 tiles)");
  REQUIRE(workspace != nullptr && aligned(workspace, 256), "workspace NULL or not 256-byte aligned");
  REQUIRE(workspace_bytes >= gs::binsort_ws_bytes(n, pair_capacity), "workspace too small");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int32_t TX = (width + 15) / 16, TY = (height + 15) / 16;
  hipError_t e = hipSuccess;
  if (part != GS_BIN_PAIRS) {
    e = gs::launch_binsort_stage1(proj, proj_bin, n, vis_idx, vis_count, TX, TY, num_pairs_dev, workspace,
                                  pair_capacity, st);
    if (e != hipSuccess) return hip_status(e, "gs_bin_sort_async (depth sort)");
  }
  if (part != GS_BIN_DEPTH)
    e = gs::launch_binsort_stage2(proj, n, vis_idx, vis_count, -1, TX, TY, keys, vals, tile_ranges, tile_order,
                                  workspace, pair_capacity, st);
  return hip_status(e, "gs_bin_sort_async");
}

gs_status gs_render_fwd(const float* proj, int64_t n, const int32_t* vals, const uint32_t* tile_ranges,
                        const uint32_t* tile_order, int64_t num_pairs, int32_t width, int32_t height, float* image,
                        float* T_final, uint32_t* last, uint32_t* tile_processed, void* split_ws,
                        size_t split_ws_bytes, int32_t segment_len, void* stream) {
  CHECK(check_size(width, height));
  REQUIRE(n >= 0 && num_pairs >= 0 && num_pairs < (int64_t(1) << 31), "n / num_pairs out of range");
  REQUIRE(tile_ranges && image && T_final && last, "NULL output or tile_ranges");
  if (num_pairs > 0) REQUIRE(proj && vals && aligned(proj, 16), "NULL or misaligned proj / vals");
  int seg_shift = 0;
  CHECK(check_split(split_ws, split_ws_bytes, width, height, segment_len, seg_shift));
  return hip_status(gs::launch_render_fwd(proj, vals, tile_ranges, tile_order, num_pairs, width, height, image,
                                          T_final, last, tile_processed, split_ws, seg_shift,
                                          static_cast<hipStream_t>(stream)),
                    "gs_render_fwd");
}

gs_status gs_loss(const float* image, const float* target, int32_t width, int32_t height, float w_l1,
                  float w_ssim, float* loss, float* dL_dimage, void* workspace, size_t workspace_bytes,
                  void* stream) {
  CHECK(check_size(width, height));
  REQUIRE(image && target && loss && dL_dimage, "NULL argument");
  REQUIRE(std::isfinite(w_l1) && std::isfinite(w_ssim), "loss weights not finite");
  REQUIRE(workspace != nullptr && aligned(workspace, 256), "workspace NULL or not 256-byte aligned");
  REQUIRE(workspace_bytes >= gs::loss_ws_bytes(width, height), "workspace too small");
  static const gs::SsimWindow win = make_window();
  return hip_status(gs::launch_loss(image, target, width, height, w_l1, w_ssim, win, loss, dL_dimage, workspace,
                                    static_cast<hipStream_t>(stream)),
                    "gs_loss");
}

gs_status gs_render_bwd(const float* proj, int64_t n, const int32_t* vals, const uint32_t* tile_ranges,
                        const uint32_t* tile_order, int64_t num_pairs, int32_t width, int32_t height,
                        const float* T_final, const uint32_t* last, const float* dL_dimage, float* grad2d,
                        const void* split_ws, size_t split_ws_bytes, int32_t segment_len,
                        const gs_param_grads* param_grads, uint64_t* visits, uint8_t* touched,
                        int32_t touched_slot, void* stream) {
  CHECK(check_size(width, height));
  REQUIRE(n >= 0 && n < (int64_t(1) << 31), "n = %lld out of range", (long long)n);
  REQUIRE(num_pairs >= 0 && num_pairs < (int64_t(1) << 31), "num_pairs out of range");
  REQUIRE(tile_ranges && T_final && last && dL_dimage, "NULL argument");
  if (num_pairs > 0 || (param_grads != nullptr && n > 0)) {
    REQUIRE(grad2d != nullptr && aligned(grad2d, 16), "grad2d NULL or not 16-byte aligned");
  }
  if (num_pairs > 0) REQUIRE(proj && vals && aligned(proj, 16), "NULL or misaligned proj / vals");
  REQUIRE(visits == nullptr || aligned(visits, 8), "visits not 8-byte aligned");
  if (touched != nullptr) {
    REQUIRE(aligned(touched, 16), "touched not 16-byte aligned");
    REQUIRE(touched_slot >= 0 && touched_slot < GS_TOUCHED_SLOTS, "touched_slot = %d out of range", touched_slot);
    REQUIRE(param_grads == nullptr, "touched with param_grads (the screen-space rows are consumed in the call)");
  }
  int seg_shift = 0;
  CHECK(check_split(split_ws, split_ws_bytes, width, height, segment_len, seg_shift));
  gs::CamArgs c{};
  if (param_grads != nullptr) {
    CHECK(check_camera(param_grads->cam, c));
    REQUIRE(c.width == width && c.height == height, "param_grads->cam is %dx%d, the image %dx%d", c.width, c.height,
            width, height);
    REQUIRE(n < GS_MAX_PLANE_ROWS, "n = %lld out of range with param_grads", (long long)n);
    REQUIRE(param_grads->ld >= n, "param_grads->ld < n");
    REQUIRE(param_grads->vis_count != nullptr, "param_grads->vis_count is NULL");
    if (n > 0)
      REQUIRE(param_grads->params && param_grads->vis_idx && param_grads->grads, "NULL array in param_grads");
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = gs::launch_render_bwd(proj, vals, tile_ranges, tile_order, num_pairs, width, height, T_final, last,
                                       dL_dimage, grad2d, touched != nullptr ? touched + touched_slot : nullptr,
                                       split_ws, seg_shift, visits, st);
  if (e == hipSuccess && param_grads != nullptr)
    e = gs::launch_project_bwd(param_grads->params, n, param_grads->ld, c, param_grads->vis_idx,
                               param_grads->vis_count, grad2d, param_grads->grads, st);
  return hip_status(e, "gs_render_bwd");
}

gs_status gs_project_bwd(const float* params, int64_t n, int64_t ld, const gs_camera* cam, const int32_t* vis_idx,
                         const int64_t* vis_count, float* grad2d, float* grads, void* stream) {
  gs::CamArgs c;
  CHECK(check_camera(cam, c));
  REQUIRE(n >= 0 && n < GS_MAX_PLANE_ROWS, "n = %lld out of range", (long long)n);
  REQUIRE(ld >= n, "ld < n");
  REQUIRE(vis_count != nullptr, "vis_count is NULL");
  if (n > 0) {
    REQUIRE(params && vis_idx && grad2d && grads, "NULL array");
    REQUIRE(aligned(grad2d, 16), "grad2d not 16-byte aligned");
  }
  return hip_status(gs::launch_project_bwd(params, n, ld, c, vis_idx, vis_count, grad2d, grads,
                                           static_cast<hipStream_t>(stream)),
                    "gs_project_bwd");
}

gs_status gs_sparse_adam(float* params, float* grads, float* m, float* v, int64_t n, int64_t ld,
                         uint8_t* union_flags, int32_t* union_idx, int64_t* union_count, float lr, float beta1,
                         float beta2, float eps, float bias_c1, float bias_c2, void* workspace,
                         size_t workspace_bytes, void* stream) {
  REQUIRE(n >= 0 && n < GS_MAX_PLANE_ROWS, "n = %lld out of range", (long long)n);
  REQUIRE(ld >= n, "ld < n");
  REQUIRE(union_count != nullptr, "union_count is NULL");
  if (n > 0) {
    REQUIRE(params && grads && m && v && union_flags && union_idx, "NULL array");
    REQUIRE(aligned(union_flags, 16), "union_flags not 16-byte aligned");
  }
  REQUIRE(std::isfinite(lr) && std::isfinite(beta1) && std::isfinite(beta2) && std::isfinite(eps), "non-finite scalar");
  REQUIRE(bias_c1 > 0.0f && bias_c2 > 0.0f, "bias corrections must be > 0");
  REQUIRE(workspace != nullptr && aligned(workspace, 256), "workspace NULL or not 256-byte aligned");
  REQUIRE(workspace_bytes >= adam_ws_bytes(n), "workspace too small");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = gs::launch_compact(union_flags, n, union_idx, union_count, true, workspace, st);
  if (e == hipSuccess)
    e = gs::launch_sparse_adam(params, grads, m, v, n, ld, union_idx, union_count, lr, beta1, beta2, eps, bias_c1,
                               bias_c2, st);
  return hip_status(e, "gs_sparse_adam");
}

gs_status gs_sparse_adam_noalloc(float* params, float* grads, float* m, float* v, int64_t n, int64_t ld,
                                 uint8_t* union_flags, int32_t* union_idx, int64_t* union_count, float lr,
                                 float beta1, float beta2, float eps, float bias_c1, float bias_c2, void* stream) {
  REQUIRE(n >= 0 && n <= GS_NOALLOC_MAX_N, "n = %lld outside [0, %lld]: the union compaction needs %zu scratch "
          "bytes, the allocation-free entry holds %zu", (long long)n, (long long)GS_NOALLOC_MAX_N,
          adam_ws_bytes(n), size_t(GS_NOALLOC_SCRATCH_BYTES));
  REQUIRE(adam_ws_bytes(n) <= size_t(GS_NOALLOC_SCRATCH_BYTES), "n = %lld: scratch too small", (long long)n);
  REQUIRE(ld >= n, "ld < n");
  REQUIRE(union_count != nullptr, "union_count is NULL");
  if (n > 0) {
    REQUIRE(params && grads && m && v && union_flags && union_idx, "NULL array");
    REQUIRE(aligned(union_flags, 16), "union_flags not 16-byte aligned");
  }
  REQUIRE(std::isfinite(lr) && std::isfinite(beta1) && std::isfinite(beta2) && std::isfinite(eps), "non-finite scalar");
  REQUIRE(bias_c1 > 0.0f && bias_c2 > 0.0f, "bias corrections must be > 0");
  static_assert(GS_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
  void* ws = nullptr;
  CHECK(scratch_address(&ws));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // (k_count writes every block count k_scan_counts and k_write read)
  hipError_t e = gs::launch_compact(union_flags, n, union_idx, union_count, true, ws, st);
  if (e == hipSuccess)
    e = gs::launch_sparse_adam(params, grads, m, v, n, ld, union_idx, union_count, lr, beta1, beta2, eps, bias_c1,
                               bias_c2, st);
  return hip_status(e, "gs_sparse_adam_noalloc");
}

gs_status gs_project_bwd_adam(float* params, float* grads, float* m, float* v, int64_t n, int64_t ld,
                              const gs_camera* cams, int32_t num_views, float* const* grad2d, uint8_t* touched,
                              uint8_t* union_flags, int32_t* union_idx, int64_t* union_count,
                              const gs_camera* next_cam,
                              float* next_proj, float* next_proj_bin, uint8_t* next_flags, float lr, float beta1,
                              float beta2, float eps, float bias_c1, float bias_c2, void* workspace,
                              size_t workspace_bytes, void* stream) {
  REQUIRE(num_views >= 0 && num_views <= GS_MAX_FUSED_VIEWS, "num_views = %d outside [0, %d]", int(num_views),
          GS_MAX_FUSED_VIEWS);
  REQUIRE(num_views == 0 || (cams != nullptr && grad2d != nullptr), "cams / grad2d NULL");
  REQUIRE(touched == nullptr || aligned(touched, 16), "touched not 16-byte aligned");
  gs::FusedViews fv{};
  fv.count = num_views;
  fv.touched = touched;
  for (int32_t w = 0; w < num_views; ++w) {
    CHECK(check_camera(cams + w, fv.cam[w]));
    fv.grad2d[w] = grad2d[w];
  }
  REQUIRE(n >= 0 && n < GS_MAX_PLANE_ROWS, "n = %lld out of range", (long long)n);
  REQUIRE(ld >= n, "ld < n");
  REQUIRE(union_count != nullptr, "union_count is NULL");
  if (n > 0) {
    REQUIRE(params && m && v && union_flags && union_idx, "NULL array");
    REQUIRE(aligned(union_flags, 16), "union_flags not 16-byte aligned");
    for (int32_t w = 0; w < num_views; ++w)
      REQUIRE(fv.grad2d[w] != nullptr && aligned(fv.grad2d[w], 16), "grad2d[%d] NULL or not 16-byte aligned",
              int(w));
  }
  REQUIRE(std::isfinite(lr) && std::isfinite(beta1) && std::isfinite(beta2) && std::isfinite(eps), "non-finite scalar");
  REQUIRE(bias_c1 > 0.0f && bias_c2 > 0.0f, "bias corrections must be > 0");
  REQUIRE(workspace != nullptr && aligned(workspace, 256), "workspace NULL or not 256-byte aligned");
  REQUIRE(workspace_bytes >= adam_ws_bytes(n), "workspace too small");
  REQUIRE((next_cam == nullptr) == (next_proj == nullptr) && (next_cam == nullptr) == (next_flags == nullptr),
          "next_cam, next_proj and next_flags: all NULL or none");
  REQUIRE(next_cam != nullptr || next_proj_bin == nullptr, "next_proj_bin given without next_proj");
  if (next_cam != nullptr) {
    CHECK(check_camera(next_cam, fv.next));
    REQUIRE(aligned(next_proj, 16), "next_proj not 16-byte aligned");
    REQUIRE(next_proj_bin == nullptr || aligned(next_proj_bin, 16), "next_proj_bin not 16-byte aligned");
    fv.next_proj = next_proj;
    fv.next_bin = next_proj_bin;
    fv.next_flags = next_flags;
    fv.union_flags = union_flags;
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = gs::launch_compact(union_flags, n, union_idx, union_count, true, workspace, st);
  if (e == hipSuccess)
    e = gs::launch_project_adam(params, grads, m, v, n, ld, fv, union_idx, union_count, lr, beta1, beta2, eps,
                                bias_c1, bias_c2, st);
  return hip_status(e, "gs_project_bwd_adam");
}

gs_status gs_visible_list(uint8_t* flags, int64_t n, int32_t* vis_idx, int64_t* vis_count, void* workspace,
                          size_t workspace_bytes, void* stream) {
  REQUIRE(n >= 0 && n < (int64_t(1) << 31), "n = %lld out of range", (long long)n);
  REQUIRE(vis_count != nullptr, "vis_count is NULL");
  if (n > 0) REQUIRE(flags && vis_idx && aligned(flags, 16), "NULL or misaligned flags / vis_idx");
  REQUIRE(workspace != nullptr && aligned(workspace, 256), "workspace NULL or not 256-byte aligned");
  REQUIRE(workspace_bytes >= gs::compact_ws_bytes(n), "workspace too small");
  return hip_status(gs::launch_compact(flags, n, vis_idx, vis_count, true, workspace,
                                       static_cast<hipStream_t>(stream)),
                    "gs_visible_list");
}

gs_status gs_view_overlap(const int32_t* lists, int64_t ld, const int64_t* counts, int32_t num_views, int64_t n,
                          int64_t* inter, double* weights, void* workspace, size_t workspace_bytes, void* stream) {
  REQUIRE(num_views >= 0 && num_views <= GS_MAX_COUPLED_VIEWS, "num_views = %d out of range", num_views);
  REQUIRE(n >= 0 && n < (int64_t(1) << 31), "n = %lld out of range", (long long)n);
  REQUIRE(ld >= 1, "ld = %lld < 1", (long long)ld);
  if (num_views == 0) return ok();
  REQUIRE(lists != nullptr && counts != nullptr, "lists or counts is NULL");
  REQUIRE(aligned(counts, 8), "counts not 8-byte aligned");
  REQUIRE(inter != nullptr && aligned(inter, 8), "inter NULL or not 8-byte aligned");
  REQUIRE(weights == nullptr || aligned(weights, 8), "weights not 8-byte aligned");
  REQUIRE(aligned(lists, 4), "lists not 4-byte aligned");
  const size_t need = gs::coupling_ws_bytes(n, num_views);
  if (need > 0) {
    REQUIRE(workspace != nullptr && aligned(workspace, 256), "workspace NULL or not 256-byte aligned");
    REQUIRE(workspace_bytes >= need, "workspace too small (%zu < %zu)", workspace_bytes, need);
  }
  return hip_status(gs::launch_view_overlap(lists, ld, counts, num_views, n, inter, weights, workspace,
                                            static_cast<hipStream_t>(stream)),
                    "gs_view_overlap");
}

gs_status gs_view_priority(const double* weights, int32_t num_views, const int32_t* prev, int32_t num_prev,
                           double* score, void* stream) {
  REQUIRE(num_views >= 0 && num_views <= GS_MAX_COUPLED_VIEWS, "num_views = %d out of range", num_views);
  REQUIRE(num_prev >= 0, "num_prev = %d < 0", num_prev);
  if (num_views == 0) return ok();
  REQUIRE(weights != nullptr && aligned(weights, 8), "weights NULL or not 8-byte aligned");
  REQUIRE(score != nullptr && aligned(score, 8), "score NULL or not 8-byte aligned");
  REQUIRE(num_prev == 0 || prev != nullptr, "prev is NULL");
  return hip_status(gs::launch_view_priority(weights, num_views, prev, num_prev, score,
                                             static_cast<hipStream_t>(stream)),
                    "gs_view_priority");
}

gs_status gs_tile_partition(const uint32_t* cost, int32_t num_tiles, int32_t num_blocks, int32_t* bounds,
                            void* stream) {
  REQUIRE(num_tiles >= 1 && num_tiles <= GS_MAX_PARTITION_TILES, "num_tiles = %d out of range", num_tiles);
  REQUIRE(num_blocks >= 1 && num_blocks <= GS_MAX_TILE_BLOCKS, "num_blocks = %d out of range", num_blocks);
  REQUIRE(cost != nullptr && aligned(cost, 4), "cost NULL or misaligned");
  REQUIRE(bounds != nullptr && aligned(bounds, 4), "bounds NULL or misaligned");
  return hip_status(gs::launch_tile_partition(cost, num_tiles, num_blocks, bounds, static_cast<hipStream_t>(stream)),
                    "gs_tile_partition");
}

gs_status gs_pack_records(const float* proj, int64_t n, const int32_t* vis_idx, const int64_t* vis_count,
                          int32_t width, int32_t height, const int32_t* bounds, int32_t num_blocks,
                          int64_t capacity, int64_t* send_offsets, int32_t* send_idx, float* send_rec,
                          void* workspace, size_t workspace_bytes, void* stream) {
  CHECK(check_size(width, height));
  REQUIRE(n >= 0 && n < (int64_t(1) << 31), "n = %lld out of range", (long long)n);
  REQUIRE(num_blocks >= 1 && num_blocks <= GS_MAX_TILE_BLOCKS, "num_blocks = %d out of range", num_blocks);
  REQUIRE(capacity >= 0 && capacity < (int64_t(1) << 40), "capacity out of range");
  REQUIRE(vis_count != nullptr && aligned(vis_count, 8), "vis_count NULL or misaligned");
  REQUIRE(bounds != nullptr && aligned(bounds, 4), "bounds NULL or misaligned");
  REQUIRE(send_offsets != nullptr && aligned(send_offsets, 8), "send_offsets NULL or misaligned");
  if (n > 0) REQUIRE(proj != nullptr && aligned(proj, 16) && vis_idx != nullptr, "NULL or misaligned proj / vis_idx");
  if (capacity > 0) {
    REQUIRE(send_idx != nullptr, "send_idx is NULL");
    REQUIRE(send_rec == nullptr || aligned(send_rec, 16), "send_rec not 16-byte aligned");
  }
  REQUIRE(workspace != nullptr && aligned(workspace, 256), "workspace NULL or not 256-byte aligned");
  REQUIRE(workspace_bytes >= gs::pack_ws_bytes(n, num_blocks), "workspace too small");
  return hip_status(gs::launch_pack_records(proj, n, vis_idx, vis_count, (width + 15) / 16, bounds, num_blocks,
                                            capacity, send_offsets, send_idx, send_rec, workspace,
                                            static_cast<hipStream_t>(stream)),
                    "gs_pack_records");
}

gs_status gs_unpack_grads(const float* recv_grad, const int64_t* send_offsets, const int32_t* send_idx,
                          int32_t num_blocks, int64_t capacity, float* grad2d, int64_t n, void* stream) {
  REQUIRE(num_blocks >= 1 && num_blocks <= GS_MAX_TILE_BLOCKS, "num_blocks = %d out of range", num_blocks);
  REQUIRE(capacity >= 0 && capacity < (int64_t(1) << 40), "capacity out of range");
  REQUIRE(n >= 0 && n < (int64_t(1) << 31), "n = %lld out of range", (long long)n);
  REQUIRE(send_offsets != nullptr && aligned(send_offsets, 8), "send_offsets NULL or misaligned");
  if (capacity > 0)
    REQUIRE(recv_grad != nullptr && aligned(recv_grad, 16) && send_idx != nullptr,
            "NULL or misaligned recv_grad / send_idx");
  if (n > 0) REQUIRE(grad2d != nullptr && aligned(grad2d, 16), "grad2d NULL or not 16-byte aligned");
  if (capacity == 0 || n == 0) return ok();
  return hip_status(gs::launch_unpack_grads(recv_grad, send_offsets, send_idx, num_blocks, capacity, grad2d, n,
                                            static_cast<hipStream_t>(stream)),
                    "gs_unpack_grads");
}

gs_status gs_densify_stats(const float* grad2d, const int32_t* vis_idx, const int64_t* vis_count, int64_t n,
                           float* accum, int32_t* denom, void* stream) {
  REQUIRE(n >= 0 && n < (int64_t(1) << 31), "n = %lld out of range", (long long)n);
  REQUIRE(vis_count != nullptr && aligned(vis_count, 8), "vis_count NULL or misaligned");
  if (n == 0) return ok();
  REQUIRE(grad2d != nullptr && vis_idx != nullptr && accum != nullptr && denom != nullptr, "NULL argument");
  REQUIRE(aligned(grad2d, 4) && aligned(vis_idx, 4) && aligned(accum, 4) && aligned(denom, 4), "misaligned array");
  return hip_status(gs::launch_densify_stats(grad2d, vis_idx, vis_count, n, accum, denom,
                                             static_cast<hipStream_t>(stream)),
                    "gs_densify_stats");
}

gs_status gs_densify(const float* params, const float* m, const float* v, int64_t n, int64_t ld,
                     const float* accum, const int32_t* denom, const float* normals, float grad_threshold,
                     float log_scale_threshold, float logit_threshold, float log_shrink, float* out_params,
                     float* out_m, float* out_v, int64_t ld_out, int64_t* out_n, void* workspace,
                     size_t workspace_bytes, void* stream) {
  REQUIRE(n >= 0 && n < (int64_t(1) << 30), "n = %lld out of range", (long long)n);
  REQUIRE(ld >= n && ld >= 1, "ld < n");
  REQUIRE(ld_out >= 0 && ld_out < (int64_t(1) << 31), "ld_out out of range");
  REQUIRE(out_n != nullptr && aligned(out_n, 8), "out_n NULL or misaligned");
  if (n > 0)
    REQUIRE(params && m && v && accum && denom && normals, "NULL params / m / v / accum / denom / normals");
  if (ld_out > 0) REQUIRE(out_params && out_m && out_v, "NULL out_params / out_m / out_v");
  REQUIRE(workspace != nullptr && aligned(workspace, 256), "workspace NULL or not 256-byte aligned");
  REQUIRE(workspace_bytes >= gs::densify_ws_bytes(n), "workspace too small");
  return hip_status(gs::launch_densify(params, m, v, n, ld, accum, denom, normals, grad_threshold,
                                       log_scale_threshold, logit_threshold, log_shrink, out_params, out_m, out_v,
                                       ld_out, out_n, workspace, static_cast<hipStream_t>(stream)),
                    "gs_densify");
}

}  // extern "C"
