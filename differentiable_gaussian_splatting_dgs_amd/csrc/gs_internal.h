// Internal declarations shared by the translation units of libgs: the
// camera as passed to kernels and the host-side launchers each kernel file
// provides to the C-ABI layer.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gs {

// Camera as a kernel argument (by value).
struct CamArgs {
  float R[9];
  float t[3];
  float campos[3];
  float fx, fy, cx, cy, near_z;
  int32_t width, height, tiles_x, tiles_y;
};

// Gaussian-window weights of the SSIM loss (11 taps, sigma 1.5).
struct SsimWindow {
  float g[11];
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// --- preprocess (preprocess.hip) -----------------------------------------
size_t preprocess_ws_bytes(int64_t n);
// proj_bin: NULL, or [n][4] that also gets each record's last four words.
hipError_t launch_preprocess(const float* params, int64_t n, int64_t ld, const CamArgs& cam,
                             float* proj, float* proj_bin, int32_t* vis_idx, int64_t* vis_count,
                             uint8_t* union_flags, void* ws, hipStream_t st);
// Up to kMaxPreprocessViews views in one pass over the parameters: view w's
// records to proj[w], its visibility bytes to the w-th n-byte slice of the
// workspace, then its ascending list to vis_idx[w] / vis_count[w].
constexpr int kMaxPreprocessViews = 16;
struct PreViews {
  CamArgs cam[kMaxPreprocessViews];
  float4* proj[kMaxPreprocessViews];
  float4* bin[kMaxPreprocessViews];   // NULL, or the dense copy of the records' last four words
  uint8_t* flags[kMaxPreprocessViews];
  int32_t count;
};
size_t preprocess_views_ws_bytes(int64_t n, int32_t num_views);
hipError_t launch_preprocess_views(const float* params, int64_t n, int64_t ld, const CamArgs* cams, int32_t num_views,
                                   float* const* proj, float* const* proj_bin, int32_t* const* vis_idx,
                                   int64_t* vis_count, uint8_t* union_flags, int32_t max_workgroups, void* ws,
                                   hipStream_t st);

// --- compaction of a flag array into ascending indices (compact.hip) -----
size_t compact_ws_bytes(int64_t n);
// flags[i] != 0 -> idx listed; if clear_flags, flags are zeroed afterwards.
hipError_t launch_compact(uint8_t* flags, int64_t n, int32_t* idx, int64_t* count, bool clear_flags,
                          void* ws, hipStream_t st);

// --- bin sort (binsort.hip) ------------------------------------------------
size_t binsort_ws_bytes(int64_t n, int64_t pair_capacity);
// True when the sort runs on the super-tile path, where the 64-bit keys are
// an output only (may be NULL); the plain LSD path sorts them in place.
bool binsort_keys_optional(int32_t tiles_x, int32_t tiles_y);
// Stage 1 (asynchronous): depth sort of the visible list and the pair
// count M, left in device memory at binsort_count_ptr(ws, ...) (and at
// num_pairs_dev if given).
// proj_bin: NULL, or the records' last four words again, densely [n][4]
// (what the depth gather reads, 16 instead of 64 bytes per Gaussian).
hipError_t launch_binsort_stage1(const float* proj, const float* proj_bin, int64_t n, const int32_t* vis_idx,
                                 const int64_t* vis_count,
                                 int32_t tiles_x, int32_t tiles_y, int64_t* num_pairs_dev, void* ws,
                                 int64_t pair_capacity, hipStream_t st);
int64_t* binsort_count_ptr(void* ws, int64_t n, int64_t pair_capacity);
// Stage 2: the pairs in key order and the tile ranges.  M_host >= 0: the
// count read by the caller (<= the capacity); M_host < 0: the count stays
// on the device (an overflow leaves empty ranges and untouched pairs).
hipError_t launch_binsort_stage2(const float* proj, int64_t n, const int32_t* vis_idx, const int64_t* vis_count,
                                 int64_t M_host, int32_t tiles_x, int32_t tiles_y, uint64_t* keys, int32_t* vals,
                                 uint32_t* ranges, uint32_t* tile_order, void* ws, int64_t pair_capacity,
                                 hipStream_t st);

// --- rasteriser (raster_fwd.hip / raster_bwd.hip) ---------------------------
// The split backward's state (checkpoints and work lists, see
// raster_common.hpp), sized for the image; images of 2^25 tiles or more
// run unsplit.
size_t raster_split_bytes(int32_t width, int32_t height);
bool raster_split_fits(int32_t width, int32_t height);
// split: NULL or raster_split_bytes(width, height) of device memory; segments of
// 2^seg_shift list entries (seg_shift >= 6), the same for both passes.
hipError_t launch_render_fwd(const float* proj, const int32_t* vals, const uint32_t* ranges,
                             const uint32_t* tile_order, int64_t num_pairs, int32_t width, int32_t height,
                             float* image, float* T_final, uint32_t* last, uint32_t* tile_processed, void* split,
                             int seg_shift, hipStream_t st);
hipError_t launch_render_bwd(const float* proj, const int32_t* vals, const uint32_t* ranges,
                             const uint32_t* tile_order, int64_t num_pairs, int32_t width, int32_t height,
                             const float* T_final, const uint32_t* last, const float* dL_dimage, float* grad2d,
                             uint8_t* touched, const void* split, int seg_shift, uint64_t* visits, hipStream_t st);
hipError_t launch_project_bwd(const float* params, int64_t n, int64_t ld, const CamArgs& cam,
                              const int32_t* vis_idx, const int64_t* vis_count, float* grad2d, float* grads,
                              hipStream_t st);

// --- loss (loss.hip) --------------------------------------------------------
size_t loss_ws_bytes(int32_t width, int32_t height);
hipError_t launch_loss(const float* image, const float* target, int32_t width, int32_t height,
                       float w_l1, float w_ssim, const SsimWindow& win, float* loss, float* dL_dimage,
                       void* ws, hipStream_t st);

// --- sparse Adam (adam.hip) ---------------------------------------------------
// Views whose projection backward is fused into the Adam pass.
constexpr int kMaxFusedViews = 16;
// The touched map: a row of 16 bytes per Gaussian, byte w set by the raster
// backward of fused view w when it flushes gradient into the row.
constexpr int kTouchedStride = 16;
struct FusedViews {
  CamArgs cam[kMaxFusedViews];
  float* grad2d[kMaxFusedViews];
  int32_t count;
  // Optional: the touched map ([n][16] bytes; byte w of a row non-zero when
  // view w may have a non-zero screen-space row there).  Rows whose byte is
  // zero are not read; the pass clears the bytes of the rows it updates.
  uint8_t* touched;
  // Optional (next_proj != NULL): each updated row is then projected with
  // `next` into next_proj, next_flags[row] = 1 and union_flags[row] = 1 if
  // it is visible there (the preprocess of the view rendered next).
  CamArgs next;
  float* next_proj;
  float* next_bin;     // NULL, or the dense copy of the next records' last four words
  uint8_t* next_flags;
  uint8_t* union_flags;
};
hipError_t launch_project_adam(float* params, float* grads, float* m, float* v, int64_t n, int64_t ld,
                               const FusedViews& views, const int32_t* rows, const int64_t* row_count, float lr,
                               float beta1, float beta2, float eps, float bc1, float bc2, hipStream_t st);
hipError_t launch_sparse_adam(float* params, float* grads, float* m, float* v, int64_t n, int64_t ld,
                              const int32_t* rows, const int64_t* row_count, float lr, float beta1,
                              float beta2, float eps, float bc1, float bc2, hipStream_t st);

// --- view coupling (coupling.hip) ---------------------------------------------
constexpr int kMaxCoupledViews = 65536;
// bitmap workspace of the overlap pass
size_t coupling_ws_bytes(int64_t n, int32_t num_views);
// lists: [B][ld] int32, view v ascending in its first counts[v] entries;
// inter: [B][B] int64 intersection counts; weights: NULL or [B][B] fp64 Jaccard.
hipError_t launch_view_overlap(const int32_t* lists, int64_t ld, const int64_t* counts, int B, int64_t n,
                               int64_t* inter, double* weights, void* ws, hipStream_t st);
hipError_t launch_view_priority(const double* weights, int B, const int32_t* prev, int nprev, double* score,
                                hipStream_t st);

// --- tile blocks and the sparse all-to-all's two ends (shard.hip) -----------
constexpr int kMaxTileBlocks = 64;
constexpr int32_t kMaxPartitionTiles = 1 << 21;
size_t pack_ws_bytes(int64_t n, int32_t num_blocks);
hipError_t launch_tile_partition(const uint32_t* cost, int32_t T, int32_t K, int32_t* bounds, hipStream_t st);
hipError_t launch_pack_records(const float* proj, int64_t n, const int32_t* vis_idx, const int64_t* vis_count,
                               int32_t tiles_x, const int32_t* bounds, int32_t K, int64_t capacity,
                               int64_t* send_offsets, int32_t* send_idx, float* send_rec, void* ws,
                               hipStream_t st);
hipError_t launch_unpack_grads(const float* recv, const int64_t* send_offsets, const int32_t* send_idx, int32_t K,
                               int64_t capacity, float* grad2d, int64_t n, hipStream_t st);

// --- densification (densify.hip) ----------------------------------------------
size_t densify_ws_bytes(int64_t n);
hipError_t launch_densify_stats(const float* grad2d, const int32_t* vis_idx, const int64_t* vis_count, int64_t n,
                                float* accum, int32_t* denom, hipStream_t st);
hipError_t launch_densify(const float* params, const float* m, const float* v, int64_t n, int64_t ld,
                          const float* accum, const int32_t* denom, const float* normals, float grad_threshold,
                          float log_scale_threshold, float logit_threshold, float log_shrink, float* out_params,
                          float* out_m, float* out_v, int64_t ld_out, int64_t* out_n, void* ws, hipStream_t st);

}  // namespace gs
