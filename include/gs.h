/*
 * libgs -- one training step of 3D Gaussian Splatting on an AMD MI355X
 * (gfx950), as a C ABI over hand-written HIP kernels.
 *
 * The step (Grendel-GS notes, "Grendel-GS: On Scaling Up 3D Gaussian
 * Splatting Training", section "Background -- training pipeline"):
 * project each Gaussian to screen space (2D mean, depth, cover radius,
 * colour); for each pixel find the covering Gaussians, sort them by depth
 * and alpha-composite them; L1 + SSIM loss; back-propagate into the
 * Gaussian parameters.  The Odin summary page ("Odin: Primitive-Level
 * Synchronization for Distributed Point-Based Neural Rendering", section
 * "Background and motivation") adds that each view reads and writes only a
 * sparse, view-dependent set of primitive indices: gs_preprocess emits that
 * set as a sorted list, gs_render_bwd writes gradients only for it, and
 * gs_sparse_adam updates only the union of the sets of a batch.
 *
 * Conventions for every entry point:
 *  - Pointers marked "device" are caller-owned device memory (e.g. PyTorch
 *    tensors' data_ptr()); the library never allocates, frees or keeps
 *    them.  "host" pointers are read or written during the call only.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and is asynchronous unless stated otherwise.  Only gs_bin_sort blocks
 *    (one device-to-host read of the pair count).
 *  - Errors are returned as gs_status; gs_last_error() gives a
 *    thread-local message.  Argument checks happen on the host before any
 *    work is enqueued: on GS_ERR_INVALID_ARG nothing was launched.
 *  - Concurrent calls on distinct streams with distinct buffers are safe.
 *
 * Parameter layout: 59 fp32 planes, plane-major params[k * ld + i] for
 * Gaussian i (Grendel-GS notes, parameter table): planes 0-2 position,
 * 3-5 log-scale, 6-9 quaternion (w, x, y, z; normalised by the library),
 * 10 opacity logit, 11 + 3k + c spherical-harmonic coefficient of basis
 * k = 0..15 (degree <= 3) and colour channel c.
 *
 * Images are planar [3][H][W] fp32; per-pixel planes are [H][W].  Tiles are
 * 16x16 pixels (Grendel-GS notes, "pixel-wise distribution"), numbered
 * tile = ty * TX + tx with TX = ceil(W / 16), TY = ceil(H / 16).
 */
#ifndef GS_H
#define GS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gs_status {
  GS_OK = 0,
  GS_ERR_INVALID_ARG = 1, /* bad pointer, size, alignment or workspace */
  GS_ERR_CAPACITY = 2,    /* more Gaussian-tile pairs than pair_capacity */
  GS_ERR_HIP = 3          /* a HIP runtime call failed */
} gs_status;

/* Pinhole camera, world -> camera x_c = R x_w + t (R row-major); camera axes
 * x right, y down, z forward; pixel (i, j) is sampled at (i + 1/2, j + 1/2).
 * Gaussians with camera-space z <= near_z are not visible. */
typedef struct gs_camera {
  int32_t width, height;
  float fx, fy, cx, cy;
  float R[9];
  float t[3];
  float campos[3]; /* camera centre in world coordinates (view direction of the SH colour) */
  float near_z;
} gs_camera;

/* Projected record of a Gaussian: 16 32-bit words, 64-byte aligned rows.
 *   0 u, 1 v            screen mean (pixels)
 *   2 A, 3 B, 4 C       conic = inverse screen covariance, power =
 *                       -(A dx^2 + C dy^2)/2 - B dx dy
 *   5 opacity           sigmoid(logit)
 *   6 r, 7 g, 8 b       colour max(0, SH(view dir) + 1/2)
 *   9, 10               culling half-extents (library-internal)
 *  11 radius (int32)    ceil(3 sqrt(largest eigenvalue of the covariance))
 *  12 depth (float)     camera-space z
 *  13 x0 | x1 << 16, 14 y0 | y1 << 16   half-open tile rectangle
 *  15 tiles (uint32)    (x1 - x0) (y1 - y0); 0 when not visible
 * Words 0-11 and 13-15 are zero (9, 10: -inf) for Gaussians that are not
 * visible. */
#define GS_PROJ_WORDS 16
/* floats per Gaussian in the screen-space gradient buffer of gs_render_bwd:
 * dL/d(u, v, A, B, C, opacity, r, g, b) then 3 unused */
#define GS_GRAD2D_WORDS 12
/* most views whose projection backward gs_project_bwd_adam fuses */
#define GS_MAX_FUSED_VIEWS 16
/* bytes per Gaussian in the touched map of gs_render_bwd and
 * gs_project_bwd_adam (one slot per fused view) */
#define GS_TOUCHED_SLOTS 16
/* most views gs_preprocess_views projects in one call */
#define GS_MAX_PREPROCESS_VIEWS 16
/* most views gs_view_overlap couples in one call */
#define GS_MAX_COUPLED_VIEWS 65536
/* most tile blocks of gs_tile_partition / gs_pack_records, and most tiles
 * gs_tile_partition splits */
#define GS_MAX_TILE_BLOCKS 64
#define GS_MAX_PARTITION_TILES (1 << 21)
/* most Gaussians (n) of the calls that read or write the [59][ld] parameter
 * planes (gs_preprocess, gs_preprocess_views, gs_project_bwd, gs_render_bwd
 * with param_grads, gs_sparse_adam, gs_project_bwd_adam): their kernels
 * address a row by a
 * 32-bit byte offset; larger n is rejected with GS_ERR_INVALID_ARG */
#define GS_MAX_PLANE_ROWS ((int64_t)1 << 30)

typedef enum gs_op {
  GS_OP_PREPROCESS = 0,
  GS_OP_BIN_SORT = 1,
  GS_OP_LOSS = 2,
  GS_OP_SPARSE_ADAM = 3,
  GS_OP_RASTER = 4,
  GS_OP_VIEW_OVERLAP = 5,
  GS_OP_PACK = 6,
  GS_OP_DENSIFY = 7,
  GS_OP_PREPROCESS_VIEWS = 8
} gs_op;

/* Static description of a status code (never NULL). */
const char* gs_status_string(int status);
/* Thread-local detail of the last failing call on this thread ("" if none). */
const char* gs_last_error(void);
/* Library interface version (1). */
int gs_version(void);

/* Workspace bytes an entry point needs (host, no device work):
 *   GS_OP_PREPROCESS  n
 *   GS_OP_BIN_SORT    n, pair_capacity
 *   GS_OP_LOSS        width, height
 *   GS_OP_SPARSE_ADAM n
 *   GS_OP_RASTER      width, height: split_ws of gs_render_fwd / gs_render_bwd
 *   GS_OP_VIEW_OVERLAP n, width = num_views
 *   GS_OP_PACK        n, width = num_blocks
 *   GS_OP_DENSIFY     n
 *   GS_OP_PREPROCESS_VIEWS n, width = num_views
 * Unused arguments are ignored.  The workspace is caller-owned device
 * memory, 256-byte aligned; its contents need no initialisation and are
 * scratch between calls. */
gs_status gs_workspace_size(gs_op op, int64_t n, int32_t width, int32_t height, int64_t pair_capacity,
                            size_t* bytes);

/* Projection of n Gaussians for one view and the view's visible set
 * (Grendel-GS notes, training pipeline: "Gaussian transform"; Odin summary
 * page: the sparse, view-dependent primitive set).
 *   params       device, [59][ld] fp32, ld >= n
 *   cam          host
 *   proj         device out, [n][GS_PROJ_WORDS], 16-byte aligned
 *   proj_bin     device out, or NULL: [n][4] fp32, 16-byte aligned, each
 *                record's last four words again (depth, rectangle, tile
 *                count), densely: what gs_bin_sort reads, 16 bytes per
 *                Gaussian instead of a 64-byte record's
 *   vis_idx      device out, [n] int32: the visible indices in ascending
 *                order in the first *vis_count entries
 *   vis_count    device out, int64 scalar
 *   union_flags  device in/out, [n] uint8, 16-byte aligned, or NULL: set to
 *                1 for every visible Gaussian, never cleared here (the batch
 *                union consumed by gs_sparse_adam)
 *   workspace    device, >= gs_workspace_size(GS_OP_PREPROCESS) bytes
 * Visible = all 59 parameters finite, z > near_z, non-degenerate
 * quaternion and screen covariance, finite projection, and a non-empty
 * tile rectangle. */
gs_status gs_preprocess(const float* params, int64_t n, int64_t ld, const gs_camera* cam, float* proj,
                        float* proj_bin, int32_t* vis_idx, int64_t* vis_count, uint8_t* union_flags, void* workspace,
                        size_t workspace_bytes, void* stream);

/* gs_preprocess of several views in one pass over the parameters (the same
 * passages): each Gaussian's 59 parameters are read once and projected with
 * every camera in turn, so a batch's views cost one read of the parameter
 * planes instead of one per view.  Each view's records, visible list and
 * count are bit for bit those of gs_preprocess with that camera.
 *   cams         host array of num_views (1..GS_MAX_PREPROCESS_VIEWS)
 *                cameras
 *   proj         host array of num_views device pointers, one buffer per
 *                view: [n][GS_PROJ_WORDS], 16-byte aligned
 *   proj_bin     NULL, or a host array of num_views device pointers (each
 *                NULL or as gs_preprocess's proj_bin)
 *   vis_idx      host array of num_views device pointers: [n] int32 each,
 *                as gs_preprocess's
 *   vis_count    device out, [num_views] int64: view w's count at w
 *   union_flags  as gs_preprocess: set for a Gaussian visible in any of
 *                the views
 *   max_workgroups  0: one workgroup per 256 Gaussians; else at most this
 *                many, each walking the Gaussians with a stride (fewer
 *                loads in flight: a caller running the call beside
 *                latency-bound work keeps its share of the HBM bandwidth
 *                small; the results do not depend on it)
 *   workspace    device, >= gs_workspace_size(GS_OP_PREPROCESS_VIEWS, n,
 *                num_views) bytes (the views' visibility bytes and the
 *                compaction's counts)
 * Errors: GS_ERR_INVALID_ARG for num_views outside the range, an invalid
 * camera, a NULL or misaligned buffer, max_workgroups < 0, or as
 * gs_preprocess. */
gs_status gs_preprocess_views(const float* params, int64_t n, int64_t ld, const gs_camera* cams, int32_t num_views,
                              float* const* proj, float* const* proj_bin, int32_t* const* vis_idx,
                              int64_t* vis_count, uint8_t* union_flags, int32_t max_workgroups, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Gaussian-tile pairs sorted by depth within each tile, and the tile ranges
 * (Grendel-GS notes, training pipeline: "find the covering Gaussians, sort
 * by depth"; Odin summary page, stage task graph: range extraction).
 *   proj, vis_idx, vis_count   device, from gs_preprocess (same n, view)
 *   proj_bin     device or NULL: gs_preprocess's proj_bin of the same view;
 *                when given, the depths, rectangles and tile counts come
 *                from it (16 bytes per Gaussian) instead of proj's records;
 *                results are the same either way
 *   keys         device out, [pair_capacity] uint64: (tile << 32) | bit
 *                pattern of the fp32 depth, ascending; equal keys in
 *                ascending Gaussian index.  May be NULL when the image is
 *                at most 256 tiles wide and tall (4096 pixels): the keys
 *                then go unwritten (vals and tile_ranges determine them:
 *                the tile from the range, the depth from the record)
 *   vals         device out, [pair_capacity] int32 Gaussian index per pair
 *   num_pairs    host out: M, the number of pairs
 *   tile_ranges  device out, [TX*TY][2] uint32: [start, end) of each tile's
 *                pairs, [0, 0) for empty tiles
 *   tile_order   device out or NULL, [TX*TY] uint32: a launch order of the
 *                tiles for the rasterisers -- tiles by descending bit length
 *                of their pair count, ties in tile order (a schedule only:
 *                results do not depend on it)
 *   workspace    device, >= gs_workspace_size(GS_OP_BIN_SORT, n, .., pair_capacity)
 * Blocks the calling thread once, to read M.  If M > pair_capacity the call
 * writes *num_pairs = M, returns GS_ERR_CAPACITY and writes neither pairs
 * nor ranges.  pair_capacity must be < 2^31. */
gs_status gs_bin_sort(const float* proj, const float* proj_bin, int64_t n, const int32_t* vis_idx,
                      const int64_t* vis_count, int32_t width, int32_t height, uint64_t* keys, int32_t* vals,
                      int64_t pair_capacity, int64_t* num_pairs, uint32_t* tile_ranges, uint32_t* tile_order,
                      void* workspace, size_t workspace_bytes, void* stream);

/* gs_bin_sort without the blocking read: the same outputs, with M written to
 * the device (same passages).
 *   num_pairs_dev  device out, 8-byte aligned: M, valid in stream order
 * Nothing blocks.  If M > pair_capacity: *num_pairs_dev = M, keys and vals
 * are not written, every tile range is [0, 0) (and tile_order a valid order
 * of those empty tiles); the caller detects this by comparing
 * *num_pairs_dev with pair_capacity once the stream has reached it.  The
 * rasterisers take pair_capacity as their num_pairs bound then.
 *   part           GS_BIN_ALL; or the two halves as two calls with the same
 *                  arguments, in stream order: GS_BIN_DEPTH (the visible
 *                  Gaussians in depth order and the pair count M, kept in
 *                  the workspace; num_pairs_dev written) then GS_BIN_PAIRS
 *                  (the pairs, ranges and order from them) -- so that other
 *                  work can be ordered between the depth sort and the pairs
 *                  (Grendel-GS notes, training pipeline: the covering
 *                  Gaussians found and sorted by depth per tile).
 * GS_ERR_INVALID_ARG also for another part value. */
#define GS_BIN_ALL 0
#define GS_BIN_DEPTH 1
#define GS_BIN_PAIRS 2
gs_status gs_bin_sort_async(const float* proj, const float* proj_bin, int64_t n, const int32_t* vis_idx,
                            const int64_t* vis_count, int32_t width, int32_t height, uint64_t* keys, int32_t* vals,
                            int64_t pair_capacity, int64_t* num_pairs_dev, uint32_t* tile_ranges,
                            uint32_t* tile_order, void* workspace, size_t workspace_bytes, int32_t part,
                            void* stream);

/* Front-to-back alpha compositing per 16x16 tile (Grendel-GS notes,
 * training pipeline: "alpha compositing").  Per pixel, over its tile's
 * pairs in order: power as in GS_PROJ_WORDS; skip if power > 0;
 * alpha = min(0.99, opacity e^power), skip if alpha < 1/255; stop before the
 * Gaussian that would bring the transmittance T (1 - alpha) below 1e-4;
 * C += colour alpha T; T *= 1 - alpha.  Black background.
 *   proj, vals, tile_ranges, num_pairs   device/host, from gs_preprocess and gs_bin_sort
 *   tile_order   device or NULL: gs_bin_sort's launch order (NULL = tile order)
 *   image        device out, [3][H][W]
 *   T_final      device out, [H][W] final transmittance
 *   last         device out, [H][W] uint32: 1 + list position (within the
 *                tile's range) of the last composited Gaussian, 0 if none
 *   tile_processed  device out or NULL, [TX*TY] uint32: per tile, the
 *                largest number of list entries any of its pixels read
 *                (up to and including the stopping one)
 *   split_ws, split_ws_bytes  device workspace or NULL: at least
 *                gs_workspace_size(GS_OP_RASTER, 0, width, height) bytes,
 *                256-byte aligned.  The forward records, for every
 *                quarter-tile whose list reaches past segment_len entries,
 *                the per-pixel state (transmittance, colour behind) at each
 *                multiple of segment_len it reaches (at most 31 per quarter;
 *                room for one state per quarter of the image, beyond
 *                which lists stay whole) and lists the segments
 *                gs_render_bwd can run in parallel; ignored for images of
 *                2^25 tiles or more.  Pass it unchanged, with the same
 *                segment_len, to the gs_render_bwd of this view.
 *   segment_len  list entries per segment: a power of two in [64, 65536]
 *                (ignored when split_ws is NULL) */
gs_status gs_render_fwd(const float* proj, int64_t n, const int32_t* vals, const uint32_t* tile_ranges,
                        const uint32_t* tile_order, int64_t num_pairs, int32_t width, int32_t height, float* image,
                        float* T_final, uint32_t* last, uint32_t* tile_processed, void* split_ws,
                        size_t split_ws_bytes, int32_t segment_len, void* stream);

/* Loss of a rendered image against a target (Grendel-GS notes, training
 * pipeline: "L1 + SSIM loss"):
 *   L = w_l1 mean|I - I_t| + w_ssim (1 - mean SSIM), means over 3 H W;
 * SSIM per channel with the 11x11 Gaussian window of sigma 1.5, zero
 * padding, C1 = 0.01^2, C2 = 0.03^2.  w_ssim = 0 skips the SSIM work.
 *   image, target   device, [3][H][W]
 *   loss            device out, fp32 scalar
 *   dL_dimage       device out, [3][H][W]
 *   workspace       device, >= gs_workspace_size(GS_OP_LOSS, .., W, H) */
gs_status gs_loss(const float* image, const float* target, int32_t width, int32_t height, float w_l1,
                  float w_ssim, float* loss, float* dL_dimage, void* workspace, size_t workspace_bytes,
                  void* stream);

/* Raster backward of one view (Grendel-GS notes, training pipeline:
 * "back-propagation"): per pixel, the composited Gaussians in reverse order
 * with the transmittance rebuilt by division and the colour of what lies
 * behind carried along; the partials of every (pixel, Gaussian) are summed
 * per Gaussian into its screen-space gradient.
 *   proj, vals, tile_ranges, num_pairs, T_final, last   from the forward
 *   tile_order   device or NULL: gs_bin_sort's launch order (NULL = tile order)
 *   dL_dimage    device, [3][H][W]
 *   grad2d       device in/out, [n][GS_GRAD2D_WORDS] fp32, 16-byte aligned:
 *                dL/d(u, v, A, B, C, opacity, r, g, b) of the view are ADDED
 *                to the rows of the Gaussians in the pairs.  Those rows must
 *                be zero on entry (allocate zeroed; gs_project_bwd re-zeroes
 *                the rows it consumes, so the buffer stays zero between
 *                views).
 *   split_ws, split_ws_bytes, segment_len  NULL, or what the gs_render_fwd of this view
 *                was given (its contents as it left them): the listed
 *                segments of long lists are then walked by separate waves
 *                from the recorded states, the rest of each list from its
 *                end (the same sums up to fp32 rounding order)
 *   param_grads  NULL (screen-space gradients only, left in grad2d for a
 *                later gs_project_bwd or gs_project_bwd_adam), or the
 *                projection backward of the view chained on in the same
 *                call (Odin summary page: a view's backward writes the
 *                gradients of its primitive set only): the view's
 *                parameter gradients dL/dparams are ADDED (+=) to
 *                param_grads->grads ([59][ld]) for the rows of its visible
 *                list, exactly as gs_project_bwd computes them, and those
 *                grad2d rows are re-zeroed (grad2d is then scratch: zero on
 *                entry and on return)
 *   visits       device, uint64 scalar, or NULL: the number of (pixel,
 *                list entry) pairs whose compositing step was
 *                back-propagated (the pixels that composited the entry)
 *                is ADDED to *visits -- the backward's unit of work (the
 *                counting costs an atomic add per wave)
 *   touched, touched_slot   NULL, or the touched map: device,
 *                [n][GS_TOUCHED_SLOTS] uint8, 16-byte aligned, and this
 *                view's slot (0 .. GS_TOUCHED_SLOTS - 1): byte
 *                touched_slot of every row the call adds gradient into is
 *                set to 1 (every row with a non-zero grad2d word is marked;
 *                a marked row may still be all zero).  Only without
 *                param_grads.  gs_project_bwd_adam reads and clears it.
 * The discrete decisions (skip, stop, 0.99 clamp) are held at the
 * forward's; the 2D mean gradient is in pixels; depth gets none.
 * Errors: GS_ERR_INVALID_ARG for sizes out of range, NULL or misaligned
 * buffers, a split workspace of the wrong size or segment length, an
 * invalid camera or ld < n in param_grads, a touched slot out of range or
 * touched with param_grads. */
typedef struct {
  const float* params;      /* device, [59][ld] fp32: the view's parameters */
  int64_t ld;               /* plane stride, >= n */
  const gs_camera* cam;     /* host: the view's camera */
  const int32_t* vis_idx;   /* device: the view's visible list (gs_preprocess) */
  const int64_t* vis_count; /* device: its length */
  float* grads;             /* device in/out, [59][ld] fp32: += dL/dparams */
} gs_param_grads;
gs_status gs_render_bwd(const float* proj, int64_t n, const int32_t* vals, const uint32_t* tile_ranges,
                        const uint32_t* tile_order, int64_t num_pairs, int32_t width, int32_t height,
                        const float* T_final, const uint32_t* last, const float* dL_dimage, float* grad2d,
                        const void* split_ws, size_t split_ws_bytes, int32_t segment_len,
                        const gs_param_grads* param_grads, uint64_t* visits, uint8_t* touched,
                        int32_t touched_slot, void* stream);

/* Projection backward of one view: the chain rule from the screen-space
 * gradients to all 59 parameters (SH coefficients and view direction, EWA
 * covariance, scale through exp, rotation through the normalised
 * quaternion, mean through the pinhole map, opacity through the sigmoid),
 * for the view's visible Gaussians only (Odin summary page: a view writes
 * only its primitive set).
 *   params, cam          as for gs_preprocess
 *   vis_idx, vis_count   device, from gs_preprocess
 *   grad2d       device in/out, from gs_render_bwd; the visible rows are
 *                read, then set to zero
 *   grads        device in/out, [59][ld]: dL/dparams ADDED (+=) for the
 *                visible rows (accumulates the views of a batch)
 * The colour clamp decision is recomputed with the forward's arithmetic. */
gs_status gs_project_bwd(const float* params, int64_t n, int64_t ld, const gs_camera* cam, const int32_t* vis_idx,
                         const int64_t* vis_count, float* grad2d, float* grads, void* stream);

/* Adam on the union of the batch's visible sets (Odin summary page: updates
 * touch only the primitives a view used; Grendel-GS notes, "Hyper-parameter
 * scaling rule": pass lr * sqrt(b) and beta^b for a batch of b views).
 *   params, grads, m, v   device, [59][ld] fp32
 *   union_flags  device in/out, [n] uint8, 16-byte aligned: rows to update
 *                (from gs_preprocess); cleared to 0 on return
 *   union_idx    device out, [n] int32: the updated rows, ascending
 *   union_count  device out, int64 scalar
 *   bias_c1, bias_c2   1 - beta1^t and 1 - beta2^t for step t (t >= 1)
 * For each listed row i and plane k:
 *   m = beta1 m + (1 - beta1) g;  v = beta2 v + (1 - beta2) g^2;
 *   p -= lr (m / bias_c1) / (sqrt(v / bias_c2) + eps);  g = 0.
 * Unlisted rows keep p, m, v and g. */
gs_status gs_sparse_adam(float* params, float* grads, float* m, float* v, int64_t n, int64_t ld,
                         uint8_t* union_flags, int32_t* union_idx, int64_t* union_count, float lr, float beta1,
                         float beta2, float eps, float bias_c1, float bias_c2, void* workspace,
                         size_t workspace_bytes, void* stream);

/* gs_sparse_adam without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving and
 * training loops, harnesses that forbid hipMalloc).  Its scratch (the union
 * compaction's per-block counts) lives in a file-scope device array of
 * GS_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds until
 * the process ends; the call allocates nothing and frees nothing.
 *   arguments and results as gs_sparse_adam.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (on different streams, or from different threads) race and must be
 * ordered by the caller.  Nothing in the array has to start at zero: each
 * call writes every word it reads before reading it.
 * Errors: as gs_sparse_adam; GS_ERR_INVALID_ARG also when n > GS_NOALLOC_MAX_N
 * (the union compaction of more rows would not fit the array); GS_ERR_HIP
 * when the array's device address cannot be obtained.  Nothing is launched
 * on an error. */
#define GS_NOALLOC_SCRATCH_BYTES (256 * 1024)
#define GS_NOALLOC_MAX_N ((int64_t)(GS_NOALLOC_SCRATCH_BYTES / 4 - 1) * 4096)
gs_status gs_sparse_adam_noalloc(float* params, float* grads, float* m, float* v, int64_t n, int64_t ld,
                                 uint8_t* union_flags, int32_t* union_idx, int64_t* union_count, float lr,
                                 float beta1, float beta2, float eps, float bias_c1, float bias_c2, void* stream);

/* gs_project_bwd of the batch's last views followed by gs_sparse_adam, in
 * one pass over the union rows (same passages as the two): each listed
 * row's parameters are read once, every fused view's parameter gradients are
 * added in view order to the accumulated ones in registers, and the update
 * consumes them at once, so the gradient planes are neither written nor read
 * back in between.  Results equal gs_project_bwd of each view (in order)
 * followed by gs_sparse_adam, up to the sign of zero gradients.
 *   cams, grad2d   host arrays of num_views (0..GS_MAX_FUSED_VIEWS) entries:
 *                  the views' cameras and the device pointers of their
 *                  gs_render_bwd screen-space gradients ([n][12], 16-byte
 *                  aligned, one buffer per view).  A row of a view is chained
 *                  when any of its 12 words is non-zero (rows outside the
 *                  view's visible set are zero: gs_render_bwd writes only
 *                  visible Gaussians, and a zero row chains to zero); chained
 *                  rows are re-zeroed.
 *   touched        NULL, or the touched map the views' gs_render_bwd calls
 *                  marked (fused view w in slot w; [n][GS_TOUCHED_SLOTS]
 *                  uint8, 16-byte aligned): a listed row's grad2d row of
 *                  view w is read only when its byte w is set, and the
 *                  listed rows' bytes are cleared (so the map is zero again
 *                  once every marked row was listed).  Same results as
 *                  without it, fewer bytes read.
 *   grads          the gradients of the batch's other views ([59][ld]),
 *                  zeroed for the listed rows; or NULL: none (taken as zero,
 *                  nothing written)
 *   next_cam, next_proj, next_flags   NULL, or the preprocess of the view
 *                rendered next, done on each listed row right after its
 *                update (Grendel-GS notes, training pipeline: the Gaussian
 *                transform): the row's projected record with next_cam goes
 *                to next_proj ([n][GS_PROJ_WORDS], 16-byte aligned) as
 *                gs_preprocess writes it, and when the row is visible
 *                next_flags[row] (device, [n] uint8) and union_flags[row]
 *                are set to 1.  Unlisted rows are not touched: a caller
 *                whose next view was one of this batch's (unlisted rows
 *                were invisible in it and keep their parameters) keeps
 *                their records and flags from that view's gs_preprocess
 *                and zero flags.  gs_visible_list turns next_flags into
 *                the view's visible list.
 *   next_proj_bin  NULL, or with next_proj: the rows' dense copies of the
 *                records' last four words, as gs_preprocess's proj_bin
 *   the other arguments as gs_sparse_adam.
 * Errors: GS_ERR_INVALID_ARG for num_views outside the range, a NULL or
 * misaligned buffer, an invalid camera, or as gs_sparse_adam. */
gs_status gs_project_bwd_adam(float* params, float* grads, float* m, float* v, int64_t n, int64_t ld,
                              const gs_camera* cams, int32_t num_views, float* const* grad2d, uint8_t* touched,
                              uint8_t* union_flags, int32_t* union_idx, int64_t* union_count,
                              const gs_camera* next_cam,
                              float* next_proj, float* next_proj_bin, uint8_t* next_flags, float lr, float beta1,
                              float beta2, float eps, float bias_c1, float bias_c2, void* workspace,
                              size_t workspace_bytes, void* stream);

/* The ascending visible list of a view from per-Gaussian visibility bytes
 * (the compaction gs_preprocess ends with; Odin summary page, "Background
 * and motivation": the sparse, view-dependent set of primitives a view
 * touches).
 *   flags        device in/out, [n] uint8, 16-byte aligned: non-zero =
 *                visible; cleared to 0 on return
 *   vis_idx, vis_count   device out, as gs_preprocess
 *   workspace    device, >= gs_workspace_size(GS_OP_PREPROCESS, n) bytes */
gs_status gs_visible_list(uint8_t* flags, int64_t n, int32_t* vis_idx, int64_t* vis_count, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Pairwise overlap of views' visible sets and their coupling weights
 * (Odin summary page, "Relative locality graph": the edge weight of two
 * data items is the Jaccard similarity of their point sets, |P_i n P_j| /
 * |P_i u P_j|, and 0 when the union is empty).  The point set of a view is
 * its visible list as gs_preprocess writes it (the page builds its graph
 * from SfM tracks ahead of time and notes a computation-based variant; the
 * visible lists are that variant's sets).
 *   lists        device, [num_views][ld] int32: view v's set in the first
 *                counts[v] entries of row v, strictly ascending, each in
 *                [0, n) (what gs_preprocess writes to vis_idx)
 *   ld           row stride of lists in entries, >= 1
 *   counts       device, [num_views] int64 (gs_preprocess's vis_count);
 *                read as min(max(counts[v], 0), ld)
 *   num_views    0 .. GS_MAX_COUPLED_VIEWS
 *   n            number of Gaussians (the universe of the sets), 0 .. 2^31-1
 *   inter        device out, [num_views][num_views] int64, 8-byte aligned:
 *                |P_i n P_j|; the diagonal holds |P_i|
 *   weights      device out, [num_views][num_views] fp64, 8-byte aligned,
 *                or NULL: w_ij, computed in fp64 as inter_ij /
 *                (inter_ii + inter_jj - inter_ij), and 0 where that union
 *                is 0 (so w_ii = 1 for a non-empty set)
 *   workspace    device, >= gs_workspace_size(GS_OP_VIEW_OVERLAP, n,
 *                num_views) bytes, 256-byte aligned
 * Entries outside [0, n) are skipped.  Lists that are not strictly
 * ascending give unspecified counts (every access stays inside the
 * buffers).  Counts are exact integers; the result does not depend on the
 * launch schedule.
 * Errors: GS_ERR_INVALID_ARG for sizes out of range or a NULL or
 * misaligned buffer. */
gs_status gs_view_overlap(const int32_t* lists, int64_t ld, const int64_t* counts, int32_t num_views, int64_t n,
                          int64_t* inter, double* weights, void* workspace, size_t workspace_bytes, void* stream);

/* Scheduling priority of every view given the previously scheduled set
 * (Odin summary page, "Relative locality graph": s(v | U_prev) is the sum
 * of w_uv over u in U_prev).
 *   weights      device, [num_views][num_views] fp64 (gs_view_overlap)
 *   prev         device, [num_prev] int32 view indices (U_prev; a repeated
 *                index is added again, one outside [0, num_views) is
 *                skipped); may be NULL when num_prev is 0
 *   score        device out, [num_views] fp64: s(v | U_prev), the terms
 *                added in fp64 in the order of prev, from 0
 * Errors: GS_ERR_INVALID_ARG for sizes out of range or a NULL buffer. */
gs_status gs_view_priority(const double* weights, int32_t num_views, const int32_t* prev, int32_t num_prev,
                           double* score, void* stream);

/* Contiguous runs of tile ids with about equal total cost (Grendel-GS
 * notes, "dynamic load balancing", pixel-wise balancing: the cumulative sum
 * of the per-block cost is searched at the multiples of total / K).
 *   cost         device, [num_tiles] uint32 cost per 16x16 tile in
 *                row-major tile order (the rasteriser's tile_processed
 *                counts are one such cost)
 *   num_tiles    1 .. GS_MAX_PARTITION_TILES
 *   num_blocks   K, 1 .. GS_MAX_TILE_BLOCKS
 *   bounds       device out, [K + 1] int32: block d is tiles
 *                [bounds[d], bounds[d + 1]); bounds[0] = 0, bounds[K] =
 *                num_tiles, and for 0 < d < K bounds[d] is the first t with
 *                K * P(t) >= d * total, P(t) the cost of tiles [0, t), in
 *                exact integer arithmetic (a block ends with the tile at
 *                which its share is reached; with no cost at all every tile
 *                is in the last block)
 * Errors: GS_ERR_INVALID_ARG for sizes out of range or a NULL buffer. */
gs_status gs_tile_partition(const uint32_t* cost, int32_t num_tiles, int32_t num_blocks, int32_t* bounds,
                            void* stream);

/* The sending end of the sparse all-to-all from the Gaussian-wise to the
 * pixel-wise split, for one view (Grendel-GS notes, "hybrid parallel
 * strategy" and "sparse all-to-all communication": each Gaussian goes only
 * to the pixel blocks its screen footprint reaches).  Block d receives the
 * visible Gaussians whose tile rectangle holds a tile of [bounds[d],
 * bounds[d + 1]), in ascending index order, each with its record.
 *   proj, vis_idx, vis_count   device, the view's gs_preprocess outputs
 *   n            number of Gaussians, 0 .. 2^31-1
 *   width, height  the view's image size (the tile grid of the rectangles)
 *   bounds       device, [num_blocks + 1] int32 (gs_tile_partition's form;
 *                other contents give other lists but no access out of
 *                bounds)
 *   num_blocks   1 .. GS_MAX_TILE_BLOCKS
 *   capacity     entries send_idx / send_rec hold
 *   send_offsets device out, [num_blocks + 1] int64, 8-byte aligned: block
 *                d's entries are [send_offsets[d], send_offsets[d + 1]);
 *                send_offsets[num_blocks] is the total.  When the total
 *                exceeds capacity no entry at or past capacity is written:
 *                call again with capacity >= the total.
 *   send_idx     device out, [capacity] int32 Gaussian indices
 *   send_rec     device out, [capacity][GS_PROJ_WORDS] records, 16-byte
 *                aligned, or NULL for indices only
 *   workspace    device, >= gs_workspace_size(GS_OP_PACK, n, num_blocks)
 *                bytes, 256-byte aligned
 * Errors: GS_ERR_INVALID_ARG for sizes out of range or a NULL or
 * misaligned buffer. */
gs_status gs_pack_records(const float* proj, int64_t n, const int32_t* vis_idx, const int64_t* vis_count,
                          int32_t width, int32_t height, const int32_t* bounds, int32_t num_blocks,
                          int64_t capacity, int64_t* send_offsets, int32_t* send_idx, float* send_rec,
                          void* workspace, size_t workspace_bytes, void* stream);

/* The receiving end of the reverse all-to-all: the screen-space gradient
 * rows the tile blocks computed for their packed Gaussians, added into the
 * Gaussians' rows block by block in ascending block order (fp32; a
 * Gaussian appears at most once per block, so the sums are deterministic).
 *   recv_grad    device, [capacity][GS_GRAD2D_WORDS] fp32, 16-byte aligned,
 *                row j for packed entry j
 *   send_offsets, send_idx   as gs_pack_records wrote them; entries at or
 *                past capacity and indices outside [0, n) are skipped
 *   grad2d       device in/out, [n][GS_GRAD2D_WORDS] fp32, 16-byte aligned
 * Errors: GS_ERR_INVALID_ARG for sizes out of range or a NULL or
 * misaligned buffer. */
gs_status gs_unpack_grads(const float* recv_grad, const int64_t* send_offsets, const int32_t* send_idx,
                          int32_t num_blocks, int64_t capacity, float* grad2d, int64_t n, void* stream);

/* One view's contribution to the densification statistic (Grendel-GS
 * notes, "training pipeline": densification clones or splits the Gaussians
 * whose screen position keeps being pulled and prunes transparent ones).
 * For every visible row i: accum[i] += |dL/d(u, v)| (pixel units, from
 * grad2d words 0 and 1; fp32 with one rounding per operation: u*u, v*v,
 * their sum, the square root, the accumulation) and denom[i] += 1.  Call
 * it after gs_render_bwd for each view whose gradients are still in grad2d.
 *   grad2d       device, [n][GS_GRAD2D_WORDS] fp32
 *   vis_idx, vis_count  device, the view's visible list (gs_preprocess)
 *   accum, denom device in/out, [n] fp32 / int32; the caller zeroes them
 *                when a densification interval starts
 * Errors: GS_ERR_INVALID_ARG for n out of range or a NULL buffer. */
gs_status gs_densify_stats(const float* grad2d, const int32_t* vis_idx, const int64_t* vis_count, int64_t n,
                           float* accum, int32_t* denom, void* stream);

/* Clone / split / prune (the same page and line), into new parameter and
 * Adam buffers:
 *   g = accum / denom (fp32; 0 where denom is 0).  A Gaussian with
 *   g >= grad_threshold densifies: if its largest log-scale is
 *   <= log_scale_threshold it is kept and cloned (an identical copy), else
 *   it is replaced by two children at mean + R(q) (exp(log-scale) * z_c),
 *   z_c = (normals[c][0][i], normals[c][1][i], normals[c][2][i]), with
 *   log-scales lowered by log_shrink and every other parameter copied.  A
 *   Gaussian whose opacity logit is not >= logit_threshold is dropped with
 *   all its copies.
 *   Output columns: the kept originals in index order, then the clones,
 *   then every split Gaussian's first child, then every second child (each
 *   group in index order).  Kept columns keep their Adam moments, new ones
 *   start from 0.
 *   params, m, v   device, [59][ld] fp32 (ld >= n)
 *   accum, denom   device, [n] (gs_densify_stats)
 *   normals        device, [2][3][n] fp32 standard normals (the caller's
 *                  random draws; read only for split Gaussians)
 *   thresholds     grad_threshold (pixel units, as accum),
 *                  log_scale_threshold = log(percent_dense * extent),
 *                  logit_threshold = logit(min_opacity),
 *                  log_shrink = log(0.8 * 2)
 *   out_params, out_m, out_v  device out, [59][ld_out] fp32; columns at or
 *                  past ld_out are not written
 *   out_n          device out, int64: the new count (may exceed ld_out:
 *                  call again with ld_out >= it; at most 2n)
 *   workspace      device, >= gs_workspace_size(GS_OP_DENSIFY, n) bytes,
 *                  256-byte aligned
 * Errors: GS_ERR_INVALID_ARG for sizes out of range, ld < n, or a NULL
 * buffer. */
gs_status gs_densify(const float* params, const float* m, const float* v, int64_t n, int64_t ld,
                     const float* accum, const int32_t* denom, const float* normals, float grad_threshold,
                     float log_scale_threshold, float logit_threshold, float log_shrink, float* out_params,
                     float* out_m, float* out_v, int64_t ld_out, int64_t* out_n, void* workspace,
                     size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GS_H */
