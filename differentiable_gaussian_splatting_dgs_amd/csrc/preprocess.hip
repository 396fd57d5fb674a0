// Projection of every Gaussian to screen space (the "Gaussian transform" of
// the Grendel-GS notes' training pipeline: 2D mean, depth, cover radius,
// colour), plus the per-view visible-index list the Odin summary page's
// "Background and motivation" describes (each view touches a sparse,
// view-dependent set of primitives).
//
// One thread per Gaussian.  Parameters are plane-major [59][ld] fp32, so
// each of the 59 loads is coalesced across the wave.  Output is one 64-byte
// record per Gaussian (four float4 stores) plus a visibility byte that the
// compaction turns into the ascending visible list.  k_preprocess_views
// does the same for several views in one pass over the parameters.
#include "project_record.hpp"

namespace gs {
namespace {

constexpr int kPT = 256;

__global__ __launch_bounds__(kPT) void k_preprocess(const float* __restrict__ params, int64_t n, int64_t ld,
                                                    CamArgs cam, float4* __restrict__ proj,
                                                    float4* __restrict__ bin, uint8_t* __restrict__ vis_flags,
                                                    uint8_t* __restrict__ union_flags) {
  const int64_t i = int64_t(blockIdx.x) * kPT + threadIdx.x;
  if (i >= n) return;
  const uint32_t off4 = uint32_t(i) << 2;
  float p[59];
#pragma unroll
  for (int k = 0; k < 59; ++k) p[k] = *plane_elem(params, ld, k, off4);
  float4 q[4];
  const bool visible = project_record(p, cam, q);
  float4* r = proj + 4 * i;
  r[0] = q[0];
  r[1] = q[1];
  r[2] = q[2];
  r[3] = q[3];
  if (bin != nullptr) bin[i] = q[3];
  vis_flags[i] = visible ? 1 : 0;
  if (union_flags != nullptr && visible) union_flags[i] = 1;
}

using ArgPreViews = const __attribute__((address_space(4))) PreViews;

// Several views at once: each thread reads its Gaussian's 59 parameters
// once and projects them with every camera in turn (the same record code
// as k_preprocess, so each view's records and flags are bit for bit what
// k_preprocess writes).  The cameras are read in place from the
// kernel-argument segment (scalar loads; the struct is the kernel's only
// argument, at the segment's start).
// (A grid smaller than n / kPT workgroups walks the Gaussians with a
// stride: fewer loads in flight, a smaller share of the HBM bandwidth.)
__global__ __launch_bounds__(kPT) void k_preprocess_views(PreViews pv, const float* __restrict__ params, int64_t n,
                                                          int64_t ld, uint8_t* __restrict__ union_flags) {
  (void)pv;
  ArgPreViews* a = (ArgPreViews*)__builtin_amdgcn_kernarg_segment_ptr();
  for (int64_t i = int64_t(blockIdx.x) * kPT + threadIdx.x; i < n; i += int64_t(gridDim.x) * kPT) {
  const uint32_t off4 = uint32_t(i) << 2;
  float p[59];
#pragma unroll
  for (int k = 0; k < 59; ++k) p[k] = *plane_elem(params, ld, k, off4);
  bool any = false;
  const int nv = a->count;
  for (int w = 0; w < nv; ++w) {
    CamArgs cam;
#pragma unroll
    for (int j = 0; j < 9; ++j) cam.R[j] = a->cam[w].R[j];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      cam.t[j] = a->cam[w].t[j];
      cam.campos[j] = a->cam[w].campos[j];
    }
    cam.fx = a->cam[w].fx;
    cam.fy = a->cam[w].fy;
    cam.cx = a->cam[w].cx;
    cam.cy = a->cam[w].cy;
    cam.near_z = a->cam[w].near_z;
    cam.width = a->cam[w].width;
    cam.height = a->cam[w].height;
    cam.tiles_x = a->cam[w].tiles_x;
    cam.tiles_y = a->cam[w].tiles_y;
    float4 q[4];
    const bool visible = project_record(p, cam, q);
    float4* r = a->proj[w] + 4 * i;
    r[0] = q[0];
    r[1] = q[1];
    r[2] = q[2];
    r[3] = q[3];
    if (a->bin[w] != nullptr) a->bin[w][i] = q[3];
    a->flags[w][i] = visible ? 1 : 0;
    any = any || visible;
  }
  if (union_flags != nullptr && any) union_flags[i] = 1;
  }
}

}  // namespace

size_t preprocess_views_ws_bytes(int64_t n, int32_t num_views) {
  return size_t(num_views) * align_up(size_t(n), 256) + compact_ws_bytes(n);
}

hipError_t launch_preprocess_views(const float* params, int64_t n, int64_t ld, const CamArgs* cams, int32_t num_views,
                                   float* const* proj, float* const* proj_bin, int32_t* const* vis_idx,
                                   int64_t* vis_count, uint8_t* union_flags, int32_t max_workgroups, void* ws,
                                   hipStream_t st) {
  if (num_views <= 0) return hipSuccess;
  PreViews pv{};
  pv.count = num_views;
  uint8_t* const flags = static_cast<uint8_t*>(ws);
  for (int32_t w = 0; w < num_views; ++w) {
    pv.cam[w] = cams[w];
    pv.proj[w] = reinterpret_cast<float4*>(proj[w]);
    pv.bin[w] = proj_bin != nullptr ? reinterpret_cast<float4*>(proj_bin[w]) : nullptr;
    pv.flags[w] = flags + size_t(w) * align_up(size_t(n), 256);
  }
  void* cws = static_cast<char*>(ws) + size_t(num_views) * align_up(size_t(n), 256);
  if (n > 0) {
    int64_t grid = (n + kPT - 1) / kPT;
    if (max_workgroups > 0 && grid > max_workgroups) grid = max_workgroups;
    k_preprocess_views<<<unsigned(grid), kPT, 0, st>>>(pv, params, n, ld, union_flags);
  }
  hipError_t e = hipGetLastError();
  // the views' lists one after another (they share the compaction's counts)
  for (int32_t w = 0; w < num_views && e == hipSuccess; ++w)
    e = launch_compact(pv.flags[w], n, vis_idx[w], vis_count + w, false, cws, st);
  return e;
}

size_t preprocess_ws_bytes(int64_t n) {
  return align_up(size_t(n), 256) + compact_ws_bytes(n);
}

hipError_t launch_preprocess(const float* params, int64_t n, int64_t ld, const CamArgs& cam,
                             float* proj, float* proj_bin, int32_t* vis_idx, int64_t* vis_count,
                             uint8_t* union_flags, void* ws, hipStream_t st) {
  uint8_t* flags = static_cast<uint8_t*>(ws);
  void* cws = static_cast<char*>(ws) + align_up(size_t(n), 256);
  if (n > 0) {
    const unsigned grid = unsigned((n + kPT - 1) / kPT);
    k_preprocess<<<grid, kPT, 0, st>>>(params, n, ld, cam, reinterpret_cast<float4*>(proj),
                                       reinterpret_cast<float4*>(proj_bin), flags, union_flags);
  }
  return launch_compact(flags, n, vis_idx, vis_count, false, cws, st);
}

}  // namespace gs
