// Projection of every Gaussian to screen space (the "Gaussian transform" of
// the Grendel-GS notes' training pipeline: 2D mean, depth, cover radius,
// colour), plus the per-view visible-index list the Odin summary page's
// "Background and motivation" describes (each view touches a sparse,
// view-dependent set of primitives).
//
// One thread per Gaussian.  Parameters are plane-major [59][ld] fp32, so
// each of the 59 loads is coalesced across the wave.  Output is one 64-byte
// record per Gaussian (four float4 stores) plus a visibility byte that the
// compaction turns into the ascending visible list.
#include "project_record.hpp"

namespace gs {
namespace {

constexpr int kPT = 256;

__global__ __launch_bounds__(kPT) void k_preprocess(const float* __restrict__ params, int64_t n, int64_t ld,
                                                    CamArgs cam, float4* __restrict__ proj,
                                                    uint8_t* __restrict__ vis_flags,
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
  vis_flags[i] = visible ? 1 : 0;
  if (union_flags != nullptr && visible) union_flags[i] = 1;
}

}  // namespace

size_t preprocess_ws_bytes(int64_t n) {
  return align_up(size_t(n), 256) + compact_ws_bytes(n);
}

hipError_t launch_preprocess(const float* params, int64_t n, int64_t ld, const CamArgs& cam,
                             float* proj, int32_t* vis_idx, int64_t* vis_count,
                             uint8_t* union_flags, void* ws, hipStream_t st) {
  uint8_t* flags = static_cast<uint8_t*>(ws);
  void* cws = static_cast<char*>(ws) + align_up(size_t(n), 256);
  if (n > 0) {
    const unsigned grid = unsigned((n + kPT - 1) / kPT);
    k_preprocess<<<grid, kPT, 0, st>>>(params, n, ld, cam, reinterpret_cast<float4*>(proj), flags,
                                       union_flags);
  }
  return launch_compact(flags, n, vis_idx, vis_count, false, cws, st);
}

}  // namespace gs
