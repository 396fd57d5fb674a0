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
#include "gs_device.hpp"

namespace gs {
namespace {

constexpr int kPT = 256;

// Culling half-extents of a Gaussian's alpha >= 1/255 footprint, used only
// to skip 8x8 pixel blocks in the rasterisers.  alpha = o e^power >= 1/255
// needs -power <= tau = ln(255 o).  The screen ellipse {d : d^T Q d <= 2 tau}
// has bounding half-widths sqrt(2 tau a), sqrt(2 tau c) with (a, b, c) the
// screen covariance.  The fp32 evaluation of power differs from the exact
// quadratic form by at most 8 eps kappa |power| (kappa = condition number,
// <= (r/3)^2 / 0.3 <= 9.3e4 for r <= 500, i.e. < 4.5%), so tau is inflated
// by 10% (+0.1); Gaussians with r > 500 are never culled.
__device__ __forceinline__ void cull_extent(float o, float a, float c, float rad, float& ex, float& ey) {
  if (!(o * 255.0f > 1.0f)) {
    ex = -__builtin_inff();     // an empty footprint: every block test culls
    ey = -__builtin_inff();
    return;
  }
  if (rad > 500.0f) {
    ex = __builtin_inff();
    ey = __builtin_inff();
    return;
  }
  const float tau = 1.1f * logf(255.0f * o) + 0.1f;
  ex = sqrtf(2.0f * tau * a) * 1.001f + 0.01f;
  ey = sqrtf(2.0f * tau * c) * 1.001f + 0.01f;
}

__global__ __launch_bounds__(kPT) void k_preprocess(const float* __restrict__ params, int64_t n, int64_t ld,
                                                    CamArgs cam, float4* __restrict__ proj,
                                                    uint8_t* __restrict__ vis_flags,
                                                    uint8_t* __restrict__ union_flags) {
  const int64_t i = int64_t(blockIdx.x) * kPT + threadIdx.x;
  if (i >= n) return;
  float p[59];
#pragma unroll
  for (int k = 0; k < 59; ++k) p[k] = params[int64_t(k) * ld + i];
  Fwd f;
  project(p, cam, f);
  float4 q0, q1, q2, q3;
  if (f.visible) {
    const float rgb0 = f.raw[0] > 0.0f ? f.raw[0] : 0.0f;
    const float rgb1 = f.raw[1] > 0.0f ? f.raw[1] : 0.0f;
    const float rgb2 = f.raw[2] > 0.0f ? f.raw[2] : 0.0f;
    float ex, ey;
    cull_extent(f.opac, f.a, f.c, f.rad, ex, ey);
    const int rad = int(fminf(f.rad, 2147483520.0f));
    const uint32_t tiles = uint32_t(f.x1 - f.x0) * uint32_t(f.y1 - f.y0);
    q0 = make_float4(f.u, f.v, f.A, f.B);
    q1 = make_float4(f.Cc, f.opac, rgb0, rgb1);
    q2 = make_float4(rgb2, ex, ey, __builtin_bit_cast(float, rad));
    q3 = make_float4(f.tz, __builtin_bit_cast(float, uint32_t(f.x0) | (uint32_t(f.x1) << 16)),
                     __builtin_bit_cast(float, uint32_t(f.y0) | (uint32_t(f.y1) << 16)),
                     __builtin_bit_cast(float, tiles));
  } else {
    q0 = make_float4(0.f, 0.f, 0.f, 0.f);
    q1 = q0;
    q2 = make_float4(0.f, -__builtin_inff(), -__builtin_inff(), 0.f);
    q3 = make_float4(f.tz, 0.f, 0.f, 0.f);
  }
  float4* r = proj + 4 * i;
  r[0] = q0;
  r[1] = q1;
  r[2] = q2;
  r[3] = q3;
  vis_flags[i] = f.visible ? 1 : 0;
  if (union_flags != nullptr && f.visible) union_flags[i] = 1;
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
