// The projected record of one Gaussian (the "Gaussian transform" of the
// Grendel-GS notes' training pipeline: 2D mean, conic, opacity, colour,
// cover radius, depth, tile rectangle), as the preprocess writes it and as
// the optimiser pass writes it for the next view after updating a row.
#pragma once

#include "gs_device.hpp"

namespace gs {

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

// Projects the 59 parameters `p` with `cam` into the record's four float4
// words (u, v, A, B | C, opacity, r, g | b, cull extent x, y, radius bits |
// depth, x0 | x1 << 16, y0 | y1 << 16, tile count); returns visibility.
__device__ __forceinline__ bool project_record(const float (&p)[59], const CamArgs& cam, float4 (&q)[4]) {
  Fwd f;
  project(p, cam, f);
  if (f.visible) {
    const float rgb0 = f.raw[0] > 0.0f ? f.raw[0] : 0.0f;
    const float rgb1 = f.raw[1] > 0.0f ? f.raw[1] : 0.0f;
    const float rgb2 = f.raw[2] > 0.0f ? f.raw[2] : 0.0f;
    float ex, ey;
    cull_extent(f.opac, f.a, f.c, f.rad, ex, ey);
    const int rad = int(fminf(f.rad, 2147483520.0f));
    const uint32_t tiles = uint32_t(f.x1 - f.x0) * uint32_t(f.y1 - f.y0);
    q[0] = make_float4(f.u, f.v, f.A, f.B);
    q[1] = make_float4(f.Cc, f.opac, rgb0, rgb1);
    q[2] = make_float4(rgb2, ex, ey, __builtin_bit_cast(float, rad));
    q[3] = make_float4(f.tz, __builtin_bit_cast(float, uint32_t(f.x0) | (uint32_t(f.x1) << 16)),
                       __builtin_bit_cast(float, uint32_t(f.y0) | (uint32_t(f.y1) << 16)),
                       __builtin_bit_cast(float, tiles));
  } else {
    q[0] = make_float4(0.f, 0.f, 0.f, 0.f);
    q[1] = q[0];
    q[2] = make_float4(0.f, -__builtin_inff(), -__builtin_inff(), 0.f);
    q[3] = make_float4(f.tz, 0.f, 0.f, 0.f);
  }
  return f.visible;
}

}  // namespace gs
