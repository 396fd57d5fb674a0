// Pieces shared by the forward and backward rasterisers.
//
// Work layout: four waves (64 lanes each) per 16x16 tile, wave q owning the
// tile's 8x8 quarter q (x + 8 (q & 1), y + 8 (q >> 1)); lane l owns the
// pixel at offset (l & 7, l >> 3) of it.  The tile's depth-sorted list is
// consumed in chunks of 64 entries: lane l stages entry l's record in LDS
// and tests the Gaussian's alpha >= 1/255 footprint box against the
// quarters; one ballot gives the 64-bit set of chunk entries that can
// reach the wave's quarter.  The loop then visits only set bits (scalar
// bit scans), so Gaussians that cannot reach a quarter cost it no vector
// work.
#pragma once

#include "gs_device.hpp"

namespace gs {

constexpr int kChunk = 64;

// Waves (one per quarter) per tile.
constexpr int kWPT = 4;

// Workgroup -> (tile, quarter).  Tiles are taken in `order` (longest
// lists first) when given, so the heavy ones start early and light ones
// fill the gaps.  Returns -1 for workgroups past the end.
__device__ __forceinline__ int order_tile(const uint32_t* __restrict__ order, int nT, int& q0) {
  const int rank = int(blockIdx.x) / kWPT;
  q0 = int(blockIdx.x) % kWPT;
  if (rank >= nT) return -1;
  return order != nullptr ? int(order[rank]) : rank;
}

inline unsigned raster_grid(int nT) { return unsigned(nT * kWPT); }

// e^x for x in [-5.6, 0]: the written exponential without its range
// checks (which never trigger there), so the same bits as pexp.
__device__ __forceinline__ float pexp_core(float x) {
  const float kf = rintf(x * 1.44269504088896341f);
  float r = fmaf(-kf, 0.693145751953125f, x);
  r = fmaf(-kf, 1.428606820309417232e-6f, r);
  float p = 1.0f / 5040.0f;
  p = fmaf(p, r, 1.0f / 720.0f);
  p = fmaf(p, r, 1.0f / 120.0f);
  p = fmaf(p, r, 1.0f / 24.0f);
  p = fmaf(p, r, 1.0f / 6.0f);
  p = fmaf(p, r, 0.5f);
  p = fmaf(p, r, 1.0f);
  p = fmaf(p, r, 1.0f);
  return ldexpf(p, static_cast<int>(kf));
}

// A Gaussian as the rasterisers read it from LDS: (u, v, -A/2, -B),
// (-C/2, opacity, r, g), b.
struct RasterRec {
  float4 a;
  float4 c;
  float b;
};

// One list entry's record as loaded from HBM: the first 11 words of the
// projected record (u, v, A, B | C, opacity, r, g | b, cull extent x, y)
// and the Gaussian's index (-1: no entry).
struct EntryRec {
  float4 q0, q1;
  float b, ex, ey;
  int32_t g;
};

__device__ __forceinline__ int32_t load_index(const int32_t* __restrict__ vals, uint32_t j, bool valid) {
  return valid ? vals[j] : -1;
}

__device__ __forceinline__ EntryRec load_entry(const float4* __restrict__ proj, int32_t g) {
  EntryRec r;
  r.g = g;
  if (g >= 0) {
    const float4* q = proj + 4 * int64_t(g);
    r.q0 = q[0];
    r.q1 = q[1];
    const float4 q2 = q[2];
    r.b = q2.x;
    r.ex = q2.y;
    r.ey = q2.z;
  } else {
    r.q0 = r.q1 = make_float4(0.f, 0.f, 0.f, 0.f);
    r.b = r.ex = r.ey = 0.f;
  }
  return r;
}

// The chunk is consumed while the next one is in flight: the records of
// chunk c + 1 and the list indices of chunk c + 2 are loaded before chunk c
// is staged, so the two dependent HBM round trips (index, then record) of
// a chunk overlap the compositing of the one before it.
//
// Stage a loaded entry (if any) into LDS slot `lane` and return its 4-bit
// quarter-overlap mask: the Gaussian's alpha >= 1/255 box
// [u - ex, u + ex] x [v - ey, v + ey] against the quarters' pixel-centre
// ranges [b0 + 8k, b0 + 8k + 7].  bx0/by0: pixel-centre coordinate of the
// tile's first pixel.
__device__ __forceinline__ uint32_t stage_entry(const EntryRec& r, float bx0, float by0, float4* s_a, float4* s_c,
                                                float* s_b, int32_t* s_g, int lane) {
  uint32_t m = 0;
  if (r.g >= 0) {
    s_a[lane] = make_float4(r.q0.x, r.q0.y, -0.5f * r.q0.z, -r.q0.w);
    s_c[lane] = make_float4(-0.5f * r.q1.x, r.q1.y, r.q1.z, r.q1.w);
    s_b[lane] = r.b;
    if (s_g != nullptr) s_g[lane] = r.g;
    const float lx = r.q0.x - r.ex, hx = r.q0.x + r.ex, ly = r.q0.y - r.ey, hy = r.q0.y + r.ey;
    const bool x0 = hx >= bx0 && lx <= bx0 + 7.0f;
    const bool x1 = hx >= bx0 + 8.0f && lx <= bx0 + 15.0f;
    const bool y0 = hy >= by0 && ly <= by0 + 7.0f;
    const bool y1 = hy >= by0 + 8.0f && ly <= by0 + 15.0f;
    m = uint32_t(x0 && y0) | (uint32_t(x1 && y0) << 1) | (uint32_t(x0 && y1) << 2) | (uint32_t(x1 && y1) << 3);
  }
  return m;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) {
    const uint32_t o = uint32_t(__shfl_xor(int(v), d, 64));
    v = o > v ? o : v;
  }
  return v;
}

}  // namespace gs
