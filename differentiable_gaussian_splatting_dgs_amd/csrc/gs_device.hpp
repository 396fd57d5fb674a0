// Device-side helpers shared by the HIP kernels of libgs (gfx950, wave64).
//
// The fp32 arithmetic here follows the canonical operation order of the
// projection and compositing rules (explicit fmaf, IEEE division and
// square root, no contraction: the library is built with
// -ffp-contract=off), so every discrete decision -- culling, radius, tile
// rectangle, alpha skip, transmittance stop, colour clamp -- is taken on
// exactly the same fp32 values as the checker's.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gs_internal.h"

namespace gs {

constexpr int kTile = 16;          // 16x16 pixel tiles (Grendel-GS notes, pixel-wise distribution)
constexpr int kBlock = 256;        // one thread per tile pixel in the rasterisers
constexpr int kRecWords = 16;      // 32-bit words per projected record

// Projected record of one Gaussian, 16 words (64 B, float4-aligned):
//   q0 = (u, v, conic A, conic B)        q1 = (conic C, opacity, r, g)
//   q2 = (b, cull_ex, cull_ey, radius)   q3 = (depth, rect_x, rect_y, tiles)
// rect_x = x0 | x1 << 16, rect_y = y0 | y1 << 16 (half-open tile ranges);
// radius and tiles are integers stored bitwise; cull_ex/ey are half-extents
// outside which the Gaussian's alpha is provably below 1/255.
enum : int {
  kU = 0, kV, kA, kB, kC, kOpac, kR, kG, kBl, kCullX, kCullY, kRadius,
  kDepth, kRectX, kRectY, kTiles
};

// ---------------------------------------------------------------------------
// Written exponential: Cody-Waite reduction with ln 2 split into a 16-bit
// head and a tail, degree-7 Taylor polynomial of e^r by fmaf Horner, 2^k
// scaling.  NaN -> NaN, x < -87 -> 0, x > 88 -> +inf.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float pexp(float x) {
  if (x != x) return x;
  if (x < -87.0f) return 0.0f;
  if (x > 88.0f) return __builtin_inff();
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

// Real SH normalisation constants (degree <= 3, no Condon-Shortley phase),
// fp64 decimal rounded once to fp32.
#define GS_SH_C0 ((float)0.28209479177387814)
#define GS_SH_C1 ((float)0.48860251190291992)
#define GS_SH_C2A ((float)1.0925484305920792)
#define GS_SH_C2B ((float)0.31539156525252005)
#define GS_SH_C2C ((float)0.54627421529603959)
#define GS_SH_C3A ((float)0.59004358992664352)
#define GS_SH_C3B ((float)2.8906114426405538)
#define GS_SH_C3C ((float)0.45704579946446572)
#define GS_SH_C3D ((float)0.37317633259011540)
#define GS_SH_C3E ((float)1.4453057213202769)

__device__ __forceinline__ void sh_eval(float x, float y, float z, float Y[16]) {
  const float xx = x * x, yy = y * y, zz = z * z;
  const float xy = x * y, yz = y * z, xz = x * z;
  Y[0] = GS_SH_C0;
  Y[1] = GS_SH_C1 * y;
  Y[2] = GS_SH_C1 * z;
  Y[3] = GS_SH_C1 * x;
  Y[4] = GS_SH_C2A * xy;
  Y[5] = GS_SH_C2A * yz;
  Y[6] = GS_SH_C2B * fmaf(3.0f, zz, -1.0f);
  Y[7] = GS_SH_C2A * xz;
  Y[8] = GS_SH_C2C * (xx - yy);
  Y[9] = (GS_SH_C3A * y) * fmaf(3.0f, xx, -yy);
  Y[10] = (GS_SH_C3B * xy) * z;
  Y[11] = (GS_SH_C3C * y) * fmaf(5.0f, zz, -1.0f);
  Y[12] = (GS_SH_C3D * z) * fmaf(5.0f, zz, -3.0f);
  Y[13] = (GS_SH_C3C * x) * fmaf(5.0f, zz, -1.0f);
  Y[14] = (GS_SH_C3E * z) * (xx - yy);
  Y[15] = (GS_SH_C3A * x) * fmaf(-3.0f, yy, xx);
}

__device__ __forceinline__ bool isfin(float v) { return __builtin_isfinite(v); }

// Forward projection values of one Gaussian that the backward also needs.
struct Fwd {
  float tx, ty, tz, iz, ux, uy;
  float s[3];
  float qn, w, x, y, z;          // quaternion norm^2 and unit quaternion
  float r[9];                    // rotation of the unit quaternion, row-major
  float S[6];                    // Sigma: 00 01 02 11 12 22
  float T[6];                    // T = J R: rows (T00 T01 T02), (T10 T11 T12)
  float a, b, c, det;            // screen covariance incl. 0.3 dilation
  float A, B, Cc;                // conic
  float u, v, rad;               // mean and radius (float)
  float dir[3], dn;              // unit view direction, |x - campos|
  float raw[3];                  // SH(d) + 1/2
  float opac;
  bool visible;
  int x0, y0, x1, y1;
};

__device__ __forceinline__ float clamp_tiles(float v, int hi) {
  return v < 0.0f ? 0.0f : (v > float(hi) ? float(hi) : v);
}

// Canonical fp32 projection (EWA local-affine, 0.3 dilation, 3-sigma radius,
// 16x16 tile rectangle, SH colour, sigmoid opacity).  `p` holds the 59
// parameters of the Gaussian.
__device__ __forceinline__ void project(const float* __restrict__ p, const CamArgs& cam, Fwd& f) {
  const float R0 = cam.R[0], R1 = cam.R[1], R2 = cam.R[2];
  const float R3 = cam.R[3], R4 = cam.R[4], R5 = cam.R[5];
  const float R6 = cam.R[6], R7 = cam.R[7], R8 = cam.R[8];
  const float X = p[0], Y = p[1], Z = p[2];
  bool ok = true;
#pragma unroll
  for (int k = 0; k < 59; ++k) ok = ok && isfin(p[k]);
  f.tx = fmaf(R2, Z, fmaf(R1, Y, R0 * X)) + cam.t[0];
  f.ty = fmaf(R5, Z, fmaf(R4, Y, R3 * X)) + cam.t[1];
  f.tz = fmaf(R8, Z, fmaf(R7, Y, R6 * X)) + cam.t[2];
  ok = ok && f.tz > cam.near_z;
  f.s[0] = pexp(p[3]);
  f.s[1] = pexp(p[4]);
  f.s[2] = pexp(p[5]);
  const float qw = p[6], qx = p[7], qy = p[8], qz = p[9];
  f.qn = fmaf(qz, qz, fmaf(qy, qy, fmaf(qx, qx, qw * qw)));
  ok = ok && f.qn > 0.0f && isfin(f.qn);
  const float qi = 1.0f / sqrtf(f.qn);
  const float w = qw * qi, x = qx * qi, y = qy * qi, z = qz * qi;
  f.w = w; f.x = x; f.y = y; f.z = z;
  const float xx = x * x, yy = y * y, zz = z * z;
  const float xy = x * y, xz = x * z, yz = y * z;
  const float wx = w * x, wy = w * y, wz = w * z;
  float* r = f.r;
  r[0] = 1.0f - 2.0f * (yy + zz); r[1] = 2.0f * (xy - wz); r[2] = 2.0f * (xz + wy);
  r[3] = 2.0f * (xy + wz); r[4] = 1.0f - 2.0f * (xx + zz); r[5] = 2.0f * (yz - wx);
  r[6] = 2.0f * (xz - wy); r[7] = 2.0f * (yz + wx); r[8] = 1.0f - 2.0f * (xx + yy);
  const float m00 = r[0] * f.s[0], m01 = r[1] * f.s[1], m02 = r[2] * f.s[2];
  const float m10 = r[3] * f.s[0], m11 = r[4] * f.s[1], m12 = r[5] * f.s[2];
  const float m20 = r[6] * f.s[0], m21 = r[7] * f.s[1], m22 = r[8] * f.s[2];
  const float S00 = fmaf(m02, m02, fmaf(m01, m01, m00 * m00));
  const float S01 = fmaf(m02, m12, fmaf(m01, m11, m00 * m10));
  const float S02 = fmaf(m02, m22, fmaf(m01, m21, m00 * m20));
  const float S11 = fmaf(m12, m12, fmaf(m11, m11, m10 * m10));
  const float S12 = fmaf(m12, m22, fmaf(m11, m21, m10 * m20));
  const float S22 = fmaf(m22, m22, fmaf(m21, m21, m20 * m20));
  f.S[0] = S00; f.S[1] = S01; f.S[2] = S02; f.S[3] = S11; f.S[4] = S12; f.S[5] = S22;
  f.iz = 1.0f / f.tz;
  f.ux = f.tx * f.iz;
  f.uy = f.ty * f.iz;
  const float jx = cam.fx * f.iz, jy = cam.fy * f.iz;
  const float T00 = jx * fmaf(-f.ux, R6, R0), T01 = jx * fmaf(-f.ux, R7, R1), T02 = jx * fmaf(-f.ux, R8, R2);
  const float T10 = jy * fmaf(-f.uy, R6, R3), T11 = jy * fmaf(-f.uy, R7, R4), T12 = jy * fmaf(-f.uy, R8, R5);
  f.T[0] = T00; f.T[1] = T01; f.T[2] = T02; f.T[3] = T10; f.T[4] = T11; f.T[5] = T12;
  const float a00 = fmaf(T02, S02, fmaf(T01, S01, T00 * S00));
  const float a01 = fmaf(T02, S12, fmaf(T01, S11, T00 * S01));
  const float a02 = fmaf(T02, S22, fmaf(T01, S12, T00 * S02));
  const float a10 = fmaf(T12, S02, fmaf(T11, S01, T10 * S00));
  const float a11 = fmaf(T12, S12, fmaf(T11, S11, T10 * S01));
  const float a12 = fmaf(T12, S22, fmaf(T11, S12, T10 * S02));
  const float c00 = fmaf(a02, T02, fmaf(a01, T01, a00 * T00));
  const float c01 = fmaf(a02, T12, fmaf(a01, T11, a00 * T10));
  const float c11 = fmaf(a12, T12, fmaf(a11, T11, a10 * T10));
  f.a = c00 + 0.3f;
  f.b = c01;
  f.c = c11 + 0.3f;
  f.det = fmaf(f.a, f.c, -(f.b * f.b));
  ok = ok && f.det > 0.0f && isfin(f.det);
  const float idet = 1.0f / f.det;
  f.A = f.c * idet;
  f.B = -f.b * idet;
  f.Cc = f.a * idet;
  const float mid = 0.5f * (f.a + f.c);
  float disc = fmaf(mid, mid, -f.det);
  disc = disc > 0.0f ? disc : 0.0f;
  const float lam = mid + sqrtf(disc);
  f.rad = ceilf(3.0f * sqrtf(lam));
  f.u = fmaf(cam.fx, f.ux, cam.cx);
  f.v = fmaf(cam.fy, f.uy, cam.cy);
  const float fx0 = clamp_tiles(floorf((f.u - f.rad) * 0.0625f), cam.tiles_x);
  const float fx1 = clamp_tiles(floorf((f.u + f.rad) * 0.0625f) + 1.0f, cam.tiles_x);
  const float fy0 = clamp_tiles(floorf((f.v - f.rad) * 0.0625f), cam.tiles_y);
  const float fy1 = clamp_tiles(floorf((f.v + f.rad) * 0.0625f) + 1.0f, cam.tiles_y);
  ok = ok && isfin(f.u) && isfin(f.v) && isfin(f.rad) && isfin(f.A) && isfin(f.B) && isfin(f.Cc);
  const float dx = X - cam.campos[0], dy = Y - cam.campos[1], dz = Z - cam.campos[2];
  f.dn = sqrtf(fmaf(dz, dz, fmaf(dy, dy, dx * dx)));
  const float idn = 1.0f / f.dn;
  f.dir[0] = dx * idn; f.dir[1] = dy * idn; f.dir[2] = dz * idn;
  float Yb[16];
  sh_eval(f.dir[0], f.dir[1], f.dir[2], Yb);
#pragma unroll
  for (int ch = 0; ch < 3; ++ch) {
    float acc = Yb[0] * p[11 + ch];
#pragma unroll
    for (int k = 1; k < 16; ++k) acc = fmaf(Yb[k], p[11 + 3 * k + ch], acc);
    f.raw[ch] = acc + 0.5f;
    ok = ok && isfin(f.raw[ch]);
  }
  f.opac = 1.0f / (1.0f + pexp(-p[10]));
  f.x0 = 0; f.y0 = 0; f.x1 = 0; f.y1 = 0;
  if (ok) {
    f.x0 = int(fx0); f.x1 = int(fx1); f.y0 = int(fy0); f.y1 = int(fy1);
    ok = (f.x1 - f.x0) > 0 && (f.y1 - f.y0) > 0;
  }
  f.visible = ok;
}

// Element (k, i) of a plane-major [planes][ld] fp32 array, given i as the
// byte offset i * 4 (i < 2^30, so it fits 32 bits): the plane's start is the
// same for every lane, so the access is one global load or store of a
// scalar-register base plus a 32-bit lane offset, with no 64-bit address
// arithmetic per lane.  (The base passes through an empty asm that pins it
// to scalar registers, so the compiler cannot fold the lane offset into a
// per-lane 64-bit address instead.)
template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T* plane_elem(T* base, int64_t ld, int k,
                                                                          uint32_t off4) {
  using G = __attribute__((address_space(1))) T;
  using GB = typename std::conditional<std::is_const<T>::value, const __attribute__((address_space(1))) char,
                                       __attribute__((address_space(1))) char>::type;
  uint64_t pb = reinterpret_cast<uint64_t>(base + int64_t(k) * ld);
  asm volatile("" : "+s"(pb));
  return reinterpret_cast<G*>(reinterpret_cast<GB*>(pb) + off4);
}

// ---------------------------------------------------------------------------
// wave64 helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// number of set bits of `mask` below the calling lane
__device__ __forceinline__ int count_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Lanes whose `d` (an nbits-bit value) equals the calling lane's, among `active`.
template <int NBITS>
__device__ __forceinline__ uint64_t match_bits(uint32_t d, uint64_t active) {
  uint64_t m = active;
#pragma unroll
  for (int b = 0; b < NBITS; ++b) {
    const bool bit = (d >> b) & 1u;
    const uint64_t bb = ballot(bit);
    m &= bit ? bb : ~bb;
  }
  return m;
}

// Sum of v over the 64 lanes; the total lands in lane 63 (other lanes hold
// partial sums).  DPP row shuffles within 16-lane rows, then row
// broadcasts 15 and 31 (GFX9 family).
__device__ __forceinline__ float wave_sum_to_lane63(float v) {
  int x = __builtin_bit_cast(int, v);
  // quad_perm [1,0,3,2]
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));
  x = __builtin_bit_cast(int, v);
  // quad_perm [2,3,0,1]
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));
  x = __builtin_bit_cast(int, v);
  // row_half_mirror
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false));
  x = __builtin_bit_cast(int, v);
  // row_mirror
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false));
  x = __builtin_bit_cast(int, v);
  // row_bcast:15 into rows 1 and 3
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false));
  x = __builtin_bit_cast(int, v);
  // row_bcast:31 into rows 2 and 3
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false));
  return v;
}

}  // namespace gs
