// CPU oracle for one 3D Gaussian Splatting training step.
//
// TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
// call this file; only the tests, the smoke check and the CPU-baseline leg
// of the benchmark use it.  It shares no code with the HIP library.
//
// What it computes follows the Grendel-GS notes ("Grendel-GS: On Scaling Up
// 3D Gaussian Splatting Training"), section "Background -- what 3D Gaussian
// splatting is": the 59-float primitive (parameter table) and the training
// pipeline (Gaussian transform -> per-pixel cover / depth sort / alpha
// composite -> L1 + SSIM loss -> back-propagation), with the Odin summary
// page ("Odin: Primitive-Level Synchronization ...", section "Background and
// motivation") adding that a view reads and writes only a sparse,
// view-dependent set of primitive indices.  The pages give no formulas; every
// formula below is the standard 3D Gaussian Splatting reading of those
// steps, and where the pages are silent the reading taken is the one listed
// in the readings table of the design notes.
//
// Plain on purpose: one Gaussian / one pixel / one pair at a time, no
// blocking or fusion, library sort, direct (non-separable) SSIM window.
// OpenMP only splits independent iterations; every reduction is done in a
// fixed order, so results do not depend on the thread count.
//
// Two precisions:
//  * fp32 "canonical" -- the forward quantities that feed a discrete decision
//    (culling, radius, tile rectangle, alpha skip, transmittance stop, colour
//    clamp) are evaluated in fp32 with a fixed operation order, explicit
//    fmaf, IEEE division and square root, and the written exponentials
//    `pexp` and (compositing weight) `aexp` below.  The GPU library obeys
//    the same contract, so these
//    decisions, the sort keys and the image agree bit for bit.
//  * fp64 -- the smooth function with every discrete decision frozen at the
//    fp32 run's outcome.  Its gradient is the exact derivative the backward
//    pass must reproduce; central differences pin it.
//
// Parity pins: see tests/test_oracle_*.py.  Functions without a pin are
// marked "parity unpinned".

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <type_traits>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

extern "C" {

struct or_camera {
  int32_t width, height;
  float fx, fy, cx, cy;
  float R[9];        // world -> camera rotation, row-major
  float t[3];        // world -> camera translation
  float campos[3];   // camera centre, world
  float near_z;      // cull plane (camera-space z)
};

}  // extern "C"

namespace {

constexpr int kTile = 16;  // Grendel-GS notes, "Pixel-wise distribution": 16x16 pixel blocks

// ---------------------------------------------------------------------------
// The written exponential (fp32).  Cody-Waite reduction x = k ln2 + r with
// k = rint(x log2 e) and ln2 split in a 16-bit head and a tail, then the
// degree-7 Taylor polynomial of e^r on |r| <= ln2/2 by Horner with fmaf, then
// scaling by 2^k.  Truncation error r^8/8! <= 5.2e-9, below half an ulp.
// Inputs below -87 give 0 (so results are never subnormal), above 88 give
// +inf, NaN propagates.
// ---------------------------------------------------------------------------
float pexp(float x) {
  if (x != x) return x;
  if (x < -87.0f) return 0.0f;
  if (x > 88.0f) return INFINITY;
  const float kf = std::rint(x * 1.44269504088896341f);
  float r = std::fma(-kf, 0.693145751953125f, x);
  r = std::fma(-kf, 1.428606820309417232e-6f, r);
  float p = 1.0f / 5040.0f;
  p = std::fma(p, r, 1.0f / 720.0f);
  p = std::fma(p, r, 1.0f / 120.0f);
  p = std::fma(p, r, 1.0f / 24.0f);
  p = std::fma(p, r, 1.0f / 6.0f);
  p = std::fma(p, r, 0.5f);
  p = std::fma(p, r, 1.0f);
  p = std::fma(p, r, 1.0f);
  return std::ldexp(p, static_cast<int>(kf));
}

inline float xexp(float x) { return pexp(x); }
inline double xexp(double x) { return std::exp(x); }

// ---------------------------------------------------------------------------
// The compositing weight's exponential (fp32), for x in [-5.6, 0] only: the
// compositing rule never asks for it elsewhere (power > 0 and power < -5.6
// are skipped first).  2^t with t = x log2 e rounded once: t = k + f with
// k = rint(t) and f = t - k (exact, |f| <= 1/2), then 2^f by a degree-5
// polynomial 1 + f (c1 + f (c2 + f (c3 + f (c4 + f c5)))) by Horner with
// fmaf, then scaling by 2^k.  The coefficients are a near-minimax fit of
// 2^f on [-1/2, 1/2] in relative error (least squares reweighted by
// Lawson's iteration), 9.2e-8 there; with the rounding of t (at most
// 2^-21 for |t| < 8.1, a relative 3.3e-7 in 2^t) and of the evaluation the
// result is within 6e-7 relative of e^x.  Never subnormal: e^-5.6 > 2^-9.
// ---------------------------------------------------------------------------
float aexp(float x) {
  const float t = x * 1.44269504088896341f;
  const float kf = std::rint(t);
  const float f = t - kf;
  float p = 0x1.5bb9e4p-10f;
  p = std::fma(p, f, 0x1.3cea7ap-7f);
  p = std::fma(p, f, 0x1.c6b752p-5f);
  p = std::fma(p, f, 0x1.ebf9bcp-3f);
  p = std::fma(p, f, 0x1.62e42ap-1f);
  p = std::fma(p, f, 1.0f);
  return std::ldexp(p, static_cast<int>(kf));
}

// Real spherical harmonics of degree <= 3 (no Condon-Shortley phase), the
// view-dependent colour of the 48 SH coefficients in the Grendel-GS
// parameter table.  Constants are the normalisations sqrt((2l+1)/(4 pi) *
// (l-m)!/(l+m)!) (times sqrt 2 for m != 0), fp64 decimal, rounded once.
template <class F> struct SHC {
  static constexpr F c0 = F(0.28209479177387814);
  static constexpr F c1 = F(0.48860251190291992);
  static constexpr F c2a = F(1.0925484305920792);
  static constexpr F c2b = F(0.31539156525252005);
  static constexpr F c2c = F(0.54627421529603959);
  static constexpr F c3a = F(0.59004358992664352);
  static constexpr F c3b = F(2.8906114426405538);
  static constexpr F c3c = F(0.45704579946446572);
  static constexpr F c3d = F(0.37317633259011540);
  static constexpr F c3e = F(1.4453057213202769);
};

template <class F> void sh_basis(F x, F y, F z, F Y[16]) {
  using C = SHC<F>;
  const F xx = x * x, yy = y * y, zz = z * z;
  const F xy = x * y, yz = y * z, xz = x * z;
  Y[0] = C::c0;
  Y[1] = C::c1 * y;
  Y[2] = C::c1 * z;
  Y[3] = C::c1 * x;
  Y[4] = C::c2a * xy;
  Y[5] = C::c2a * yz;
  Y[6] = C::c2b * std::fma(F(3), zz, F(-1));
  Y[7] = C::c2a * xz;
  Y[8] = C::c2c * (xx - yy);
  Y[9] = (C::c3a * y) * std::fma(F(3), xx, -yy);
  Y[10] = (C::c3b * xy) * z;
  Y[11] = (C::c3c * y) * std::fma(F(5), zz, F(-1));
  Y[12] = (C::c3d * z) * std::fma(F(5), zz, F(-3));
  Y[13] = (C::c3c * x) * std::fma(F(5), zz, F(-1));
  Y[14] = (C::c3e * z) * (xx - yy);
  Y[15] = (C::c3a * x) * std::fma(F(-3), yy, xx);
}

// d Y_k / d(x, y, z), the unit-vector components taken as independent.
void sh_basis_grad(double x, double y, double z, double dY[16][3]) {
  using C = SHC<double>;
  std::memset(dY, 0, sizeof(double) * 48);
  dY[1][1] = C::c1;
  dY[2][2] = C::c1;
  dY[3][0] = C::c1;
  dY[4][0] = C::c2a * y; dY[4][1] = C::c2a * x;
  dY[5][1] = C::c2a * z; dY[5][2] = C::c2a * y;
  dY[6][2] = 6.0 * C::c2b * z;
  dY[7][0] = C::c2a * z; dY[7][2] = C::c2a * x;
  dY[8][0] = 2.0 * C::c2c * x; dY[8][1] = -2.0 * C::c2c * y;
  dY[9][0] = 6.0 * C::c3a * x * y; dY[9][1] = C::c3a * (3.0 * x * x - 3.0 * y * y);
  dY[10][0] = C::c3b * y * z; dY[10][1] = C::c3b * x * z; dY[10][2] = C::c3b * x * y;
  dY[11][1] = C::c3c * (5.0 * z * z - 1.0); dY[11][2] = 10.0 * C::c3c * y * z;
  dY[12][2] = C::c3d * (15.0 * z * z - 3.0);
  dY[13][0] = C::c3c * (5.0 * z * z - 1.0); dY[13][2] = 10.0 * C::c3c * x * z;
  dY[14][0] = 2.0 * C::c3e * x * z; dY[14][1] = -2.0 * C::c3e * y * z; dY[14][2] = C::c3e * (x * x - y * y);
  dY[15][0] = C::c3a * (3.0 * x * x - 3.0 * y * y); dY[15][1] = -6.0 * C::c3a * x * y;
}

// Magnitudes of the same polynomials: every monomial taken absolutely, so
// the result bounds what an fp32 evaluation rounds against (used by the
// error bounds of the backward).
void sh_basis_mag(double x, double y, double z, double Y[16], double dY[16][3]) {
  using C = SHC<double>;
  x = std::fabs(x); y = std::fabs(y); z = std::fabs(z);
  Y[0] = C::c0; Y[1] = C::c1 * y; Y[2] = C::c1 * z; Y[3] = C::c1 * x;
  Y[4] = C::c2a * x * y; Y[5] = C::c2a * y * z; Y[6] = C::c2b * (3 * z * z + 1); Y[7] = C::c2a * x * z;
  Y[8] = C::c2c * (x * x + y * y); Y[9] = C::c3a * y * (3 * x * x + y * y); Y[10] = C::c3b * x * y * z;
  Y[11] = C::c3c * y * (5 * z * z + 1); Y[12] = C::c3d * z * (5 * z * z + 3); Y[13] = C::c3c * x * (5 * z * z + 1);
  Y[14] = C::c3e * z * (x * x + y * y); Y[15] = C::c3a * x * (x * x + 3 * y * y);
  std::memset(dY, 0, sizeof(double) * 48);
  dY[1][1] = C::c1; dY[2][2] = C::c1; dY[3][0] = C::c1;
  dY[4][0] = C::c2a * y; dY[4][1] = C::c2a * x;
  dY[5][1] = C::c2a * z; dY[5][2] = C::c2a * y;
  dY[6][2] = 6.0 * C::c2b * z;
  dY[7][0] = C::c2a * z; dY[7][2] = C::c2a * x;
  dY[8][0] = 2.0 * C::c2c * x; dY[8][1] = 2.0 * C::c2c * y;
  dY[9][0] = 6.0 * C::c3a * x * y; dY[9][1] = C::c3a * (3.0 * x * x + 3.0 * y * y);
  dY[10][0] = C::c3b * y * z; dY[10][1] = C::c3b * x * z; dY[10][2] = C::c3b * x * y;
  dY[11][1] = C::c3c * (5.0 * z * z + 1.0); dY[11][2] = 10.0 * C::c3c * y * z;
  dY[12][2] = C::c3d * (15.0 * z * z + 3.0);
  dY[13][0] = C::c3c * (5.0 * z * z + 1.0); dY[13][2] = 10.0 * C::c3c * x * z;
  dY[14][0] = 2.0 * C::c3e * x * z; dY[14][1] = 2.0 * C::c3e * y * z; dY[14][2] = C::c3e * (x * x + y * y);
  dY[15][0] = C::c3a * (3.0 * x * x + 3.0 * y * y); dY[15][1] = 6.0 * C::c3a * x * y;
}

// ---------------------------------------------------------------------------
// Projection of one Gaussian ("Gaussian transform" of the Grendel-GS
// training pipeline: 3D Gaussian -> screen-space 2D mean, depth, cover
// radius and colour).  EWA local-affine reading: camera-space mean
// t = R x + t_c; covariance Sigma = Rq S S Rq^T with S = diag(exp(log s)) and
// Rq from the normalised quaternion; screen covariance T Sigma T^T + 0.3 I with
// T = J R and J the Jacobian of the pinhole map at t; conic = its inverse;
// radius = ceil(3 sqrt(lambda_max)); 16x16 tile rectangle of the square
// [u - r, u + r] x [v - r, v + r]; colour = max(0, SH(d) + 1/2) at the unit
// view direction d; opacity = sigmoid(logit).
// ---------------------------------------------------------------------------
template <class F> struct Proj {
  bool visible;
  F u, v, depth;
  F a, b, c;          // screen covariance incl. the 0.3 dilation
  F A, B, C;          // conic
  F opacity;
  F rgb[3];
  F rgb_raw[3];       // SH(d) + 1/2 before the clamp
  bool rgb_pos[3];    // raw colour > 0 (gradient passes)
  int32_t radius;
  int32_t rect[4];    // x0, y0, x1, y1 (half-open, tiles)
  uint32_t tiles;
  // intermediates of the forward, consumed by the backward
  F iz, ux, uy;       // 1/t_z, t_x/t_z, t_y/t_z
  F s[3];             // exp(log-scale)
  F qn, q[4];         // |q|^2 and the unit quaternion (w, x, y, z)
  F R[9];             // rotation of the unit quaternion, row-major
  F S[6];             // Sigma: 00 01 02 11 12 22
  F T[6];             // T = J R: rows (T00 T01 T02), (T10 T11 T12)
  F det;              // det of the dilated screen covariance
  F dir[3], dn;       // unit view direction and |x - campos|
};

// fp32 intermediates widened to fp64 (exact)
Proj<double> widen(const Proj<float>& f) {
  Proj<double> d;
  d.visible = f.visible;
  d.u = f.u; d.v = f.v; d.depth = f.depth;
  d.a = f.a; d.b = f.b; d.c = f.c;
  d.A = f.A; d.B = f.B; d.C = f.C;
  d.opacity = f.opacity;
  for (int k = 0; k < 3; ++k) {
    d.rgb[k] = f.rgb[k]; d.rgb_raw[k] = f.rgb_raw[k]; d.rgb_pos[k] = f.rgb_pos[k];
    d.s[k] = f.s[k]; d.dir[k] = f.dir[k];
  }
  d.radius = f.radius;
  for (int k = 0; k < 4; ++k) { d.rect[k] = f.rect[k]; d.q[k] = f.q[k]; }
  d.tiles = f.tiles;
  d.iz = f.iz; d.ux = f.ux; d.uy = f.uy; d.qn = f.qn; d.det = f.det; d.dn = f.dn;
  for (int k = 0; k < 9; ++k) d.R[k] = f.R[k];
  for (int k = 0; k < 6; ++k) { d.S[k] = f.S[k]; d.T[k] = f.T[k]; }
  return d;
}

template <class F> inline F clampf_tiles(F v, int hi) {
  return v < F(0) ? F(0) : (v > F(hi) ? F(hi) : v);
}

template <class F> inline bool finite(F v) { return std::isfinite(v); }

template <class F>
void project_one(const F p[59], const or_camera& cam, Proj<F>& o) {
  std::memset(&o, 0, sizeof(o));
  const F R0 = cam.R[0], R1 = cam.R[1], R2 = cam.R[2];
  const F R3 = cam.R[3], R4 = cam.R[4], R5 = cam.R[5];
  const F R6 = cam.R[6], R7 = cam.R[7], R8 = cam.R[8];
  const F X = p[0], Y = p[1], Z = p[2];
  const F tx = std::fma(R2, Z, std::fma(R1, Y, R0 * X)) + F(cam.t[0]);
  const F ty = std::fma(R5, Z, std::fma(R4, Y, R3 * X)) + F(cam.t[1]);
  const F tz = std::fma(R8, Z, std::fma(R7, Y, R6 * X)) + F(cam.t[2]);
  o.depth = tz;
  bool vis = tz > F(cam.near_z);

  const F s0 = xexp(p[3]), s1 = xexp(p[4]), s2 = xexp(p[5]);
  const F qw = p[6], qx = p[7], qy = p[8], qz = p[9];
  const F qn = std::fma(qz, qz, std::fma(qy, qy, std::fma(qx, qx, qw * qw)));
  vis = vis && qn > F(0) && finite(qn);
  const F qi = F(1) / std::sqrt(qn);
  const F w = qw * qi, x = qx * qi, y = qy * qi, z = qz * qi;
  o.qn = qn; o.q[0] = w; o.q[1] = x; o.q[2] = y; o.q[3] = z;
  o.s[0] = s0; o.s[1] = s1; o.s[2] = s2;
  const F xx = x * x, yy = y * y, zz = z * z;
  const F xy = x * y, xz = x * z, yz = y * z;
  const F wx = w * x, wy = w * y, wz = w * z;
  const F r00 = F(1) - F(2) * (yy + zz), r01 = F(2) * (xy - wz), r02 = F(2) * (xz + wy);
  const F r10 = F(2) * (xy + wz), r11 = F(1) - F(2) * (xx + zz), r12 = F(2) * (yz - wx);
  const F r20 = F(2) * (xz - wy), r21 = F(2) * (yz + wx), r22 = F(1) - F(2) * (xx + yy);
  o.R[0] = r00; o.R[1] = r01; o.R[2] = r02; o.R[3] = r10; o.R[4] = r11; o.R[5] = r12;
  o.R[6] = r20; o.R[7] = r21; o.R[8] = r22;
  // M = Rq diag(s)
  const F m00 = r00 * s0, m01 = r01 * s1, m02 = r02 * s2;
  const F m10 = r10 * s0, m11 = r11 * s1, m12 = r12 * s2;
  const F m20 = r20 * s0, m21 = r21 * s1, m22 = r22 * s2;
  // Sigma = M M^T
  const F S00 = std::fma(m02, m02, std::fma(m01, m01, m00 * m00));
  const F S01 = std::fma(m02, m12, std::fma(m01, m11, m00 * m10));
  const F S02 = std::fma(m02, m22, std::fma(m01, m21, m00 * m20));
  const F S11 = std::fma(m12, m12, std::fma(m11, m11, m10 * m10));
  const F S12 = std::fma(m12, m22, std::fma(m11, m21, m10 * m20));
  const F S22 = std::fma(m22, m22, std::fma(m21, m21, m20 * m20));
  o.S[0] = S00; o.S[1] = S01; o.S[2] = S02; o.S[3] = S11; o.S[4] = S12; o.S[5] = S22;
  // T = J R : rows jx (R_0k - ux R_2k), jy (R_1k - uy R_2k)
  const F iz = F(1) / tz;
  const F ux = tx * iz, uy = ty * iz;
  const F jx = F(cam.fx) * iz, jy = F(cam.fy) * iz;
  const F T00 = jx * std::fma(-ux, R6, R0), T01 = jx * std::fma(-ux, R7, R1), T02 = jx * std::fma(-ux, R8, R2);
  const F T10 = jy * std::fma(-uy, R6, R3), T11 = jy * std::fma(-uy, R7, R4), T12 = jy * std::fma(-uy, R8, R5);
  o.iz = iz; o.ux = ux; o.uy = uy;
  o.T[0] = T00; o.T[1] = T01; o.T[2] = T02; o.T[3] = T10; o.T[4] = T11; o.T[5] = T12;
  // rows of T Sigma
  const F a00 = std::fma(T02, S02, std::fma(T01, S01, T00 * S00));
  const F a01 = std::fma(T02, S12, std::fma(T01, S11, T00 * S01));
  const F a02 = std::fma(T02, S22, std::fma(T01, S12, T00 * S02));
  const F a10 = std::fma(T12, S02, std::fma(T11, S01, T10 * S00));
  const F a11 = std::fma(T12, S12, std::fma(T11, S11, T10 * S01));
  const F a12 = std::fma(T12, S22, std::fma(T11, S12, T10 * S02));
  const F c00 = std::fma(a02, T02, std::fma(a01, T01, a00 * T00));
  const F c01 = std::fma(a02, T12, std::fma(a01, T11, a00 * T10));
  const F c11 = std::fma(a12, T12, std::fma(a11, T11, a10 * T10));
  const F ca = c00 + F(0.3), cb = c01, cc = c11 + F(0.3);
  o.a = ca; o.b = cb; o.c = cc;
  const F det = std::fma(ca, cc, -(cb * cb));
  o.det = det;
  vis = vis && det > F(0) && finite(det);
  const F idet = F(1) / det;
  o.A = cc * idet;
  o.B = -cb * idet;
  o.C = ca * idet;
  const F mid = F(0.5) * (ca + cc);
  F disc = std::fma(mid, mid, -det);
  disc = disc > F(0) ? disc : F(0);
  const F lam = mid + std::sqrt(disc);
  const F rf = std::ceil(F(3) * std::sqrt(lam));
  o.u = std::fma(F(cam.fx), ux, F(cam.cx));
  o.v = std::fma(F(cam.fy), uy, F(cam.cy));
  const int TX = (cam.width + kTile - 1) / kTile, TY = (cam.height + kTile - 1) / kTile;
  const F x0 = clampf_tiles(std::floor((o.u - rf) * F(0.0625)), TX);
  const F x1 = clampf_tiles(std::floor((o.u + rf) * F(0.0625)) + F(1), TX);
  const F y0 = clampf_tiles(std::floor((o.v - rf) * F(0.0625)), TY);
  const F y1 = clampf_tiles(std::floor((o.v + rf) * F(0.0625)) + F(1), TY);
  vis = vis && finite(o.u) && finite(o.v) && finite(rf) && finite(o.A) && finite(o.B) && finite(o.C);
  // colour
  const F dx = X - F(cam.campos[0]), dy = Y - F(cam.campos[1]), dz = Z - F(cam.campos[2]);
  const F dn = std::sqrt(std::fma(dz, dz, std::fma(dy, dy, dx * dx)));
  const F idn = F(1) / dn;
  o.dn = dn;
  o.dir[0] = dx * idn; o.dir[1] = dy * idn; o.dir[2] = dz * idn;
  F Yb[16];
  sh_basis<F>(o.dir[0], o.dir[1], o.dir[2], Yb);
  for (int ch = 0; ch < 3; ++ch) {
    F acc = Yb[0] * p[11 + ch];
    for (int k = 1; k < 16; ++k) acc = std::fma(Yb[k], p[11 + 3 * k + ch], acc);
    const F raw = acc + F(0.5);
    o.rgb_raw[ch] = raw;
    o.rgb_pos[ch] = raw > F(0);
    o.rgb[ch] = raw > F(0) ? raw : F(0);
    vis = vis && finite(raw);
  }
  o.opacity = F(1) / (F(1) + xexp(-p[10]));
  vis = vis && finite(o.opacity);
  for (int k = 0; k < 59; ++k) vis = vis && finite(p[k]);
  if (vis) {
    o.rect[0] = static_cast<int32_t>(x0);
    o.rect[1] = static_cast<int32_t>(y0);
    o.rect[2] = static_cast<int32_t>(x1);
    o.rect[3] = static_cast<int32_t>(y1);
    const int64_t nt = int64_t(o.rect[2] - o.rect[0]) * int64_t(o.rect[3] - o.rect[1]);
    vis = nt > 0;
    o.tiles = vis ? static_cast<uint32_t>(nt) : 0u;
    o.radius = static_cast<int32_t>(std::min(rf, F(2147483520.0f)));
  }
  if (!vis) {
    o.rect[0] = o.rect[1] = o.rect[2] = o.rect[3] = 0;
    o.tiles = 0;
    o.radius = 0;
  }
  o.visible = vis;
}

template <class F> void load_params(const float* params, int64_t ld, int64_t i, F p[59]) {
  for (int k = 0; k < 59; ++k) p[k] = F(params[k * ld + i]);
}

// ---------------------------------------------------------------------------
// Compositing rule for one pixel against one Gaussian (fp32, the decisions).
// Returns 0 = skipped, 1 = composited, 2 = stop before compositing.
// power = -1/2 (A dx^2 + C dy^2) - B dx dy at the pixel centre, skip if
// power > 0; alpha = min(0.99, o e^power), skip if alpha < 1/255; stop if
// T (1 - alpha) < 1e-4 (standard 3DGS constants: readings table).
// ---------------------------------------------------------------------------
struct Step32 {
  int kind;
  float alpha;        // after the 0.99 clamp
  bool clamped;       // o e^power > 0.99
  float next_T;
};

inline Step32 composite_step(float u, float v, float A, float B, float C, float o,
                             float pxc, float pyc, float T) {
  Step32 s{0, 0.0f, false, T};
  const float dx = pxc - u, dy = pyc - v;
  const float hA = -0.5f * A, hC = -0.5f * C, nB = -B;
  const float power = std::fma(dx, std::fma(hA, dx, nB * dy), (hC * dy) * dy);
  // power < -5.6: o e^power < e^-5.6 < 1/255 (o <= 1), the skip below
  if (power > 0.0f || power < -5.6f) return s;
  const float araw = o * aexp(power);
  const float alpha = std::min(0.99f, araw);
  if (alpha < 1.0f / 255.0f) return s;
  const float nt = T * (1.0f - alpha);
  if (nt < 0.0001f) { s.kind = 2; return s; }
  s.kind = 1;
  s.alpha = alpha;
  s.clamped = araw > 0.99f;
  s.next_T = nt;
  return s;
}

struct ProjSoA {
  // fp32 canonical projection of all Gaussians
  std::vector<Proj<float>> g;
};

void project_all(const float* params, int64_t n, int64_t ld, const or_camera& cam,
                 std::vector<Proj<float>>& out) {
  out.resize(n);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    float p[59];
    load_params<float>(params, ld, i, p);
    project_one<float>(p, cam, out[i]);
  }
}

uint32_t float_bits(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }

// Composited sequence of one pixel in fp32: list positions (within the
// tile's range) of the Gaussians composited, in order, plus the clamp flags.
struct PixelTrace {
  std::vector<int32_t> pos;
  std::vector<uint8_t> clamped;
  float T_final;
  uint32_t last;
  uint32_t read;      // list entries read: up to and including the stopping one
  float rgb[3];
};

void trace_pixel(const std::vector<Proj<float>>& g, const int32_t* list, int64_t len,
                 int px, int py, PixelTrace& tr) {
  tr.pos.clear();
  tr.clamped.clear();
  float T = 1.0f, Cr = 0.0f, Cg = 0.0f, Cb = 0.0f;
  uint32_t last = 0;
  tr.read = uint32_t(len);
  const float pxc = float(px) + 0.5f, pyc = float(py) + 0.5f;
  for (int64_t j = 0; j < len; ++j) {
    const Proj<float>& q = g[list[j]];
    const Step32 s = composite_step(q.u, q.v, q.A, q.B, q.C, q.opacity, pxc, pyc, T);
    if (s.kind == 2) { tr.read = uint32_t(j + 1); break; }
    if (s.kind == 0) continue;
    const float wgt = s.alpha * T;
    Cr = std::fma(q.rgb[0], wgt, Cr);
    Cg = std::fma(q.rgb[1], wgt, Cg);
    Cb = std::fma(q.rgb[2], wgt, Cb);
    T = s.next_T;
    last = uint32_t(j + 1);
    tr.pos.push_back(int32_t(j));
    tr.clamped.push_back(s.clamped);
  }
  tr.T_final = T;
  tr.last = last;
  tr.rgb[0] = Cr; tr.rgb[1] = Cg; tr.rgb[2] = Cb;
}

// Per-tile sorted Gaussian lists straight from the definition: the visible
// Gaussians whose tile rectangle holds the tile, ordered by (depth bits,
// index).
void tile_lists(const std::vector<Proj<float>>& g, int TX, int TY,
                std::vector<std::vector<int32_t>>& lists) {
  const int64_t n = int64_t(g.size());
  lists.assign(size_t(TX) * TY, {});
  for (int64_t i = 0; i < n; ++i) {
    if (!g[i].visible) continue;
    for (int ty = g[i].rect[1]; ty < g[i].rect[3]; ++ty)
      for (int tx = g[i].rect[0]; tx < g[i].rect[2]; ++tx)
        lists[size_t(ty) * TX + tx].push_back(int32_t(i));
  }
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < int64_t(lists.size()); ++t) {
    std::sort(lists[t].begin(), lists[t].end(), [&](int32_t a, int32_t b) {
      const uint32_t da = float_bits(g[a].depth), db = float_bits(g[b].depth);
      return da != db ? da < db : a < b;
    });
  }
}

// ---------------------------------------------------------------------------
// SSIM window: 11 x 11, outer product of the normalised 1-D Gaussian with
// sigma 1.5 (the window named in the workload description); constants
// C1 = 0.01^2, C2 = 0.03^2 for a unit dynamic range (Wang et al. 2004).
// ---------------------------------------------------------------------------
void ssim_window(double w[11][11]) {
  double g[11], s = 0.0;
  for (int k = 0; k < 11; ++k) { g[k] = std::exp(-double((k - 5) * (k - 5)) / (2.0 * 1.5 * 1.5)); s += g[k]; }
  for (int k = 0; k < 11; ++k) g[k] /= s;
  for (int i = 0; i < 11; ++i)
    for (int j = 0; j < 11; ++j) w[i][j] = g[i] * g[j];
}

// zero-padded "same" 2-D correlation of one plane with the 11x11 window
void conv11(const double* in, int W, int H, const double w[11][11], double* out) {
#pragma omp parallel for schedule(static)
  for (int y = 0; y < H; ++y)
    for (int x = 0; x < W; ++x) {
      double acc = 0.0;
      for (int i = 0; i < 11; ++i) {
        const int yy = y + i - 5;
        if (yy < 0 || yy >= H) continue;
        for (int j = 0; j < 11; ++j) {
          const int xx = x + j - 5;
          if (xx < 0 || xx >= W) continue;
          acc += w[i][j] * in[size_t(yy) * W + xx];
        }
      }
      out[size_t(y) * W + x] = acc;
    }
}

// ---------------------------------------------------------------------------
// Magnitude type for error bounds of the backward pass: every + and - adds
// absolute values and every product multiplies them, so the result bounds
// the sum of |terms| a floating-point evaluation of the same expression
// accumulates rounding error against.
// ---------------------------------------------------------------------------
struct Mag {
  double v = 0.0;
  Mag() = default;
  explicit Mag(double x) : v(std::fabs(x)) {}
};
inline Mag operator+(Mag a, Mag b) { Mag r; r.v = a.v + b.v; return r; }
inline Mag operator-(Mag a, Mag b) { Mag r; r.v = a.v + b.v; return r; }
inline Mag operator-(Mag a) { return a; }
inline Mag operator*(Mag a, double d) { Mag r; r.v = a.v * std::fabs(d); return r; }
inline Mag operator*(double d, Mag a) { return a * d; }
inline Mag operator/(Mag a, double d) { Mag r; r.v = a.v / std::fabs(d); return r; }
inline Mag& operator+=(Mag& a, Mag b) { a.v += b.v; return a; }
inline double val(double x) { return x; }
inline double val(Mag m) { return m.v; }
template <class V> inline V mk(double x);
template <> inline double mk<double>(double x) { return x; }
template <> inline Mag mk<Mag>(double x) { return Mag(x); }

// ---------------------------------------------------------------------------
// Backward of the projection for one Gaussian: the exact chain rule of
// project_one, evaluated at the forward intermediates `f` (fp64 ones, or the
// fp32 forward's widened), with the colour clamp held at rgb_pos.
// g2d = dL/d(u, v, A, B, C, opacity, r, g, b); writes dL/dparam into g[59].
// ---------------------------------------------------------------------------
template <class V>
void project_backward_one(const Proj<double>& f, const double p[59], const or_camera& cam, const bool rgb_pos[3],
                          const V g2d[9], V g[59]) {
  const double R[9] = {cam.R[0], cam.R[1], cam.R[2], cam.R[3], cam.R[4], cam.R[5], cam.R[6], cam.R[7], cam.R[8]};
  const double* s = f.s;
  const double w = f.q[0], x = f.q[1], y = f.q[2], z = f.q[3];
  const double qn = std::sqrt(f.qn);
  double Rq[3][3], M[3][3], S[3][3], T[2][3];
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j) {
      Rq[i][j] = f.R[3 * i + j];
      M[i][j] = Rq[i][j] * s[j];
    }
  const int sidx[3][3] = {{0, 1, 2}, {1, 3, 4}, {2, 4, 5}};
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j) S[i][j] = f.S[sidx[i][j]];
  for (int i = 0; i < 2; ++i)
    for (int k = 0; k < 3; ++k) T[i][k] = f.T[3 * i + k];
  // For the error-bound instantiation (V = Mag) every product sum the
  // backward forms from forward values enters with its terms' magnitudes.
  constexpr bool kMag = std::is_same<V, Mag>::value;
  double TS[2][3];
  for (int i = 0; i < 2; ++i)
    for (int k = 0; k < 3; ++k)
      TS[i][k] = kMag ? std::fabs(T[i][0] * S[0][k]) + std::fabs(T[i][1] * S[1][k]) + std::fabs(T[i][2] * S[2][k])
                      : T[i][0] * S[0][k] + T[i][1] * S[1][k] + T[i][2] * S[2][k];
  const double a = f.a, b = f.b, c = f.c;
  const double det2 = f.det * f.det;
  const double o = f.opacity;
  const double iz = f.iz, ux = f.ux, uy = f.uy;
  const double jx = double(cam.fx) * iz, jy = double(cam.fy) * iz;

  const V gu = g2d[0], gv = g2d[1], gA = g2d[2], gB = g2d[3], gC = g2d[4], go = g2d[5];
  for (int k = 0; k < 59; ++k) g[k] = mk<V>(0.0);
  // opacity logit
  g[10] = go * (o * (1.0 - o));
  // colour -> SH coefficients and view direction
  const double* d = f.dir;
  double Yb[16], dY[16][3];
  if (kMag) {
    sh_basis_mag(d[0], d[1], d[2], Yb, dY);
  } else {
    sh_basis<double>(d[0], d[1], d[2], Yb);
    sh_basis_grad(d[0], d[1], d[2], dY);
  }
  V graw[3];
  for (int ch = 0; ch < 3; ++ch) graw[ch] = rgb_pos[ch] ? g2d[6 + ch] : mk<V>(0.0);
  V gd[3] = {mk<V>(0.0), mk<V>(0.0), mk<V>(0.0)};
  for (int k = 0; k < 16; ++k) {
    V gY = mk<V>(0.0);
    for (int ch = 0; ch < 3; ++ch) {
      g[11 + 3 * k + ch] = graw[ch] * Yb[k];
      gY += graw[ch] * p[11 + 3 * k + ch];
    }
    for (int e = 0; e < 3; ++e) gd[e] += gY * dY[k][e];
  }
  // through d = (x - campos) / |x - campos|
  V gdd = gd[0] * d[0] + gd[1] * d[1] + gd[2] * d[2];
  V gpos[3];
  for (int e = 0; e < 3; ++e) gpos[e] = (gd[e] - gdd * d[e]) / f.dn;
  // conic (A, B, C) = (c, -b, a) / det
  const V ga = gA * (-c * c / det2) + gB * (b * c / det2) + gC * (-b * b / det2);
  const V gb = gA * (2.0 * b * c / det2) + gB * (-(a * c + b * b) / det2) + gC * (2.0 * a * b / det2);
  const V gc = gA * (-b * b / det2) + gB * (a * b / det2) + gC * (-a * a / det2);
  // full-matrix gradient of the 2x2 screen covariance
  const V G2[2][2] = {{ga, gb * 0.5}, {gb * 0.5, gc}};
  // Sigma: G_Sigma = T^T G2 T
  V GS[3][3];
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j) {
      V acc = mk<V>(0.0);
      for (int r = 0; r < 2; ++r)
        for (int q = 0; q < 2; ++q) acc += G2[r][q] * (T[r][i] * T[q][j]);
      GS[i][j] = acc;
    }
  // T: G_T = 2 G2 T Sigma
  V GT[2][3];
  for (int r = 0; r < 2; ++r)
    for (int k = 0; k < 3; ++k) {
      V acc = mk<V>(0.0);
      for (int q = 0; q < 2; ++q) acc += G2[r][q] * (2.0 * TS[q][k]);
      GT[r][k] = acc;
    }
  // J = T R^T gradient: G_J = G_T R^T
  V GJ[2][3];
  for (int r = 0; r < 2; ++r)
    for (int m = 0; m < 3; ++m) {
      V acc = mk<V>(0.0);
      for (int k = 0; k < 3; ++k) acc += GT[r][k] * R[3 * m + k];
      GJ[r][m] = acc;
    }
  // J = [[fx/tz, 0, -fx tx/tz^2], [0, fy/tz, -fy ty/tz^2]]; u = fx tx/tz + cx
  V gtx = GJ[0][2] * (-jx * iz) + gu * jx;
  V gty = GJ[1][2] * (-jy * iz) + gv * jy;
  V gtz = GJ[0][0] * (-jx * iz) + GJ[0][2] * (2.0 * jx * ux * iz) + GJ[1][1] * (-jy * iz) +
          GJ[1][2] * (2.0 * jy * uy * iz) + gu * (-jx * ux) + gv * (-jy * uy);
  // t = R x + t_c
  for (int e = 0; e < 3; ++e) g[e] = gpos[e] + gtx * R[e] + gty * R[3 + e] + gtz * R[6 + e];
  // Sigma = M M^T : G_M = 2 G_Sigma M
  V GM[3][3];
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j) {
      V acc = mk<V>(0.0);
      for (int k = 0; k < 3; ++k) acc += GS[i][k] * (2.0 * M[k][j]);
      GM[i][j] = acc;
    }
  // M = Rq diag(s)
  V GR[3][3];
  for (int j = 0; j < 3; ++j) {
    V gs = mk<V>(0.0);
    for (int i = 0; i < 3; ++i) {
      gs += GM[i][j] * Rq[i][j];
      GR[i][j] = GM[i][j] * s[j];
    }
    g[3 + j] = gs * s[j];  // s = exp(log s)
  }
  // rotation matrix of the unit quaternion
  const V gw = (GR[0][1] * (-z) + GR[0][2] * y + GR[1][0] * z + GR[1][2] * (-x) + GR[2][0] * (-y) + GR[2][1] * x) * 2.0;
  const V gx = (GR[0][1] * y + GR[0][2] * z + GR[1][0] * y + GR[1][1] * (-2.0 * x) + GR[1][2] * (-w) +
                GR[2][0] * z + GR[2][1] * w + GR[2][2] * (-2.0 * x)) * 2.0;
  const V gy = (GR[0][0] * (-2.0 * y) + GR[0][1] * x + GR[0][2] * w + GR[1][0] * x + GR[1][2] * z +
                GR[2][0] * (-w) + GR[2][1] * z + GR[2][2] * (-2.0 * y)) * 2.0;
  const V gz = (GR[0][0] * (-2.0 * z) + GR[0][1] * (-w) + GR[0][2] * x + GR[1][0] * w + GR[1][1] * (-2.0 * z) +
                GR[1][2] * y + GR[2][0] * x + GR[2][1] * y) * 2.0;
  // q_hat = q / |q|
  const V gdot = gw * w + gx * x + gy * y + gz * z;
  g[6] = (gw - gdot * w) / qn;
  g[7] = (gx - gdot * x) / qn;
  g[8] = (gy - gdot * y) / qn;
  g[9] = (gz - gdot * z) / qn;
}

}  // namespace

// ===========================================================================
// C API (numpy via ctypes).  All arrays are caller-owned, C-contiguous.
// ===========================================================================
extern "C" {

int or_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void or_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

float or_pexp(float x) { return pexp(x); }
float or_aexp(float x) { return aexp(x); }

void or_sh_basis_f64(const double* dirs, int64_t n, double* Y) {
  for (int64_t i = 0; i < n; ++i) sh_basis<double>(dirs[3 * i], dirs[3 * i + 1], dirs[3 * i + 2], Y + 16 * i);
}
void or_sh_basis_f32(const float* dirs, int64_t n, float* Y) {
  for (int64_t i = 0; i < n; ++i) sh_basis<float>(dirs[3 * i], dirs[3 * i + 1], dirs[3 * i + 2], Y + 16 * i);
}

// fp32 canonical projection.  Outputs per Gaussian: mean2d [n][2],
// depth [n], cov2d [n][3] (a, b, c incl. dilation), conic [n][3],
// opacity [n], rgb [n][3], rgb_pos [n][3], radius [n], rect [n][4],
// tiles [n], visible [n].
void or_preprocess(const float* params, int64_t n, int64_t ld, const or_camera* cam,
                   float* mean2d, float* depth, float* cov2d, float* conic, float* opacity,
                   float* rgb, uint8_t* rgb_pos, int32_t* radius, int32_t* rect,
                   uint32_t* tiles, uint8_t* visible) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    float p[59];
    load_params<float>(params, ld, i, p);
    Proj<float> o;
    project_one<float>(p, *cam, o);
    mean2d[2 * i] = o.u; mean2d[2 * i + 1] = o.v;
    depth[i] = o.depth;
    cov2d[3 * i] = o.a; cov2d[3 * i + 1] = o.b; cov2d[3 * i + 2] = o.c;
    conic[3 * i] = o.A; conic[3 * i + 1] = o.B; conic[3 * i + 2] = o.C;
    opacity[i] = o.opacity;
    for (int c = 0; c < 3; ++c) { rgb[3 * i + c] = o.rgb[c]; rgb_pos[3 * i + c] = o.rgb_pos[c]; }
    radius[i] = o.radius;
    for (int c = 0; c < 4; ++c) rect[4 * i + c] = o.rect[c];
    tiles[i] = o.tiles;
    visible[i] = o.visible;
  }
}

// Same projection in fp64 (no decision freezing; the pins on closed forms
// use it).
void or_preprocess_f64(const double* params, int64_t n, int64_t ld, const or_camera* cam,
                       double* mean2d, double* depth, double* cov2d, double* conic,
                       double* opacity, double* rgb) {
  for (int64_t i = 0; i < n; ++i) {
    double p[59];
    for (int k = 0; k < 59; ++k) p[k] = params[k * ld + i];
    Proj<double> o;
    project_one<double>(p, *cam, o);
    mean2d[2 * i] = o.u; mean2d[2 * i + 1] = o.v;
    depth[i] = o.depth;
    cov2d[3 * i] = o.a; cov2d[3 * i + 1] = o.b; cov2d[3 * i + 2] = o.c;
    conic[3 * i] = o.A; conic[3 * i + 1] = o.B; conic[3 * i + 2] = o.C;
    opacity[i] = o.opacity;
    for (int c = 0; c < 3; ++c) rgb[3 * i + c] = o.rgb[c];
  }
}

// The projection's intermediates in fp64 for the covariance pins: the
// rotation of the normalised quaternion R_q [n][9] (row-major), the world
// covariance Sigma = R_q S^2 R_q^T [n][9] (full, row-major) and the screen
// covariance before the 0.3 dilation [n][3] (a, b, c).
void or_projection_internals_f64(const double* params, int64_t n, int64_t ld, const or_camera* cam, double* Rq,
                                 double* Sigma, double* cov2d_raw) {
  for (int64_t i = 0; i < n; ++i) {
    double p[59];
    for (int k = 0; k < 59; ++k) p[k] = params[k * ld + i];
    Proj<double> o;
    project_one<double>(p, *cam, o);
    for (int k = 0; k < 9; ++k) Rq[9 * i + k] = o.R[k];
    const double* S = o.S;   // 00 01 02 11 12 22
    const double full[9] = {S[0], S[1], S[2], S[1], S[3], S[4], S[2], S[4], S[5]};
    for (int k = 0; k < 9; ++k) Sigma[9 * i + k] = full[k];
    cov2d_raw[3 * i] = o.a - 0.3;
    cov2d_raw[3 * i + 1] = o.b;
    cov2d_raw[3 * i + 2] = o.c - 0.3;
  }
}

// Gaussian-tile pairs sorted by (tile, depth bits, index): keys
// (tile << 32 | depth bits), values = Gaussian index, ranges [T][2].
// Returns M; writes at most `cap` pairs (pass cap = 0 to count only).
int64_t or_bin(const float* params, int64_t n, int64_t ld, const or_camera* cam,
               uint64_t* keys, int32_t* vals, int64_t cap, uint32_t* ranges) {
  std::vector<Proj<float>> g;
  project_all(params, n, ld, *cam, g);
  const int TX = (cam->width + kTile - 1) / kTile, TY = (cam->height + kTile - 1) / kTile;
  std::vector<std::pair<uint64_t, int32_t>> pairs;
  for (int64_t i = 0; i < n; ++i) {
    if (!g[i].visible) continue;
    for (int ty = g[i].rect[1]; ty < g[i].rect[3]; ++ty)
      for (int tx = g[i].rect[0]; tx < g[i].rect[2]; ++tx)
        pairs.emplace_back((uint64_t(uint32_t(ty * TX + tx)) << 32) | float_bits(g[i].depth), int32_t(i));
  }
  const int64_t M = int64_t(pairs.size());
  if (cap == 0) return M;
  std::sort(pairs.begin(), pairs.end());
  const int64_t m = std::min(M, cap);
  for (int64_t k = 0; k < m; ++k) { keys[k] = pairs[k].first; vals[k] = pairs[k].second; }
  if (ranges) {
    std::memset(ranges, 0, sizeof(uint32_t) * 2 * size_t(TX) * TY);
    for (int64_t k = 0; k < M; ++k) {
      const uint32_t t = uint32_t(pairs[k].first >> 32);
      if (k == 0 || uint32_t(pairs[k - 1].first >> 32) != t) ranges[2 * t] = uint32_t(k);
      if (k == M - 1 || uint32_t(pairs[k + 1].first >> 32) != t) ranges[2 * t + 1] = uint32_t(k + 1);
    }
  }
  return M;
}

// fp32 render.  image [3][H][W], T_final [H][W], last [H][W] (list
// position + 1 of the last composited Gaussian, 0 if none),
// tile_processed [T] = max over the tile's pixels of the entries read
// (last, or the stop position + 1).
void or_render(const float* params, int64_t n, int64_t ld, const or_camera* cam,
               float* image, float* T_final, uint32_t* last, uint32_t* tile_processed) {
  std::vector<Proj<float>> g;
  project_all(params, n, ld, *cam, g);
  const int W = cam->width, H = cam->height;
  const int TX = (W + kTile - 1) / kTile, TY = (H + kTile - 1) / kTile;
  std::vector<std::vector<int32_t>> lists;
  tile_lists(g, TX, TY, lists);
  const size_t P = size_t(W) * H;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t t = 0; t < int64_t(TX) * TY; ++t) {
    const int tx = int(t % TX), ty = int(t / TX);
    const std::vector<int32_t>& L = lists[t];
    uint32_t tile_max = 0;
    PixelTrace tr;
    for (int py = ty * kTile; py < std::min(H, (ty + 1) * kTile); ++py)
      for (int px = tx * kTile; px < std::min(W, (tx + 1) * kTile); ++px) {
        trace_pixel(g, L.data(), int64_t(L.size()), px, py, tr);
        const size_t pix = size_t(py) * W + px;
        for (int c = 0; c < 3; ++c) image[c * P + pix] = tr.rgb[c];
        T_final[pix] = tr.T_final;
        last[pix] = tr.last;
        tile_max = std::max(tile_max, tr.read);
      }
    if (tile_processed) tile_processed[t] = tile_max;
  }
}

// Per pixel, the number of Gaussians it composited (fp32 rule of or_render):
// counts [H][W].  Their sum is the number of (pixel, list entry) steps a
// backward pass back-propagates.
void or_composited_counts(const float* params, int64_t n, int64_t ld, const or_camera* cam, uint32_t* counts) {
  std::vector<Proj<float>> g;
  project_all(params, n, ld, *cam, g);
  const int W = cam->width, H = cam->height;
  const int TX = (W + kTile - 1) / kTile, TY = (H + kTile - 1) / kTile;
  std::vector<std::vector<int32_t>> lists;
  tile_lists(g, TX, TY, lists);
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t t = 0; t < int64_t(TX) * TY; ++t) {
    const int tx = int(t % TX), ty = int(t / TX);
    const std::vector<int32_t>& L = lists[t];
    PixelTrace tr;
    for (int py = ty * kTile; py < std::min(H, (ty + 1) * kTile); ++py)
      for (int px = tx * kTile; px < std::min(W, (tx + 1) * kTile); ++px) {
        trace_pixel(g, L.data(), int64_t(L.size()), px, py, tr);
        counts[size_t(py) * W + px] = uint32_t(tr.pos.size());
      }
  }
}

// Brute-force render: every pixel scans ALL n Gaussians, keeps the visible
// ones whose tile rectangle holds the pixel's tile, sorts them by (depth
// bits, index) and composites.  Must equal or_render bit for bit.
void or_render_brute(const float* params, int64_t n, int64_t ld, const or_camera* cam,
                     float* image, float* T_final, uint32_t* last) {
  std::vector<Proj<float>> g;
  project_all(params, n, ld, *cam, g);
  const int W = cam->width, H = cam->height;
  const size_t P = size_t(W) * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (int py = 0; py < H; ++py) {
    std::vector<int32_t> cand;
    PixelTrace tr;
    for (int px = 0; px < W; ++px) {
      const int tx = px / kTile, ty = py / kTile;
      cand.clear();
      for (int64_t i = 0; i < n; ++i)
        if (g[i].visible && tx >= g[i].rect[0] && tx < g[i].rect[2] && ty >= g[i].rect[1] && ty < g[i].rect[3])
          cand.push_back(int32_t(i));
      std::sort(cand.begin(), cand.end(), [&](int32_t a, int32_t b) {
        const uint32_t da = float_bits(g[a].depth), db = float_bits(g[b].depth);
        return da != db ? da < db : a < b;
      });
      trace_pixel(g, cand.data(), int64_t(cand.size()), px, py, tr);
      const size_t pix = size_t(py) * W + px;
      for (int c = 0; c < 3; ++c) image[c * P + pix] = tr.rgb[c];
      T_final[pix] = tr.T_final;
      last[pix] = tr.last;
    }
  }
}

// Sampled pixels composited against given per-tile lists (values and
// [start, end) ranges of a sorted pair array, e.g. one produced elsewhere
// and checked against the definition separately): for pixel k at (px[k],
// py[k]) its tile's list is composited with the same per-pixel rule as
// or_render.  rgb [k][3], T_final [k], last [k].
void or_composite_pixels(const float* params, int64_t n, int64_t ld, const or_camera* cam, const int32_t* vals,
                         const uint32_t* ranges, const int32_t* px, const int32_t* py, int64_t count, float* rgb,
                         float* T_final, uint32_t* last) {
  std::vector<Proj<float>> g;
  project_all(params, n, ld, *cam, g);
  const int TX = (cam->width + kTile - 1) / kTile;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t k = 0; k < count; ++k) {
    const int64_t t = int64_t(py[k] / kTile) * TX + px[k] / kTile;
    const uint32_t a = ranges[2 * t], b = ranges[2 * t + 1];
    PixelTrace tr;
    trace_pixel(g, vals + a, int64_t(b) - int64_t(a), px[k], py[k], tr);
    for (int c = 0; c < 3; ++c) rgb[3 * k + c] = tr.rgb[c];
    T_final[k] = tr.T_final;
    last[k] = tr.last;
  }
}

// Loss (fp64) of a rendered image against a target, both [3][H][W] fp32:
// L = w_l1 * mean|I - I_t| + w_ssim * (1 - mean SSIM), means over 3 H W.
// dL/dI [3][H][W].  The L1 subgradient at 0 is 0.  Returns L; also writes
// the mean L1 and mean SSIM.
double or_loss(const float* image, const float* target, int W, int H, double w_l1, double w_ssim,
               double* dL, double* l1_out, double* ssim_out) {
  const size_t P = size_t(W) * H;
  const double inv = 1.0 / (3.0 * double(P));
  std::vector<double> rowsum(size_t(3) * H, 0.0);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < int64_t(3) * H; ++r) {
    double acc = 0.0;
    for (int x = 0; x < W; ++x) {
      const size_t k = size_t(r) * W + x;
      const double d = double(image[k]) - double(target[k]);
      acc += std::fabs(d);
      dL[k] = w_l1 * inv * (d > 0 ? 1.0 : (d < 0 ? -1.0 : 0.0));
    }
    rowsum[r] = acc;
  }
  double l1 = 0.0;
  for (double v : rowsum) l1 += v;
  l1 *= inv;
  double ssim_mean = 1.0;
  if (w_ssim != 0.0) {
    double w[11][11];
    ssim_window(w);
    const double C1 = 0.01 * 0.01, C2 = 0.03 * 0.03;
    std::vector<double> x(P), y(P), xx(P), yy(P), xy(P), mx(P), my(P), sxx(P), syy(P), sxy(P);
    std::vector<double> dmx(P), dxx(P), dxy(P), bmx(P), bxx(P), bxy(P);
    double total = 0.0;
    for (int c = 0; c < 3; ++c) {
      for (size_t k = 0; k < P; ++k) {
        x[k] = image[c * P + k];
        y[k] = target[c * P + k];
        xx[k] = x[k] * x[k]; yy[k] = y[k] * y[k]; xy[k] = x[k] * y[k];
      }
      conv11(x.data(), W, H, w, mx.data());
      conv11(y.data(), W, H, w, my.data());
      conv11(xx.data(), W, H, w, sxx.data());
      conv11(yy.data(), W, H, w, syy.data());
      conv11(xy.data(), W, H, w, sxy.data());
      std::vector<double> rs(H, 0.0);
#pragma omp parallel for schedule(static)
      for (int r = 0; r < H; ++r) {
        double acc = 0.0;
        for (int q = 0; q < W; ++q) {
          const size_t k = size_t(r) * W + q;
          const double mux = mx[k], muy = my[k];
          const double vx = sxx[k] - mux * mux, vy = syy[k] - muy * muy, cxy = sxy[k] - mux * muy;
          const double A1 = 2.0 * mux * muy + C1, A2 = 2.0 * cxy + C2;
          const double B1 = mux * mux + muy * muy + C1, B2 = vx + vy + C2;
          const double D = B1 * B2;
          const double S = A1 * A2 / D;
          acc += S;
          // partials of S wrt mu_x, E[x^2], E[xy]
          dmx[k] = (2.0 * muy * A2 - 2.0 * muy * A1) / D - S * (2.0 * mux * B2 - 2.0 * mux * B1) / D;
          dxx[k] = -S * B1 / D;
          dxy[k] = 2.0 * A1 / D;
        }
        rs[r] = acc;
      }
      for (double v : rs) total += v;
      // transposed window (the window is symmetric, zero padding)
      conv11(dmx.data(), W, H, w, bmx.data());
      conv11(dxx.data(), W, H, w, bxx.data());
      conv11(dxy.data(), W, H, w, bxy.data());
      const double sc = -w_ssim * inv;
      for (size_t k = 0; k < P; ++k) dL[c * P + k] += sc * (bmx[k] + 2.0 * x[k] * bxx[k] + y[k] * bxy[k]);
    }
    ssim_mean = total * inv;
  }
  if (l1_out) *l1_out = l1;
  if (ssim_out) *ssim_out = ssim_mean;
  return w_l1 * l1 + w_ssim * (1.0 - ssim_mean);
}

// ---------------------------------------------------------------------------
// fp64 forward with frozen decisions (for central differences).
// Decisions (visibility, tile lists, composited set per pixel, alpha clamp,
// colour clamp) come from the fp32 canonical run at `base`; quantities are
// evaluated in fp64 at `params64`.  Writes the fp64 image [3][H][W].
// ---------------------------------------------------------------------------
void or_render_frozen_f64(const float* base, const double* params64, int64_t n, int64_t ld,
                          const or_camera* cam, double* image) {
  std::vector<Proj<float>> g;
  project_all(base, n, ld, *cam, g);
  std::vector<Proj<double>> h(n);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double p[59];
    for (int k = 0; k < 59; ++k) p[k] = params64[k * ld + i];
    project_one<double>(p, *cam, h[i]);
    // frozen colour clamp: the raw value passes where the fp32 run said > 0
    for (int c = 0; c < 3; ++c) h[i].rgb[c] = g[i].rgb_pos[c] ? h[i].rgb_raw[c] : 0.0;
  }
  const int W = cam->width, H = cam->height;
  const int TX = (W + kTile - 1) / kTile, TY = (H + kTile - 1) / kTile;
  std::vector<std::vector<int32_t>> lists;
  tile_lists(g, TX, TY, lists);
  const size_t P = size_t(W) * H;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t t = 0; t < int64_t(TX) * TY; ++t) {
    const int tx = int(t % TX), ty = int(t / TX);
    const std::vector<int32_t>& L = lists[t];
    PixelTrace tr;
    for (int py = ty * kTile; py < std::min(H, (ty + 1) * kTile); ++py)
      for (int px = tx * kTile; px < std::min(W, (tx + 1) * kTile); ++px) {
        trace_pixel(g, L.data(), int64_t(L.size()), px, py, tr);
        double T = 1.0, C[3] = {0, 0, 0};
        const double pxc = px + 0.5, pyc = py + 0.5;
        for (size_t k = 0; k < tr.pos.size(); ++k) {
          const Proj<double>& q = h[L[tr.pos[k]]];
          const double dx = pxc - q.u, dy = pyc - q.v;
          const double power = -0.5 * (q.A * dx * dx + q.C * dy * dy) - q.B * dx * dy;
          const double alpha = tr.clamped[k] ? 0.99 : q.opacity * std::exp(power);
          for (int c = 0; c < 3; ++c) C[c] += q.rgb[c] * alpha * T;
          T *= (1.0 - alpha);
        }
        const size_t pix = size_t(py) * W + px;
        for (int c = 0; c < 3; ++c) image[c * P + pix] = C[c];
      }
  }
}

// fp64 loss of an fp64 image with the L1 sign frozen at the fp32 image's
// (same formula as or_loss otherwise).  For central differences.
double or_loss_frozen_f64(const double* image, const float* image32, const float* target, int W, int H,
                          double w_l1, double w_ssim) {
  const size_t P = size_t(W) * H;
  const double inv = 1.0 / (3.0 * double(P));
  double l1 = 0.0;
  for (size_t k = 0; k < 3 * P; ++k) {
    const double d32 = double(image32[k]) - double(target[k]);
    const double d = image[k] - double(target[k]);
    l1 += d32 > 0 ? d : (d32 < 0 ? -d : 0.0);
  }
  l1 *= inv;
  double ssim_mean = 1.0;
  if (w_ssim != 0.0) {
    double w[11][11];
    ssim_window(w);
    const double C1 = 0.01 * 0.01, C2 = 0.03 * 0.03;
    std::vector<double> x(P), y(P), xx(P), yy(P), xy(P), mx(P), my(P), sxx(P), syy(P), sxy(P);
    double total = 0.0;
    for (int c = 0; c < 3; ++c) {
      for (size_t k = 0; k < P; ++k) {
        x[k] = image[c * P + k];
        y[k] = target[c * P + k];
        xx[k] = x[k] * x[k]; yy[k] = y[k] * y[k]; xy[k] = x[k] * y[k];
      }
      conv11(x.data(), W, H, w, mx.data());
      conv11(y.data(), W, H, w, my.data());
      conv11(xx.data(), W, H, w, sxx.data());
      conv11(yy.data(), W, H, w, syy.data());
      conv11(xy.data(), W, H, w, sxy.data());
      for (size_t k = 0; k < P; ++k) {
        const double mux = mx[k], muy = my[k];
        const double vx = sxx[k] - mux * mux, vy = syy[k] - muy * muy, cxy = sxy[k] - mux * muy;
        total += (2.0 * mux * muy + C1) * (2.0 * cxy + C2) / ((mux * mux + muy * muy + C1) * (vx + vy + C2));
      }
    }
    ssim_mean = total * inv;
  }
  return w_l1 * l1 + w_ssim * (1.0 - ssim_mean);
}

// ---------------------------------------------------------------------------
// Backward of one view (fp64), "back-propagation" of the Grendel-GS
// training pipeline.  Decisions from the fp32 run, values in fp64; with
// `at_fp32` the chain rule is evaluated at the fp32 forward's values (the
// screen-space values the image was rendered from, and the projection's
// intermediates), i.e. the gradient of the rendered image; without it at
// the fp64 recomputation of the forward.
// Per pixel, reverse over its composited Gaussians with
//   dL/dc_i = alpha_i T_i G,  dL/dalpha_i = T_i (c_i - S_i) . G,
//   S_{i-1} = alpha_i c_i + (1 - alpha_i) S_i,  S_K = 0 (black background),
// then alpha = o e^power (unless clamped), power of (u, v, A, B, C).
// Outputs (all fp64):
//   g2d  [n][9]  dL/d(u, v, A, B, C, opacity, r, g, b)
//   m2d  [n][9]  sum over pixels of |partial| (magnitudes); with `gmag`
//                given, |G| is replaced by gmag in them, so passing a bound
//                on an error of G gives the bound on its effect
//   grads[59][ld] += dL/dparam  (ld = n here: dense planes)
//   mags [59][ld] += magnitudes propagated through the projection
// Per-tile partial sums are merged in tile order, so the result does not
// depend on the thread count.
// ---------------------------------------------------------------------------
// The backward given the fp32 projections `g` and the per-tile lists; with
// want_mags false the magnitudes (m2d, mags) are neither formed nor written.
static void backward_impl(const float* params, int64_t n, int64_t ld, const or_camera* cam,
                          const std::vector<Proj<float>>& g, const std::vector<std::vector<int32_t>>& lists,
                          const double* dL_dimage, const double* gmag, double* g2d, double* m2d, double* grads,
                          double* mags, int at_fp32, bool want_mags) {
  std::vector<Proj<double>> h(n);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    if (at_fp32) {
      // evaluate the raster backward at the fp32 forward's screen-space
      // values (what the rendered image was computed from)
      h[i] = widen(g[i]);
      continue;
    }
    double p[59];
    load_params<double>(params, ld, i, p);
    project_one<double>(p, *cam, h[i]);
    // frozen colour clamp: the raw value passes where the fp32 run said > 0
    for (int c = 0; c < 3; ++c) h[i].rgb[c] = g[i].rgb_pos[c] ? h[i].rgb_raw[c] : 0.0;
  }
  const int W = cam->width, H = cam->height;
  const int TX = (W + kTile - 1) / kTile, TY = (H + kTile - 1) / kTile;
  const size_t P = size_t(W) * H;
  const int64_t T = int64_t(TX) * TY;
  // per tile: partial sums per list position (value 9 + magnitude 9),
  // formed for a band of tile rows at a time (in parallel over its tiles)
  // and merged into the per-Gaussian sums in ascending tile order, so the
  // result is that of one pass over all tiles in tile order, for any band
  // height and thread count, with the partials of one band held at a time
  std::memset(g2d, 0, sizeof(double) * 9 * size_t(n));
  if (want_mags) std::memset(m2d, 0, sizeof(double) * 9 * size_t(n));
  const int band = std::max(1, (1024 + TX - 1) / TX);
  std::vector<std::vector<double>> part(size_t(band) * TX);
  for (int ty0 = 0; ty0 < TY; ty0 += band) {
    const int64_t t_lo = int64_t(ty0) * TX, t_hi = std::min<int64_t>(T, int64_t(ty0 + band) * TX);
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t t = t_lo; t < t_hi; ++t) {
      const int tx = int(t % TX), ty = int(t / TX);
      const std::vector<int32_t>& L = lists[t];
      std::vector<double>& acc = part[t - t_lo];
      acc.assign(L.size() * 18, 0.0);
      PixelTrace tr;
      std::vector<double> al, Ti;
      for (int py = ty * kTile; py < std::min(H, (ty + 1) * kTile); ++py)
        for (int px = tx * kTile; px < std::min(W, (tx + 1) * kTile); ++px) {
          trace_pixel(g, L.data(), int64_t(L.size()), px, py, tr);
          const size_t pix = size_t(py) * W + px;
          const double G[3] = {dL_dimage[pix], dL_dimage[P + pix], dL_dimage[2 * P + pix]};
          // magnitude of the image gradient used by the bound: |G|, or the
          // caller's map (e.g. a tolerance on G, to propagate it)
          const double Gm[3] = {gmag ? gmag[pix] : std::fabs(G[0]), gmag ? gmag[P + pix] : std::fabs(G[1]),
                                gmag ? gmag[2 * P + pix] : std::fabs(G[2])};
          const double pxc = px + 0.5, pyc = py + 0.5;
          const size_t K = tr.pos.size();
          al.assign(K, 0.0);
          Ti.assign(K, 0.0);
          double Tc = 1.0;
          for (size_t k = 0; k < K; ++k) {
            const Proj<double>& q = h[L[tr.pos[k]]];
            const double dx = pxc - q.u, dy = pyc - q.v;
            const double power = -0.5 * (q.A * dx * dx + q.C * dy * dy) - q.B * dx * dy;
            al[k] = tr.clamped[k] ? 0.99 : q.opacity * std::exp(power);
            Ti[k] = Tc;
            Tc *= (1.0 - al[k]);
          }
          double S[3] = {0, 0, 0};
          for (size_t kk = K; kk-- > 0;) {
            const int32_t pos = tr.pos[kk];
            const Proj<double>& q = h[L[pos]];
            const double a = al[kk], Tk = Ti[kk];
            double* o = &acc[size_t(pos) * 18];
            double dalpha = 0.0, malpha = 0.0;
            for (int c = 0; c < 3; ++c) {
              o[6 + c] += a * Tk * G[c];
              dalpha += Tk * (q.rgb[c] - S[c]) * G[c];
              if (want_mags) {
                o[9 + 6 + c] += a * Tk * Gm[c];
                malpha += Tk * (std::fabs(q.rgb[c]) + std::fabs(S[c])) * Gm[c];
              }
            }
            for (int c = 0; c < 3; ++c) S[c] = a * q.rgb[c] + (1.0 - a) * S[c];
            if (tr.clamped[kk]) continue;
            const double dx = pxc - q.u, dy = pyc - q.v;
            const double e = a / q.opacity;  // exp(power)
            const double dpow = dalpha * a, mpow = malpha * a;
            o[5] += dalpha * e;
            o[2] += dpow * (-0.5 * dx * dx);
            o[3] += dpow * (-dx * dy);
            o[4] += dpow * (-0.5 * dy * dy);
            o[0] += dpow * (q.A * dx + q.B * dy);
            o[1] += dpow * (q.B * dx + q.C * dy);
            if (want_mags) {
              o[9 + 5] += malpha * e;
              o[9 + 2] += mpow * (0.5 * dx * dx);
              o[9 + 3] += mpow * std::fabs(dx * dy);
              o[9 + 4] += mpow * (0.5 * dy * dy);
              o[9 + 0] += mpow * (std::fabs(q.A * dx) + std::fabs(q.B * dy));
              o[9 + 1] += mpow * (std::fabs(q.B * dx) + std::fabs(q.C * dy));
            }
          }
        }
    }
    for (int64_t t = t_lo; t < t_hi; ++t) {
      const std::vector<int32_t>& L = lists[t];
      for (size_t j = 0; j < L.size(); ++j) {
        const double* o = &part[t - t_lo][j * 18];
        for (int c = 0; c < 9; ++c) g2d[size_t(L[j]) * 9 + c] += o[c];
        if (want_mags)
          for (int c = 0; c < 9; ++c) m2d[size_t(L[j]) * 9 + c] += o[9 + c];
      }
      std::vector<double>().swap(part[t - t_lo]);
    }
  }
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    if (!g[i].visible) continue;
    double p[59];
    load_params<double>(params, ld, i, p);
    double gp[59];
    const Proj<double> f = at_fp32 ? widen(g[i]) : h[i];
    project_backward_one<double>(f, p, *cam, g[i].rgb_pos, &g2d[size_t(i) * 9], gp);
    for (int k = 0; k < 59; ++k) grads[k * ld + i] += gp[k];
    if (!want_mags) continue;
    Mag mp[59], m9[9];
    for (int c = 0; c < 9; ++c) m9[c].v = m2d[size_t(i) * 9 + c];
    project_backward_one<Mag>(f, p, *cam, g[i].rgb_pos, m9, mp);
    for (int k = 0; k < 59; ++k) mags[k * ld + i] += mp[k].v;
  }
}

void or_backward(const float* params, int64_t n, int64_t ld, const or_camera* cam,
                 const double* dL_dimage, const double* gmag, double* g2d, double* m2d, double* grads,
                 double* mags, int at_fp32) {
  std::vector<Proj<float>> g;
  project_all(params, n, ld, *cam, g);
  std::vector<std::vector<int32_t>> lists;
  tile_lists(g, (cam->width + kTile - 1) / kTile, (cam->height + kTile - 1) / kTile, lists);
  backward_impl(params, n, ld, cam, g, lists, dL_dimage, gmag, g2d, m2d, grads, mags, at_fp32, true);
}

// One view of the training step, stage by stage, projecting once: fp32
// projection, per-tile lists in (depth bits, index) order, the render of
// every pixel, the fp64 loss and its image gradient, and the backward at
// the fp32 forward's values (as or_backward with at_fp32), its gradients
// ADDED into grads [59][ld]; no magnitudes.  Writes image [3][H][W] and
// returns the loss.  (The plain step the CPU baseline times.)
double or_train_view(const float* params, int64_t n, int64_t ld, const or_camera* cam, const float* target,
                     double w_l1, double w_ssim, float* image, double* grads) {
  std::vector<Proj<float>> g;
  project_all(params, n, ld, *cam, g);
  const int W = cam->width, H = cam->height;
  const int TX = (W + kTile - 1) / kTile, TY = (H + kTile - 1) / kTile;
  std::vector<std::vector<int32_t>> lists;
  tile_lists(g, TX, TY, lists);
  const size_t P = size_t(W) * H;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t t = 0; t < int64_t(TX) * TY; ++t) {
    const int tx = int(t % TX), ty = int(t / TX);
    const std::vector<int32_t>& L = lists[t];
    PixelTrace tr;
    for (int py = ty * kTile; py < std::min(H, (ty + 1) * kTile); ++py)
      for (int px = tx * kTile; px < std::min(W, (tx + 1) * kTile); ++px) {
        trace_pixel(g, L.data(), int64_t(L.size()), px, py, tr);
        for (int c = 0; c < 3; ++c) image[c * P + size_t(py) * W + px] = tr.rgb[c];
      }
  }
  std::vector<double> dL(3 * P), g2d(9 * size_t(n));
  const double L = or_loss(image, target, W, H, w_l1, w_ssim, dL.data(), nullptr, nullptr);
  backward_impl(params, n, ld, cam, g, lists, dL.data(), nullptr, g2d.data(), nullptr, grads, nullptr, 1, false);
  return L;
}

// Projection backward alone (fp64): g2d [n][9] given, adds into grads
// [59][ld].  Visible Gaussians only (decisions from the fp32 run).
void or_project_backward(const float* params, int64_t n, int64_t ld, const or_camera* cam,
                         const double* g2d, double* grads) {
  std::vector<Proj<float>> g;
  project_all(params, n, ld, *cam, g);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    if (!g[i].visible) continue;
    double p[59];
    load_params<double>(params, ld, i, p);
    double gp[59];
    Proj<double> f;
    project_one<double>(p, *cam, f);
    project_backward_one<double>(f, p, *cam, g[i].rgb_pos, &g2d[size_t(i) * 9], gp);
    for (int k = 0; k < 59; ++k) grads[k * ld + i] += gp[k];
  }
}

// fp64 projection for one Gaussian's 2D outputs as a function of its 59
// parameters (u, v, A, B, C, opacity, r, g, b), colour clamp frozen at the
// fp32 decision of `base`.  For central differences of the projection
// backward.
void or_project_outputs_f64(const float* base, const double* params64, int64_t n, int64_t ld,
                            const or_camera* cam, double* out9) {
  for (int64_t i = 0; i < n; ++i) {
    float pf[59];
    load_params<float>(base, ld, i, pf);
    Proj<float> f;
    project_one<float>(pf, *cam, f);
    double p[59];
    for (int k = 0; k < 59; ++k) p[k] = params64[k * ld + i];
    Proj<double> o;
    project_one<double>(p, *cam, o);
    double* q = out9 + 9 * i;
    q[0] = o.u; q[1] = o.v; q[2] = o.A; q[3] = o.B; q[4] = o.C; q[5] = o.opacity;
    for (int c = 0; c < 3; ++c) q[6 + c] = f.rgb_pos[c] ? o.rgb_raw[c] : 0.0;
  }
}

// Adam over the listed rows only (fp64), Grendel-GS notes "Hyper-parameter
// scaling rule" for lr and betas (already scaled by the caller), bias
// corrections bc1 = 1 - beta1^t, bc2 = 1 - beta2^t:
//   m <- b1 m + (1-b1) g;  v <- b2 v + (1-b2) g^2;
//   p <- p - lr (m / bc1) / (sqrt(v / bc2) + eps).
// Unlisted rows are untouched.  Arrays are [59][ld]; rows = list of indices.
void or_adam(double* p, const double* g, double* m, double* v, int64_t ld,
             const int32_t* rows, int64_t nrows, double lr, double b1, double b2, double eps,
             double bc1, double bc2) {
#pragma omp parallel for schedule(static)
  for (int64_t s = 0; s < nrows; ++s) {
    const int64_t i = rows[s];
    for (int k = 0; k < 59; ++k) {
      const size_t q = size_t(k) * ld + i;
      m[q] = b1 * m[q] + (1.0 - b1) * g[q];
      v[q] = b2 * v[q] + (1.0 - b2) * g[q] * g[q];
      p[q] = p[q] - lr * (m[q] / bc1) / (std::sqrt(v[q] / bc2) + eps);
    }
  }
}

}  // extern "C"
