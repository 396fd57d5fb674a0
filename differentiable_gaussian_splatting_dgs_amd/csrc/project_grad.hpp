// Chain rule of the projection (the "back-propagation" step of the
// Grendel-GS notes' training pipeline): screen-space gradients of one
// Gaussian (2D mean, conic, opacity, colour) to all 59 parameters (SH
// coefficients and view direction, EWA covariance, scale via exp, rotation
// via the normalised quaternion, mean via the pinhole map).  Shared by the
// projection backward and its fusion with the optimiser step.
#pragma once

#include "gs_device.hpp"

namespace gs {

// d Y_k / d(x, y, z) of the SH basis, contracted with gY: returns the
// gradient with respect to the (unnormalised-in-form) direction components.
__device__ __forceinline__ void sh_dir_grad(float x, float y, float z, const float gY[16], float& gx, float& gy,
                                            float& gz) {
  const float xx = x * x, yy = y * y, zz = z * z;
  gx = GS_SH_C1 * gY[3] + GS_SH_C2A * (y * gY[4] + z * gY[7]) + 2.0f * GS_SH_C2C * x * gY[8] +
       6.0f * GS_SH_C3A * x * y * gY[9] + GS_SH_C3B * y * z * gY[10] + GS_SH_C3C * (5.0f * zz - 1.0f) * gY[13] +
       2.0f * GS_SH_C3E * x * z * gY[14] + GS_SH_C3A * (3.0f * xx - 3.0f * yy) * gY[15];
  gy = GS_SH_C1 * gY[1] + GS_SH_C2A * (x * gY[4] + z * gY[5]) - 2.0f * GS_SH_C2C * y * gY[8] +
       GS_SH_C3A * (3.0f * xx - 3.0f * yy) * gY[9] + GS_SH_C3B * x * z * gY[10] +
       GS_SH_C3C * (5.0f * zz - 1.0f) * gY[11] - 2.0f * GS_SH_C3E * y * z * gY[14] -
       6.0f * GS_SH_C3A * x * y * gY[15];
  gz = GS_SH_C1 * gY[2] + GS_SH_C2A * (y * gY[5] + x * gY[7]) + 6.0f * GS_SH_C2B * z * gY[6] +
       GS_SH_C3B * x * y * gY[10] + 10.0f * GS_SH_C3C * y * z * gY[11] + GS_SH_C3D * (15.0f * zz - 3.0f) * gY[12] +
       10.0f * GS_SH_C3C * x * z * gY[13] + GS_SH_C3E * (xx - yy) * gY[14];
}

// Writes a parameter gradient (kAdd: adds it to what g holds).
template <bool kAdd>
__device__ __forceinline__ void put_grad(float& d, float v) {
  if constexpr (kAdd)
    d += v;
  else
    d = v;
}

// p: the Gaussian's 59 parameters; (gu, gv, gA, gB, gC, go, gr, gg, gb): the
// screen-space gradients (record order); g: the 59 parameter gradients
// (kAdd: added to g, as g + this view's gradient).  With kShStride > 0 the
// 48 SH coefficient gradients (planes 11..58) are added to sh[j kShStride],
// j = plane - 11, instead of g (a caller that keeps them out of registers).
template <bool kAdd = false, int kShStride = 0>
__device__ __forceinline__ void project_grads(const float (&p)[59], const CamArgs& cam, float gu, float gv,
                                              float gA, float gB, float gC, float go, const float (&grgb)[3],
                                              float (&g)[59], float* sh = nullptr) {
  Fwd f;
  project(p, cam, f);
  // opacity logit
  put_grad<kAdd>(g[10], go * (f.opac * (1.0f - f.opac)));
  // colour: SH coefficients and view direction
  float Y[16];
  sh_eval(f.dir[0], f.dir[1], f.dir[2], Y);
  float gr[3];
#pragma unroll
  for (int ch = 0; ch < 3; ++ch) gr[ch] = f.raw[ch] > 0.0f ? grgb[ch] : 0.0f;
  float gY[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    if constexpr (kShStride > 0) {
      sh[(3 * k) * kShStride] += gr[0] * Y[k];
      sh[(3 * k + 1) * kShStride] += gr[1] * Y[k];
      sh[(3 * k + 2) * kShStride] += gr[2] * Y[k];
    } else {
      put_grad<kAdd>(g[11 + 3 * k], gr[0] * Y[k]);
      put_grad<kAdd>(g[12 + 3 * k], gr[1] * Y[k]);
      put_grad<kAdd>(g[13 + 3 * k], gr[2] * Y[k]);
    }
    gY[k] = gr[0] * p[11 + 3 * k] + gr[1] * p[12 + 3 * k] + gr[2] * p[13 + 3 * k];
  }
  float gdx, gdy, gdz;
  sh_dir_grad(f.dir[0], f.dir[1], f.dir[2], gY, gdx, gdy, gdz);
  const float dd = gdx * f.dir[0] + gdy * f.dir[1] + gdz * f.dir[2];
  const float idn = 1.0f / f.dn;
  float gx = (gdx - dd * f.dir[0]) * idn;
  float gy = (gdy - dd * f.dir[1]) * idn;
  float gz = (gdz - dd * f.dir[2]) * idn;
  // conic (A, B, C) = (c, -b, a) / det  ->  screen covariance (a, b, c)
  const float a = f.a, b = f.b, c = f.c;
  const float id2 = 1.0f / (f.det * f.det);
  const float ga = (-gA * c * c + gB * b * c - gC * b * b) * id2;
  const float gbb = (2.0f * gA * b * c - gB * (a * c + b * b) + 2.0f * gC * a * b) * id2;
  const float gc = (-gA * b * b + gB * a * b - gC * a * a) * id2;
  // full-matrix gradient of the 2x2 covariance
  const float G00 = ga, G01 = 0.5f * gbb, G11 = gc;
  const float* T = f.T;   // T00 T01 T02 T10 T11 T12
  const float* S = f.S;   // 00 01 02 11 12 22
  const float Sm[3][3] = {{S[0], S[1], S[2]}, {S[1], S[3], S[4]}, {S[2], S[4], S[5]}};
  // G_Sigma = T^T G2 T
  float GS[3][3];
#pragma unroll
  for (int ii = 0; ii < 3; ++ii)
#pragma unroll
    for (int jj = 0; jj < 3; ++jj)
      GS[ii][jj] = G00 * T[ii] * T[jj] + G01 * (T[ii] * T[3 + jj] + T[3 + ii] * T[jj]) + G11 * T[3 + ii] * T[3 + jj];
  // T Sigma
  float TS[2][3];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr)
#pragma unroll
    for (int kk = 0; kk < 3; ++kk)
      TS[rr][kk] = T[3 * rr] * Sm[0][kk] + T[3 * rr + 1] * Sm[1][kk] + T[3 * rr + 2] * Sm[2][kk];
  // G_T = 2 G2 (T Sigma)
  float GT[2][3];
#pragma unroll
  for (int kk = 0; kk < 3; ++kk) {
    GT[0][kk] = 2.0f * (G00 * TS[0][kk] + G01 * TS[1][kk]);
    GT[1][kk] = 2.0f * (G01 * TS[0][kk] + G11 * TS[1][kk]);
  }
  // G_J = G_T R^T (camera rotation)
  float GJ[2][3];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr)
#pragma unroll
    for (int m = 0; m < 3; ++m)
      GJ[rr][m] = GT[rr][0] * cam.R[3 * m] + GT[rr][1] * cam.R[3 * m + 1] + GT[rr][2] * cam.R[3 * m + 2];
  const float iz = f.iz, jx = cam.fx * iz, jy = cam.fy * iz;
  const float gtx = GJ[0][2] * (-jx * iz) + gu * jx;
  const float gty = GJ[1][2] * (-jy * iz) + gv * jy;
  const float gtz = GJ[0][0] * (-jx * iz) + GJ[0][2] * (2.0f * jx * f.ux * iz) + GJ[1][1] * (-jy * iz) +
                    GJ[1][2] * (2.0f * jy * f.uy * iz) - gu * jx * f.ux - gv * jy * f.uy;
  gx += cam.R[0] * gtx + cam.R[3] * gty + cam.R[6] * gtz;
  gy += cam.R[1] * gtx + cam.R[4] * gty + cam.R[7] * gtz;
  gz += cam.R[2] * gtx + cam.R[5] * gty + cam.R[8] * gtz;
  put_grad<kAdd>(g[0], gx);
  put_grad<kAdd>(g[1], gy);
  put_grad<kAdd>(g[2], gz);
  // Sigma = M M^T, M = Rq diag(s):  G_M = 2 G_Sigma M
  const float* Rq = f.r;
  float GR[3][3];
#pragma unroll
  for (int jj = 0; jj < 3; ++jj) {
    float gs = 0.0f;
#pragma unroll
    for (int ii = 0; ii < 3; ++ii) {
      const float gm = 2.0f * (GS[ii][0] * Rq[jj] * f.s[jj] + GS[ii][1] * Rq[3 + jj] * f.s[jj] +
                               GS[ii][2] * Rq[6 + jj] * f.s[jj]);
      gs += gm * Rq[3 * ii + jj];
      GR[ii][jj] = gm * f.s[jj];
    }
    put_grad<kAdd>(g[3 + jj], gs * f.s[jj]);
  }
  // rotation of the unit quaternion (w, x, y, z)
  const float w = f.w, x = f.x, y = f.y, z = f.z;
  const float gw = 2.0f * (-z * GR[0][1] + y * GR[0][2] + z * GR[1][0] - x * GR[1][2] - y * GR[2][0] + x * GR[2][1]);
  const float gqx = 2.0f * (y * GR[0][1] + z * GR[0][2] + y * GR[1][0] - 2.0f * x * GR[1][1] - w * GR[1][2] +
                            z * GR[2][0] + w * GR[2][1] - 2.0f * x * GR[2][2]);
  const float gqy = 2.0f * (-2.0f * y * GR[0][0] + x * GR[0][1] + w * GR[0][2] + x * GR[1][0] + z * GR[1][2] -
                            w * GR[2][0] + z * GR[2][1] - 2.0f * y * GR[2][2]);
  const float gqz = 2.0f * (-2.0f * z * GR[0][0] - w * GR[0][1] + x * GR[0][2] + w * GR[1][0] - 2.0f * z * GR[1][1] +
                            y * GR[1][2] + x * GR[2][0] + y * GR[2][1]);
  const float qdot = gw * w + gqx * x + gqy * y + gqz * z;
  const float iq = 1.0f / sqrtf(f.qn);
  put_grad<kAdd>(g[6], (gw - qdot * w) * iq);
  put_grad<kAdd>(g[7], (gqx - qdot * x) * iq);
  put_grad<kAdd>(g[8], (gqy - qdot * y) * iq);
  put_grad<kAdd>(g[9], (gqz - qdot * z) * iq);
}

}  // namespace gs
