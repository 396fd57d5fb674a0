// Backward pass of one view (the "back-propagation" step of the Grendel-GS
// notes' training pipeline), in two kernels, one per entry point:
//
//  k_render_bwd  -- per 16x16 tile, reverse traversal of the tile's list from
//    the last Gaussian any pixel composited.  Each pixel rebuilds its
//    transmittance by division, T_i = T_{i+1} / (1 - alpha_i), carries the
//    suffix colour S (S_{i-1} = alpha_i c_i + (1 - alpha_i) S_i, S = 0 behind
//    the last one: black background), and forms
//      dL/dc_i = alpha_i T_i G,   dL/dalpha_i = T_i (c_i - S_i) . G,
//    then chains alpha = o e^power (unless clamped at 0.99) into the opacity,
//    the conic and the 2D mean.  Skip decisions are recomputed with the same
//    fp32 arithmetic as the forward, so exactly the composited set is
//    visited.  The nine per-pixel partials of a Gaussian are summed over the
//    wave with DPP row operations, over the four waves with LDS float
//    atomics, and leave the workgroup as nine global float atomics per
//    (Gaussian, tile).
//
//  k_project_bwd -- one thread per visible Gaussian: the chain rule of the
//    projection from the screen-space gradients to all 59 parameters
//    (SH coefficients and view direction, EWA covariance, scale via exp,
//    rotation via the normalised quaternion, mean via the pinhole map),
//    accumulated (+=) into the [59][ld] gradient planes; the consumed
//    screen-space rows are zeroed so the buffer is clean for the next view.
#include "gs_device.hpp"

namespace gs {
namespace {

constexpr int kG2 = 12;   // floats per Gaussian in the screen-gradient buffer

__global__ __launch_bounds__(kBlock) void k_render_bwd(const float4* __restrict__ proj, const int32_t* __restrict__ vals,
                                                       const uint32_t* __restrict__ ranges, int64_t num_pairs,
                                                       int W, int H, int TX, const float* __restrict__ T_final,
                                                       const uint32_t* __restrict__ last,
                                                       const float* __restrict__ dL_dimage, float* __restrict__ grad2d) {
  __shared__ float4 s_q0[kBlock];   // u, v, -A/2, -B
  __shared__ float4 s_q1[kBlock];   // -C/2, opacity, r, g
  __shared__ float4 s_box[kBlock];
  __shared__ float s_b[kBlock];
  __shared__ int32_t s_gid[kBlock];
  __shared__ float s_acc[kBlock][9];
  __shared__ uint32_t s_max;
  const int tile = blockIdx.x;
  const int tx = tile % TX, ty = tile / TX;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  const int bx = tx * kTile + (w & 1) * 8, by = ty * kTile + (w >> 1) * 8;
  const int px = bx + (lane & 7), py = by + (lane >> 3);
  const bool inside = px < W && py < H;
  const float bx0 = float(bx) + 0.5f, bx1 = bx0 + 7.0f;
  const float by0 = float(by) + 0.5f, by1 = by0 + 7.0f;
  uint32_t start = ranges[2 * tile], end = ranges[2 * tile + 1];
  if (end > uint64_t(num_pairs)) end = uint32_t(num_pairs);
  if (start > end) start = end;
  const float pxc = float(px) + 0.5f, pyc = float(py) + 0.5f;
  float T = 1.0f, G0 = 0.0f, G1 = 0.0f, G2 = 0.0f;
  uint32_t lastp = 0;
  if (inside) {
    const size_t pix = size_t(py) * W + px;
    const size_t P = size_t(W) * H;
    T = T_final[pix];
    lastp = last[pix];
    G0 = dL_dimage[pix];
    G1 = dL_dimage[P + pix];
    G2 = dL_dimage[2 * P + pix];
  }
  if (t == 0) s_max = 0;
  __syncthreads();
  if (lastp > 0) atomicMax(&s_max, lastp);
  __syncthreads();
  const uint32_t stop = start + min(s_max, end - start);
  float S0 = 0.0f, S1 = 0.0f, S2 = 0.0f;
  for (uint32_t bend = stop; bend > start;) {
    const uint32_t bbeg = (bend - start > uint32_t(kBlock)) ? bend - kBlock : start;
    const int cnt = int(bend - bbeg);
    __syncthreads();
    if (t < cnt) {
      const int64_t g = vals[bbeg + t];
      const float4 q0 = proj[4 * g], q1 = proj[4 * g + 1], q2 = proj[4 * g + 2];
      s_q0[t] = make_float4(q0.x, q0.y, -0.5f * q0.z, -q0.w);
      s_q1[t] = make_float4(-0.5f * q1.x, q1.y, q1.z, q1.w);
      s_b[t] = q2.x;
      s_box[t] = make_float4(q0.x - q2.y, q0.x + q2.y, q0.y - q2.z, q0.y + q2.z);
      s_gid[t] = int32_t(g);
    }
#pragma unroll
    for (int c = 0; c < 9; ++c) s_acc[t][c] = 0.0f;
    __syncthreads();
    for (int k = cnt - 1; k >= 0; --k) {
      const uint32_t pos = bbeg + uint32_t(k) - start;    // list position
      const bool mine = pos < lastp;
      if (!__any(mine)) continue;
      const float4 box = s_box[k];
      if (box.y < bx0 || box.x > bx1 || box.w < by0 || box.z > by1) continue;
      const float4 a = s_q0[k];
      const float4 c = s_q1[k];
      const float dx = pxc - a.x, dy = pyc - a.y;
      const float power = fmaf(dx, fmaf(a.z, dx, a.w * dy), (c.x * dy) * dy);
      float e = 0.0f, araw = 0.0f, alpha = 0.0f;
      bool contrib = mine && !(power > 0.0f || power < -5.6f);
      if (contrib) {
        e = pexp(power);
        araw = c.y * e;
        alpha = fminf(0.99f, araw);
        contrib = !(alpha < 1.0f / 255.0f);
      }
      float gu = 0.f, gv = 0.f, gA = 0.f, gB = 0.f, gC = 0.f, go = 0.f, gr = 0.f, gg = 0.f, gb = 0.f;
      if (contrib) {
        const float cb = s_b[k];
        const float Ti = T / (1.0f - alpha);
        const float wgt = alpha * Ti;
        gr = wgt * G0;
        gg = wgt * G1;
        gb = wgt * G2;
        const float dal = Ti * fmaf(cb - S2, G2, fmaf(c.w - S1, G1, (c.z - S0) * G0));
        S0 = fmaf(alpha, c.z, (1.0f - alpha) * S0);
        S1 = fmaf(alpha, c.w, (1.0f - alpha) * S1);
        S2 = fmaf(alpha, cb, (1.0f - alpha) * S2);
        T = Ti;
        if (!(araw > 0.99f)) {
          go = dal * e;
          const float dp = dal * alpha;
          const float A = -2.0f * a.z, B = -a.w, C = -2.0f * c.x;
          gA = dp * (-0.5f * dx * dx);
          gB = dp * (-dx * dy);
          gC = dp * (-0.5f * dy * dy);
          gu = dp * fmaf(A, dx, B * dy);
          gv = dp * fmaf(B, dx, C * dy);
        }
      }
      if (__any(contrib)) {
        gu = wave_sum_to_lane63(gu);
        gv = wave_sum_to_lane63(gv);
        gA = wave_sum_to_lane63(gA);
        gB = wave_sum_to_lane63(gB);
        gC = wave_sum_to_lane63(gC);
        go = wave_sum_to_lane63(go);
        gr = wave_sum_to_lane63(gr);
        gg = wave_sum_to_lane63(gg);
        gb = wave_sum_to_lane63(gb);
        if (lane == 63) {
          atomicAdd(&s_acc[k][0], gu);
          atomicAdd(&s_acc[k][1], gv);
          atomicAdd(&s_acc[k][2], gA);
          atomicAdd(&s_acc[k][3], gB);
          atomicAdd(&s_acc[k][4], gC);
          atomicAdd(&s_acc[k][5], go);
          atomicAdd(&s_acc[k][6], gr);
          atomicAdd(&s_acc[k][7], gg);
          atomicAdd(&s_acc[k][8], gb);
        }
      }
    }
    __syncthreads();
    if (t < cnt) {
      float* dst = grad2d + size_t(s_gid[t]) * kG2;
#pragma unroll
      for (int c = 0; c < 9; ++c) {
        const float v = s_acc[t][c];
        if (v != 0.0f) unsafeAtomicAdd(dst + c, v);
      }
    }
    bend = bbeg;
  }
}

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

__global__ __launch_bounds__(256) void k_project_bwd(const float* __restrict__ params, int64_t n, int64_t ld,
                                                     CamArgs cam, const int32_t* __restrict__ vis,
                                                     const int64_t* __restrict__ vis_count,
                                                     float4* __restrict__ grad2d, float* __restrict__ grads) {
  const int64_t r = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (r >= *vis_count) return;
  const int64_t i = vis[r];
  const float4 ga4 = grad2d[3 * i], gb4 = grad2d[3 * i + 1], gc4 = grad2d[3 * i + 2];
  const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
  grad2d[3 * i] = z4;            // consumed: the buffer is zero again for the next view
  grad2d[3 * i + 1] = z4;
  grad2d[3 * i + 2] = z4;
  const float gu = ga4.x, gv = ga4.y, gA = ga4.z, gB = ga4.w;
  const float gC = gb4.x, go = gb4.y, grgb[3] = {gb4.z, gb4.w, gc4.x};
  float p[59];
#pragma unroll
  for (int k = 0; k < 59; ++k) p[k] = params[int64_t(k) * ld + i];
  Fwd f;
  project(p, cam, f);
  float g[59];
  // opacity logit
  g[10] = go * (f.opac * (1.0f - f.opac));
  // colour: SH coefficients and view direction
  float Y[16];
  sh_eval(f.dir[0], f.dir[1], f.dir[2], Y);
  float gr[3];
#pragma unroll
  for (int ch = 0; ch < 3; ++ch) gr[ch] = f.raw[ch] > 0.0f ? grgb[ch] : 0.0f;
  float gY[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    g[11 + 3 * k] = gr[0] * Y[k];
    g[12 + 3 * k] = gr[1] * Y[k];
    g[13 + 3 * k] = gr[2] * Y[k];
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
  g[0] = gx;
  g[1] = gy;
  g[2] = gz;
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
    g[3 + jj] = gs * f.s[jj];
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
  g[6] = (gw - qdot * w) * iq;
  g[7] = (gqx - qdot * x) * iq;
  g[8] = (gqy - qdot * y) * iq;
  g[9] = (gqz - qdot * z) * iq;
#pragma unroll
  for (int k = 0; k < 59; ++k) grads[int64_t(k) * ld + i] += g[k];
}

}  // namespace

hipError_t launch_render_bwd(const float* proj, const int32_t* vals, const uint32_t* ranges, int64_t num_pairs,
                             int32_t width, int32_t height, const float* T_final, const uint32_t* last,
                             const float* dL_dimage, float* grad2d, hipStream_t st) {
  const int TX = (width + kTile - 1) / kTile, TY = (height + kTile - 1) / kTile;
  k_render_bwd<<<unsigned(TX * TY), kBlock, 0, st>>>(reinterpret_cast<const float4*>(proj), vals, ranges, num_pairs,
                                                     width, height, TX, T_final, last, dL_dimage, grad2d);
  return hipGetLastError();
}

hipError_t launch_project_bwd(const float* params, int64_t n, int64_t ld, const CamArgs& cam,
                              const int32_t* vis_idx, const int64_t* vis_count, float* grad2d, float* grads,
                              hipStream_t st) {
  if (n == 0) return hipSuccess;
  k_project_bwd<<<unsigned((n + 255) / 256), 256, 0, st>>>(params, n, ld, cam, vis_idx, vis_count,
                                                           reinterpret_cast<float4*>(grad2d), grads);
  return hipGetLastError();
}

}  // namespace gs
