// Image loss of the training pipeline (Grendel-GS notes: "L1 + SSIM loss"):
//   L = w_l1 * mean|I - I_t| + w_ssim * (1 - mean SSIM),   means over 3 H W,
// SSIM per channel with an 11x11 Gaussian window (sigma 1.5, zero-padded
// "same" correlation), C1 = 0.01^2, C2 = 0.03^2, and dL/dI.
//
// The window is separable, so both kernels stage a 32x8 output tile plus a
// 5-pixel halo in LDS and run a horizontal then a vertical 11-tap pass.
//   k_ssim_fwd: five local moments (mu_x, mu_y, E[x^2], E[y^2], E[xy]) ->
//     per-pixel SSIM and its partials wrt (mu_x, E[x^2], E[xy]); per-block
//     sums of SSIM and |x - y|.
//   k_ssim_bwd: the transposed (= same, the window is symmetric) window
//     applied to the three partial maps, combined into dL/dI with the L1
//     subgradient (0 at 0).
//   k_finish: fixed-order reduction of the block sums into L.
#include <algorithm>

#include "gs_scan.hpp"

namespace gs {
namespace {

constexpr int kLX = 32, kLY = 8, kHalo = 5;
constexpr int kSX = kLX + 2 * kHalo, kSY = kLY + 2 * kHalo;   // 42 x 18 staged
constexpr float kC1 = 0.0001f, kC2 = 0.0009f;

__device__ __forceinline__ float block_sum(float v, float* sh) {
  v = wave_sum_to_lane63(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 63) sh[w] = v;
  __syncthreads();
  float s = 0.0f;
  for (int k = 0; k < int(blockDim.x >> 6); ++k) s += sh[k];
  __syncthreads();
  return s;
}

__global__ __launch_bounds__(256) void k_ssim_fwd(const float* __restrict__ img, const float* __restrict__ tgt, int W,
                                                  int H, SsimWindow win, float* __restrict__ maps,
                                                  float* __restrict__ partial) {
  __shared__ float sx[kSY][kSX], sy[kSY][kSX];
  __shared__ float h[5][kSY][kLX];
  __shared__ float sh[4];
  const int t = threadIdx.x, lx = t & 31, ly = t >> 5;
  const int ox = blockIdx.x * kLX, oy = blockIdx.y * kLY;
  const int x = ox + lx, y = oy + ly;
  const bool inside = x < W && y < H;
  const size_t P = size_t(W) * H;
  float ssum = 0.0f, lsum = 0.0f;
  for (int ch = 0; ch < 3; ++ch) {
    const float* I = img + ch * P;
    const float* J = tgt + ch * P;
    for (int k = t; k < kSX * kSY; k += 256) {
      const int r = k / kSX, q = k % kSX;
      const int gx = ox + q - kHalo, gy = oy + r - kHalo;
      const bool in = gx >= 0 && gx < W && gy >= 0 && gy < H;
      sx[r][q] = in ? I[size_t(gy) * W + gx] : 0.0f;
      sy[r][q] = in ? J[size_t(gy) * W + gx] : 0.0f;
    }
    __syncthreads();
    for (int k = t; k < kSY * kLX; k += 256) {
      const int r = k / kLX, q = k % kLX;
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f, a4 = 0.f;
#pragma unroll
      for (int j = 0; j < 11; ++j) {
        const float u = sx[r][q + j], v = sy[r][q + j], gj = win.g[j];
        a0 = fmaf(gj, u, a0);
        a1 = fmaf(gj, v, a1);
        a2 = fmaf(gj, u * u, a2);
        a3 = fmaf(gj, v * v, a3);
        a4 = fmaf(gj, u * v, a4);
      }
      h[0][r][q] = a0; h[1][r][q] = a1; h[2][r][q] = a2; h[3][r][q] = a3; h[4][r][q] = a4;
    }
    __syncthreads();
    float mx = 0.f, my = 0.f, exx = 0.f, eyy = 0.f, exy = 0.f;
#pragma unroll
    for (int i = 0; i < 11; ++i) {
      const float gi = win.g[i];
      mx = fmaf(gi, h[0][ly + i][lx], mx);
      my = fmaf(gi, h[1][ly + i][lx], my);
      exx = fmaf(gi, h[2][ly + i][lx], exx);
      eyy = fmaf(gi, h[3][ly + i][lx], eyy);
      exy = fmaf(gi, h[4][ly + i][lx], exy);
    }
    if (inside) {
      const float vx = exx - mx * mx, vy = eyy - my * my, cxy = exy - mx * my;
      const float A1 = 2.0f * mx * my + kC1, A2 = 2.0f * cxy + kC2;
      const float B1 = mx * mx + my * my + kC1, B2 = vx + vy + kC2;
      const float iD = 1.0f / (B1 * B2);
      const float S = A1 * A2 * iD;
      const size_t pix = size_t(y) * W + x;
      maps[(3 * ch + 0) * P + pix] = (2.0f * my * (A2 - A1) - 2.0f * S * mx * (B2 - B1)) * iD;
      maps[(3 * ch + 1) * P + pix] = -S / B2;
      maps[(3 * ch + 2) * P + pix] = 2.0f * A1 * iD;
      ssum += S;
      lsum += fabsf(sx[ly + kHalo][lx + kHalo] - sy[ly + kHalo][lx + kHalo]);
    }
    __syncthreads();
  }
  const float s = block_sum(ssum, sh);
  const float l = block_sum(lsum, sh);
  if (t == 0) {
    const size_t b = size_t(blockIdx.y) * gridDim.x + blockIdx.x;
    partial[2 * b] = l;
    partial[2 * b + 1] = s;
  }
}

__global__ __launch_bounds__(256) void k_ssim_bwd(const float* __restrict__ img, const float* __restrict__ tgt, int W,
                                                  int H, SsimWindow win, const float* __restrict__ maps, float w_l1,
                                                  float w_ssim, float* __restrict__ dL) {
  __shared__ float sm[3][kSY][kSX];
  __shared__ float h[3][kSY][kLX];
  const int t = threadIdx.x, lx = t & 31, ly = t >> 5;
  const int ox = blockIdx.x * kLX, oy = blockIdx.y * kLY;
  const int x = ox + lx, y = oy + ly;
  const bool inside = x < W && y < H;
  const size_t P = size_t(W) * H;
  const float inv = 1.0f / (3.0f * float(P));
  for (int ch = 0; ch < 3; ++ch) {
    for (int k = t; k < kSX * kSY; k += 256) {
      const int r = k / kSX, q = k % kSX;
      const int gx = ox + q - kHalo, gy = oy + r - kHalo;
      const bool in = gx >= 0 && gx < W && gy >= 0 && gy < H;
      const size_t pix = size_t(gy) * W + gx;
#pragma unroll
      for (int m = 0; m < 3; ++m) sm[m][r][q] = in ? maps[(3 * ch + m) * P + pix] : 0.0f;
    }
    __syncthreads();
    for (int k = t; k < kSY * kLX; k += 256) {
      const int r = k / kLX, q = k % kLX;
      float a0 = 0.f, a1 = 0.f, a2 = 0.f;
#pragma unroll
      for (int j = 0; j < 11; ++j) {
        const float gj = win.g[j];
        a0 = fmaf(gj, sm[0][r][q + j], a0);
        a1 = fmaf(gj, sm[1][r][q + j], a1);
        a2 = fmaf(gj, sm[2][r][q + j], a2);
      }
      h[0][r][q] = a0; h[1][r][q] = a1; h[2][r][q] = a2;
    }
    __syncthreads();
    if (inside) {
      float b0 = 0.f, b1 = 0.f, b2 = 0.f;
#pragma unroll
      for (int i = 0; i < 11; ++i) {
        const float gi = win.g[i];
        b0 = fmaf(gi, h[0][ly + i][lx], b0);
        b1 = fmaf(gi, h[1][ly + i][lx], b1);
        b2 = fmaf(gi, h[2][ly + i][lx], b2);
      }
      const size_t pix = size_t(y) * W + x;
      const float xv = img[ch * P + pix], yv = tgt[ch * P + pix];
      const float d = xv - yv;
      const float sg = d > 0.0f ? 1.0f : (d < 0.0f ? -1.0f : 0.0f);
      dL[ch * P + pix] = w_l1 * inv * sg - w_ssim * inv * (b0 + 2.0f * xv * b1 + yv * b2);
    }
    __syncthreads();
  }
}

// L1 only: dL/dI and per-block |x - y| sums
__global__ __launch_bounds__(256) void k_l1(const float* __restrict__ img, const float* __restrict__ tgt, int64_t n3,
                                            float inv_w, float* __restrict__ dL, float* __restrict__ partial) {
  __shared__ float sh[4];
  float s = 0.0f;
  const int64_t base = int64_t(blockIdx.x) * 4096;
  for (int k = threadIdx.x; k < 4096; k += 256) {
    const int64_t i = base + k;
    if (i < n3) {
      const float d = img[i] - tgt[i];
      s += fabsf(d);
      dL[i] = d > 0.0f ? inv_w : (d < 0.0f ? -inv_w : 0.0f);
    }
  }
  const float tot = block_sum(s, sh);
  if (threadIdx.x == 0) {
    partial[2 * blockIdx.x] = tot;
    partial[2 * blockIdx.x + 1] = 0.0f;
  }
}

__global__ __launch_bounds__(256) void k_finish(const float* __restrict__ partial, int nb, float inv3p, float w_l1,
                                                float w_ssim, int with_ssim, float* __restrict__ loss) {
  __shared__ double sh[2][256];
  double l = 0.0, s = 0.0;
  for (int b = threadIdx.x; b < nb; b += 256) {
    l += partial[2 * b];
    s += partial[2 * b + 1];
  }
  sh[0][threadIdx.x] = l;
  sh[1][threadIdx.x] = s;
  __syncthreads();
  for (int d = 128; d > 0; d >>= 1) {
    if (int(threadIdx.x) < d) {
      sh[0][threadIdx.x] += sh[0][threadIdx.x + d];
      sh[1][threadIdx.x] += sh[1][threadIdx.x + d];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double l1 = sh[0][0] * double(inv3p);
    const double ss = with_ssim ? sh[1][0] * double(inv3p) : 1.0;
    *loss = float(double(w_l1) * l1 + double(w_ssim) * (1.0 - ss));
  }
}

inline int64_t ssim_blocks(int32_t W, int32_t H) {
  return int64_t((W + kLX - 1) / kLX) * ((H + kLY - 1) / kLY);
}

}  // namespace

size_t loss_ws_bytes(int32_t width, int32_t height) {
  const int64_t P = int64_t(width) * height;
  const int64_t nb = std::max<int64_t>(ssim_blocks(width, height), (3 * P + 4095) / 4096);
  return align_up(sizeof(float) * 9 * size_t(P), 256) + align_up(sizeof(float) * 2 * size_t(nb), 256);
}

hipError_t launch_loss(const float* image, const float* target, int32_t width, int32_t height,
                       float w_l1, float w_ssim, const SsimWindow& win, float* loss, float* dL_dimage,
                       void* ws, hipStream_t st) {
  const int64_t P = int64_t(width) * height;
  float* maps = static_cast<float*>(ws);
  float* partial = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(sizeof(float) * 9 * size_t(P), 256));
  const float inv3p = float(1.0 / (3.0 * double(P)));
  if (w_ssim != 0.0f) {
    const dim3 grid(unsigned((width + kLX - 1) / kLX), unsigned((height + kLY - 1) / kLY));
    k_ssim_fwd<<<grid, 256, 0, st>>>(image, target, width, height, win, maps, partial);
    k_ssim_bwd<<<grid, 256, 0, st>>>(image, target, width, height, win, maps, w_l1, w_ssim, dL_dimage);
    k_finish<<<1, 256, 0, st>>>(partial, int(ssim_blocks(width, height)), inv3p, w_l1, w_ssim, 1, loss);
  } else {
    const int64_t n3 = 3 * P;
    const int nb = int((n3 + 4095) / 4096);
    k_l1<<<nb, 256, 0, st>>>(image, target, n3, w_l1 * inv3p, dL_dimage, partial);
    k_finish<<<1, 256, 0, st>>>(partial, nb, inv3p, w_l1, 0.0f, 0, loss);
  }
  return hipGetLastError();
}

}  // namespace gs
