// Image loss of the training pipeline (Grendel-GS notes: "L1 + SSIM loss"):
//   L = w_l1 * mean|I - I_t| + w_ssim * (1 - mean SSIM),   means over 3 H W,
// SSIM per channel with an 11x11 Gaussian window (sigma 1.5, zero-padded
// "same" correlation), C1 = 0.01^2, C2 = 0.03^2, and dL/dI.
//
// The window is separable.  Both SSIM kernels work on one channel of a
// 32x32 output tile per block (a 5-pixel halo staged in LDS, every thread's
// loads issued before any is waited for) and run a horizontal then a
// vertical 11-tap pass, each thread computing a short run of neighbouring
// outputs (four across or four down) from a sliding window held in
// registers.
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

constexpr int kLX = 32, kLY = 32, kHalo = 5;
constexpr int kSX = kLX + 2 * kHalo, kSY = kLY + 2 * kHalo;   // 42 x 42 staged
constexpr int kSXP = kSX + 2;                                    // row stride: 16-byte rows
constexpr int kHP = kLX + 1;                                     // horizontal-pass row stride (banks)
constexpr int kRun = 4;                                          // horizontal outputs per thread
constexpr int kRunV = 4;                                         // vertical outputs per thread
constexpr int kStage = (kSX * kSY + 255) / 256;                  // staged elements per thread
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

// 11-tap window of a run of R outputs: out[o] = sum_j g[j] in[o + j].
template <int R>
__device__ __forceinline__ void taps(const SsimWindow& win, const float (&in)[R + 10], float (&out)[R]) {
#pragma unroll
  for (int o = 0; o < R; ++o) {
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 11; ++j) a = fmaf(win.g[j], in[o + j], a);
    out[o] = a;
  }
}

// The kRun + 10 inputs of a horizontal run, as 16-byte LDS reads (the
// run's start is 16-byte aligned; neighbouring threads' runs are 16 bytes
// apart, so the reads are conflict-free).
__device__ __forceinline__ void load_run(const float* src, float (&in)[kRun + 10]) {
  const float4* s4 = reinterpret_cast<const float4*>(src);
#pragma unroll
  for (int k = 0; k < (kRun + 10 + 3) / 4; ++k) {
    const float4 q = s4[k];
    const float e[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (4 * k + c < kRun + 10) in[4 * k + c] = e[c];
  }
}

// Staging of `kN` planes of a tile with its halo: each thread holds up to
// kStage elements per plane in registers (zeros outside the image).  The
// loads of the next tile are issued before the current one is computed,
// so their latency overlaps that work.
template <int kN>
struct Staged {
  float v[kN][kStage];
};

struct TileId {
  int ox, oy, ch;
};

__device__ __forceinline__ TileId tile_id(int i, int tx, int ty) {
  TileId id;
  id.ox = (i % tx) * kLX;
  id.oy = ((i / tx) % ty) * kLY;
  id.ch = i / (tx * ty);
  return id;
}

template <int kN>
__device__ __forceinline__ void stage_load(const float* const (&src)[kN], int W, int H, int ox, int oy,
                                           Staged<kN>& st) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < kStage; ++i) {
    const int k = t + 256 * i;
    const int r = k / kSX, q = k - r * kSX;
    const int gx = ox + q - kHalo, gy = oy + r - kHalo;
    const bool in = k < kSX * kSY && gx >= 0 && gx < W && gy >= 0 && gy < H;
    const size_t g = in ? size_t(gy) * W + gx : 0;
#pragma unroll
    for (int m = 0; m < kN; ++m) st.v[m][i] = in ? src[m][g] : 0.0f;
  }
}

template <int kN>
__device__ __forceinline__ void stage_store(const Staged<kN>& st, float* lds, int lds_plane) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < kStage; ++i) {
    const int k = t + 256 * i;
    const int r = k / kSX, q = k - r * kSX;
    if (k < kSX * kSY)
#pragma unroll
      for (int m = 0; m < kN; ++m) lds[m * lds_plane + r * kSXP + q] = st.v[m][i];
  }
}

// Persistent: block b takes tiles b, b + gridDim.x, ... of the tx x ty x 3
// (channel-major) tiles; per tile the per-block sums go to partial[2 i].
__global__ __launch_bounds__(256) void k_ssim_fwd(const float* __restrict__ img, const float* __restrict__ tgt, int W,
                                                  int H, int tx, int ty, SsimWindow win, float* __restrict__ maps,
                                                  float* __restrict__ partial) {
  __shared__ __align__(16) float sxy[2][kSY][kSXP];
  __shared__ float h[5][kSY][kHP];
  __shared__ float sh[4];
  const int t = threadIdx.x;
  const size_t P = size_t(W) * H;
  const int ntiles = 3 * tx * ty;
  int i = blockIdx.x;
  if (i >= ntiles) return;
  Staged<2> st;
  {
    const TileId id = tile_id(i, tx, ty);
    const float* const src[2] = {img + id.ch * P, tgt + id.ch * P};
    stage_load<2>(src, W, H, id.ox, id.oy, st);
  }
  for (; i < ntiles; i += gridDim.x) {
    const TileId id = tile_id(i, tx, ty);
    const int ox = id.ox, oy = id.oy, ch = id.ch;
    stage_store<2>(st, &sxy[0][0][0], kSY * kSXP);
    __syncthreads();
    if (i + int(gridDim.x) < ntiles) {
      const TileId nx = tile_id(i + gridDim.x, tx, ty);
      const float* const src[2] = {img + nx.ch * P, tgt + nx.ch * P};
      stage_load<2>(src, W, H, nx.ox, nx.oy, st);
    }
    // horizontal: row r, columns c0 .. c0 + 3 of the five moment maps
    for (int task = t; task < kSY * (kLX / kRun); task += 256) {
      const int r = task / (kLX / kRun), c0 = (task % (kLX / kRun)) * kRun;
      float u[kRun + 10], v[kRun + 10], p[kRun + 10], o[kRun];
      load_run(&sxy[0][r][c0], u);
      load_run(&sxy[1][r][c0], v);
      taps<kRun>(win, u, o);
#pragma unroll
      for (int q = 0; q < kRun; ++q) h[0][r][c0 + q] = o[q];
      taps<kRun>(win, v, o);
#pragma unroll
      for (int q = 0; q < kRun; ++q) h[1][r][c0 + q] = o[q];
#pragma unroll
      for (int k = 0; k < kRun + 10; ++k) p[k] = u[k] * u[k];
      taps<kRun>(win, p, o);
#pragma unroll
      for (int q = 0; q < kRun; ++q) h[2][r][c0 + q] = o[q];
#pragma unroll
      for (int k = 0; k < kRun + 10; ++k) p[k] = v[k] * v[k];
      taps<kRun>(win, p, o);
#pragma unroll
      for (int q = 0; q < kRun; ++q) h[3][r][c0 + q] = o[q];
#pragma unroll
      for (int k = 0; k < kRun + 10; ++k) p[k] = u[k] * v[k];
      taps<kRun>(win, p, o);
#pragma unroll
      for (int q = 0; q < kRun; ++q) h[4][r][c0 + q] = o[q];
    }
    __syncthreads();
    // vertical: column lx, rows r0 .. r0 + kRunV - 1
    float ssum = 0.0f, lsum = 0.0f;
    {
      const int lx = t % kLX, r0 = (t / kLX) * kRunV;
      float m[5][kRunV];
#pragma unroll
      for (int k = 0; k < 5; ++k) {
        float col[kRunV + 10];
#pragma unroll
        for (int j = 0; j < kRunV + 10; ++j) col[j] = h[k][r0 + j][lx];
        taps<kRunV>(win, col, m[k]);
      }
      const int x = ox + lx;
#pragma unroll
      for (int q = 0; q < kRunV; ++q) {
        const int y = oy + r0 + q;
        if (x >= W || y >= H) continue;
        const float mx = m[0][q], my = m[1][q], exx = m[2][q], eyy = m[3][q], exy = m[4][q];
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
        lsum += fabsf(sxy[0][r0 + q + kHalo][lx + kHalo] - sxy[1][r0 + q + kHalo][lx + kHalo]);
      }
    }
    // (block_sum's barriers also keep the next tile's LDS writes behind
    // every read of this one)
    const float s2 = block_sum(ssum, sh);
    const float l2 = block_sum(lsum, sh);
    if (t == 0) {
      partial[2 * i] = l2;
      partial[2 * i + 1] = s2;
    }
  }
}

// Persistent like k_ssim_fwd.
__global__ __launch_bounds__(256) void k_ssim_bwd(const float* __restrict__ img, const float* __restrict__ tgt, int W,
                                                  int H, int tx, int ty, SsimWindow win, const float* __restrict__ maps,
                                                  float w_l1, float w_ssim, float* __restrict__ dL) {
  __shared__ __align__(16) float sm[3][kSY][kSXP];
  __shared__ float h[3][kSY][kHP];
  const int t = threadIdx.x;
  const size_t P = size_t(W) * H;
  const float inv = 1.0f / (3.0f * float(P));
  const int ntiles = 3 * tx * ty;
  int i = blockIdx.x;
  if (i >= ntiles) return;
  Staged<3> st;
  {
    const TileId id = tile_id(i, tx, ty);
    const float* const src[3] = {maps + (3 * id.ch) * P, maps + (3 * id.ch + 1) * P, maps + (3 * id.ch + 2) * P};
    stage_load<3>(src, W, H, id.ox, id.oy, st);
  }
  const int lx = t % kLX, r0 = (t / kLX) * kRunV;
  for (; i < ntiles; i += gridDim.x) {
    const TileId id = tile_id(i, tx, ty);
    const int ox = id.ox, oy = id.oy, ch = id.ch;
    // every read of the previous tile's LDS planes is behind this barrier
    __syncthreads();
    stage_store<3>(st, &sm[0][0][0], kSY * kSXP);
    __syncthreads();
    if (i + int(gridDim.x) < ntiles) {
      const TileId nx = tile_id(i + gridDim.x, tx, ty);
      const float* const src[3] = {maps + (3 * nx.ch) * P, maps + (3 * nx.ch + 1) * P, maps + (3 * nx.ch + 2) * P};
      stage_load<3>(src, W, H, nx.ox, nx.oy, st);
    }
    for (int task = t; task < kSY * (kLX / kRun); task += 256) {
      const int r = task / (kLX / kRun), c0 = (task % (kLX / kRun)) * kRun;
#pragma unroll
      for (int m = 0; m < 3; ++m) {
        float in[kRun + 10], o[kRun];
        load_run(&sm[m][r][c0], in);
        taps<kRun>(win, in, o);
#pragma unroll
        for (int q = 0; q < kRun; ++q) h[m][r][c0 + q] = o[q];
      }
    }
    __syncthreads();
    const int x = ox + lx;
    // the output pixels' image and target values, loaded before the taps
    float xv[kRunV], yv[kRunV];
#pragma unroll
    for (int q = 0; q < kRunV; ++q) {
      const int y = oy + r0 + q;
      const bool in = x < W && y < H;
      const size_t pix = in ? size_t(y) * W + x : 0;
      xv[q] = in ? img[ch * P + pix] : 0.0f;
      yv[q] = in ? tgt[ch * P + pix] : 0.0f;
    }
    float b[3][kRunV];
#pragma unroll
    for (int m = 0; m < 3; ++m) {
      float col[kRunV + 10];
#pragma unroll
      for (int j = 0; j < kRunV + 10; ++j) col[j] = h[m][r0 + j][lx];
      taps<kRunV>(win, col, b[m]);
    }
#pragma unroll
    for (int q = 0; q < kRunV; ++q) {
      const int y = oy + r0 + q;
      if (x >= W || y >= H) continue;
      const size_t pix = size_t(y) * W + x;
      const float d = xv[q] - yv[q];
      const float sg = d > 0.0f ? 1.0f : (d < 0.0f ? -1.0f : 0.0f);
      dL[ch * P + pix] = w_l1 * inv * sg - w_ssim * inv * (b[0][q] + 2.0f * xv[q] * b[1][q] + yv[q] * b[2][q]);
    }
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
  // each thread's strided sums in index order, their loads issued eight at
  // a time
  constexpr int kB = 8;
  for (int b0 = threadIdx.x; b0 < nb; b0 += 256 * kB) {
    float2 v[kB];
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const int b = b0 + 256 * j;
      v[j] = b < nb ? reinterpret_cast<const float2*>(partial)[b] : make_float2(0.0f, 0.0f);
    }
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      if (b0 + 256 * j < nb) {
        l += v[j].x;
        s += v[j].y;
      }
    }
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

// Workgroups of a persistent SSIM kernel: as many as fit on the device at
// once (LDS-limited), at most one per tile.
int persistent_blocks(int per_cu, int64_t tiles) {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return int(std::min<int64_t>(tiles, int64_t(cus[dev]) * per_cu));
}

inline int64_t ssim_blocks(int32_t W, int32_t H) {
  return 3 * int64_t((W + kLX - 1) / kLX) * ((H + kLY - 1) / kLY);
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
    const int tx = (width + kLX - 1) / kLX, ty = (height + kLY - 1) / kLY;
    const int64_t tiles = ssim_blocks(width, height);
    // 42.5 KB / 38.8 KB of LDS per workgroup: 3 / 4 per CU
    k_ssim_fwd<<<persistent_blocks(3, tiles), 256, 0, st>>>(image, target, width, height, tx, ty, win, maps, partial);
    k_ssim_bwd<<<persistent_blocks(4, tiles), 256, 0, st>>>(image, target, width, height, tx, ty, win, maps, w_l1,
                                                            w_ssim, dL_dimage);
    k_finish<<<1, 256, 0, st>>>(partial, int(tiles), inv3p, w_l1, w_ssim, 1, loss);
  } else {
    const int64_t n3 = 3 * P;
    const int nb = int((n3 + 4095) / 4096);
    k_l1<<<nb, 256, 0, st>>>(image, target, n3, w_l1 * inv3p, dL_dimage, partial);
    k_finish<<<1, 256, 0, st>>>(partial, nb, inv3p, w_l1, 0.0f, 0, loss);
  }
  return hipGetLastError();
}

}  // namespace gs
