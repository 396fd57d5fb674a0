// Image loss of the training pipeline (Grendel-GS notes: "L1 + SSIM loss"):
//   L = w_l1 * mean|I - I_t| + w_ssim * (1 - mean SSIM),   means over 3 H W,
// SSIM per channel with an 11x11 Gaussian window (sigma 1.5, zero-padded
// "same" correlation), C1 = 0.01^2, C2 = 0.03^2, and dL/dI.
//
// The window is separable.  Both SSIM kernels work on one channel of a
// 32x32 output tile at a time (persistent workgroups of 256 threads, the
// tiles of an eighth of the image per XCD so neighbouring halos share an
// L2; the next tile's 42x42 halo region is loaded into registers while the
// current one is computed) and run a horizontal then a vertical 11-tap
// pass over LDS: 168 horizontal runs of eight outputs (the 42 rows the
// vertical pass needs), then one vertical run of four outputs per thread.
//   k_ssim_fwd: four local moments (mu_x, mu_y, E[x^2 + y^2], E[xy]: the
//     variances enter SSIM only through sigma_x^2 + sigma_y^2, so one
//     windowed map of x^2 + y^2 serves both) -> per-pixel SSIM and its
//     partials wrt (mu_x, E[x^2], E[xy]); per-tile sums of SSIM and
//     |x - y|.
//   k_ssim_bwd: the transposed (= same, the window is symmetric) window
//     applied to the three partial maps, combined into dL/dI with the L1
//     subgradient (0 at 0).
//   the loss scalar: fixed-order fp64 reduction of the per-tile sums into
//     L, by the last workgroup of k_ssim_bwd once its tiles are done (the
//     sums are complete: k_ssim_fwd has finished); the L1-only path uses
//     k_finish.
#include <algorithm>

#include "gs_scan.hpp"

namespace gs {
namespace {

constexpr int kLX = 32, kLY = 32, kHalo = 5;
constexpr int kSX = kLX + 2 * kHalo, kSY = kLY + 2 * kHalo;   // 42 x 42 staged
constexpr int kSXP = kSX + 2;                                    // staged row stride: 16-byte rows
constexpr int kHP = kLX + 4;                                     // horizontal-pass row stride: 16-byte rows
constexpr int kRunH = 8;                                         // horizontal outputs per task
constexpr int kRunV = 4;                                         // vertical outputs per thread
constexpr int kTasksH = kSY * (kLX / kRunH);                     // 168 horizontal tasks per tile
constexpr int kStageRows = 6;                                    // staged rows per pass (6 x 42 threads)
constexpr int kStage = (kSY + kStageRows - 1) / kStageRows;      // passes: 7
constexpr float kC1 = 0.0001f, kC2 = 0.0009f;
static_assert(kLX * (kLY / kRunV) == 256, "one vertical task per thread");
static_assert(kStageRows * kSX <= 256 && kStage * kStageRows == kSY, "staging layout");

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

// Two block sums with one pair of barriers (sh: 2 x waves floats).
__device__ __forceinline__ float2 block_sum2(float a, float b, float* sh) {
  a = wave_sum_to_lane63(a);
  b = wave_sum_to_lane63(b);
  const int w = threadIdx.x >> 6, nw = int(blockDim.x >> 6);
  if ((threadIdx.x & 63) == 63) {
    sh[w] = a;
    sh[nw + w] = b;
  }
  __syncthreads();
  float2 s = make_float2(0.0f, 0.0f);
  for (int k = 0; k < nw; ++k) {
    s.x += sh[k];
    s.y += sh[nw + k];
  }
  __syncthreads();
  return s;
}

// Fixed-order reduction of nb (|x - y| sum, SSIM sum) float pairs into the
// loss by one workgroup of 256 threads: per-thread strided fp64 sums in
// index order (loads issued eight at a time), then a tree in shared memory.
__device__ __forceinline__ void finish_loss(const float* __restrict__ partial, int nb, float inv3p, float w_l1,
                                            float w_ssim, int with_ssim, float* __restrict__ loss,
                                            double (*sh)[256]) {
  double l = 0.0, s = 0.0;
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

// The kRunH + 10 inputs of a horizontal run, as 16-byte LDS reads from a
// 16-byte aligned start.
__device__ __forceinline__ void load_run(const float* src, float (&in)[kRunH + 10]) {
  const float4* s4 = reinterpret_cast<const float4*>(src);
#pragma unroll
  for (int k = 0; k < (kRunH + 10 + 3) / 4; ++k) {
    const float4 q = s4[k];
    const float e[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (4 * k + c < kRunH + 10) in[4 * k + c] = e[c];
  }
}

// A run of kRunH outputs stored as float4 pairs (the row stride keeps them
// 16-byte aligned).
__device__ __forceinline__ void store_run(float* dst, const float (&o)[kRunH]) {
  float4* d4 = reinterpret_cast<float4*>(dst);
#pragma unroll
  for (int k = 0; k < kRunH / 4; ++k) d4[k] = make_float4(o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]);
}

// The float `e` elements past a wave-uniform base.  With Ix = uint32_t (a
// plane of fewer than 2^30 pixels) the byte offset is a 32-bit lane value,
// so the access takes the scalar-base + 32-bit vector-offset form and no
// 64-bit address arithmetic per lane.
template <typename Ix>
__device__ __forceinline__ const float& elem(const float* base, Ix e) {
  return *reinterpret_cast<const float*>(reinterpret_cast<const char*>(base) + e * Ix(4));
}
template <typename Ix>
__device__ __forceinline__ float& elem(float* base, Ix e) {
  return *reinterpret_cast<float*>(reinterpret_cast<char*>(base) + e * Ix(4));
}

// Staging of `kN` planes of a tile with its halo (42 x 42): thread t < 252
// owns column t % 42 and rows t / 42 + 6 i (i = 0..6), so its column bound
// is tested once per tile and its address steps by 6 rows; values outside
// the image are zero.  The loads of the next tile are issued before the
// current one is computed, so their latency overlaps that work.
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

template <typename Ix, int kN>
__device__ __forceinline__ void stage_load(const float* const (&src)[kN], int W, int H, int ox, int oy,
                                           Staged<kN>& st) {
  const int t = threadIdx.x;
  const int q = t % kSX, r0 = t / kSX;
  const int gx = ox + q - kHalo;
  const bool colok = t < kStageRows * kSX && gx >= 0 && gx < W;
#pragma unroll
  for (int i = 0; i < kStage; ++i) {
    const int gy = oy + r0 + kStageRows * i - kHalo;
    const bool in = colok && gy >= 0 && gy < H;
    const Ix g = in ? Ix(gy) * Ix(W) + Ix(gx) : Ix(0);
#pragma unroll
    for (int m = 0; m < kN; ++m) st.v[m][i] = in ? elem<Ix>(src[m], g) : 0.0f;
  }
}

template <int kN>
__device__ __forceinline__ void stage_store(const Staged<kN>& st, float* lds, int lds_plane) {
  const int t = threadIdx.x;
  if (t >= kStageRows * kSX) return;
  const int q = t % kSX, r0 = t / kSX;
#pragma unroll
  for (int i = 0; i < kStage; ++i)
#pragma unroll
    for (int m = 0; m < kN; ++m) lds[m * lds_plane + (r0 + kStageRows * i) * kSXP + q] = st.v[m][i];
}

// Persistent tile walk, XCD-aware: workgroups go to the 8 XCDs round robin
// (workgroup b on XCD b mod 8), so XCD x's workgroups take the x-th eighth
// of the (channel-major, row-major) tile sequence: neighbouring tiles,
// whose halos overlap, are read through the same L2.
struct TileWalk {
  int first, end, step;
};

__device__ __forceinline__ TileWalk tile_walk(int ntiles) {
  const int G = int(gridDim.x), b = int(blockIdx.x);
  TileWalk w;
  if (G < 8) {
    w.first = b;
    w.end = ntiles;
    w.step = G;
    return w;
  }
  const int x = b & 7, l = b >> 3;
  const int nb = (G - x + 7) >> 3;                     // workgroups on XCD x
  const int lo = int(int64_t(ntiles) * x / 8), hi = int(int64_t(ntiles) * (x + 1) / 8);
  w.first = lo + l;
  w.end = hi;
  w.step = nb;
  return w;
}

// Per tile the per-block sums go to partial[2 i].  Ix: the type of a
// pixel offset within a plane (uint32_t below 2^30 pixels, else uint64_t).
template <typename Ix>
__global__ __launch_bounds__(256) void k_ssim_fwd(const float* __restrict__ img, const float* __restrict__ tgt, int W,
                                                  int H, int tx, int ty, SsimWindow win, float* __restrict__ maps,
                                                  float* __restrict__ partial) {
  __shared__ __align__(16) float sxy[2][kSY][kSXP];
  __shared__ __align__(16) float h[4][kSY][kHP];
  __shared__ float sh[8];
  // issue priority over the next view's binning sharing the CUs (this
  // kernel is on the step's critical path)
  __builtin_amdgcn_s_setprio(2);
  const int t = threadIdx.x;
  const size_t P = size_t(W) * H;
  const int ntiles = 3 * tx * ty;
  const TileWalk wk = tile_walk(ntiles);
  int i = wk.first;
  if (i >= wk.end) return;
  Staged<2> st;
  {
    const TileId id = tile_id(i, tx, ty);
    const float* const src[2] = {img + id.ch * P, tgt + id.ch * P};
    stage_load<Ix, 2>(src, W, H, id.ox, id.oy, st);
  }
  const int lx = t % kLX, r0 = (t / kLX) * kRunV;
  for (; i < wk.end; i += wk.step) {
    const TileId id = tile_id(i, tx, ty);
    const int ox = id.ox, oy = id.oy, ch = id.ch;
    stage_store<2>(st, &sxy[0][0][0], kSY * kSXP);
    __syncthreads();
    if (i + wk.step < wk.end) {
      const TileId nx = tile_id(i + wk.step, tx, ty);
      const float* const src[2] = {img + nx.ch * P, tgt + nx.ch * P};
      stage_load<Ix, 2>(src, W, H, nx.ox, nx.oy, st);
    }
    // horizontal: row r, columns c0 .. c0 + 7 of the four moment maps
    if (t < kTasksH) {
      const int r = t / (kLX / kRunH), c0 = (t % (kLX / kRunH)) * kRunH;
      float u[kRunH + 10], v[kRunH + 10], p[kRunH + 10], o[kRunH];
      load_run(&sxy[0][r][c0], u);
      load_run(&sxy[1][r][c0], v);
      taps<kRunH>(win, u, o);
      store_run(&h[0][r][c0], o);
      taps<kRunH>(win, v, o);
      store_run(&h[1][r][c0], o);
#pragma unroll
      for (int k = 0; k < kRunH + 10; ++k) p[k] = fmaf(u[k], u[k], v[k] * v[k]);
      taps<kRunH>(win, p, o);
      store_run(&h[2][r][c0], o);
#pragma unroll
      for (int k = 0; k < kRunH + 10; ++k) p[k] = u[k] * v[k];
      taps<kRunH>(win, p, o);
      store_run(&h[3][r][c0], o);
    }
    __syncthreads();
    // vertical: column lx, rows r0 .. r0 + kRunV - 1
    float ssum = 0.0f, lsum = 0.0f;
    {
      float m[4][kRunV];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float col[kRunV + 10];
#pragma unroll
        for (int j = 0; j < kRunV + 10; ++j) col[j] = h[k][r0 + j][lx];
        taps<kRunV>(win, col, m[k]);
      }
      const int x = ox + lx;
      float* const map0 = maps + size_t(3 * ch) * P;
      float* const map1 = map0 + P;
      float* const map2 = map1 + P;
#pragma unroll
      for (int q = 0; q < kRunV; ++q) {
        const int y = oy + r0 + q;
        if (x >= W || y >= H) continue;
        const float mx = m[0][q], my = m[1][q], ess = m[2][q], exy = m[3][q];
        const float cxy = exy - mx * my;
        const float A1 = 2.0f * mx * my + kC1, A2 = 2.0f * cxy + kC2;
        const float mm = fmaf(mx, mx, my * my);
        const float B1 = mm + kC1, B2 = (ess - mm) + kC2;
        // (hardware reciprocals: the loss feeds no discrete decision, and
        // their 1-ulp error is far inside its tolerance)
        const float iB2 = __builtin_amdgcn_rcpf(B2);
        const float iD = __builtin_amdgcn_rcpf(B1) * iB2;
        const float S = A1 * A2 * iD;
        const Ix pix = Ix(y) * Ix(W) + Ix(x);
        elem<Ix>(map0, pix) = (2.0f * my * (A2 - A1) - 2.0f * S * mx * (B2 - B1)) * iD;
        elem<Ix>(map1, pix) = -S * iB2;
        elem<Ix>(map2, pix) = 2.0f * A1 * iD;
        ssum += S;
        lsum += fabsf(sxy[0][r0 + q + kHalo][lx + kHalo] - sxy[1][r0 + q + kHalo][lx + kHalo]);
      }
    }
    // (block_sum's barriers also keep the next tile's LDS writes behind
    // every read of this one)
    const float2 ls = block_sum2(lsum, ssum, sh);
    if (t == 0) {
      partial[2 * i] = ls.x;
      partial[2 * i + 1] = ls.y;
    }
  }
}

// The same tiles, walk and offset type as k_ssim_fwd; the last workgroup (which has at
// most as many tiles as any other) first turns k_ssim_fwd's per-tile sums
// into the loss (they are complete: k_ssim_fwd has finished), so that
// single-workgroup reduction runs beside the other workgroups' tiles
// rather than after them.
template <typename Ix>
__global__ __launch_bounds__(256) void k_ssim_bwd(const float* __restrict__ img, const float* __restrict__ tgt, int W,
                                                  int H, int tx, int ty, SsimWindow win, const float* __restrict__ maps,
                                                  float w_l1, float w_ssim, float* __restrict__ dL,
                                                  const float* __restrict__ partial, float* __restrict__ loss) {
  __shared__ __align__(16) float sm[3][kSY][kSXP];
  __shared__ __align__(16) float h[3][kSY][kHP];   // (the last block reuses it for the fp64 reduction)
  __builtin_amdgcn_s_setprio(2);   // (as the forward)
  const int t = threadIdx.x;
  const size_t P = size_t(W) * H;
  const float inv = 1.0f / (3.0f * float(P));
  const int ntiles = 3 * tx * ty;
  const TileWalk wk = tile_walk(ntiles);
  int i = wk.first;
  Staged<3> st;
  if (i < wk.end) {
    const TileId id = tile_id(i, tx, ty);
    const float* const src[3] = {maps + (3 * id.ch) * P, maps + (3 * id.ch + 1) * P, maps + (3 * id.ch + 2) * P};
    stage_load<Ix, 3>(src, W, H, id.ox, id.oy, st);
  }
  if (blockIdx.x == gridDim.x - 1)   // (its LDS planes are free until the first tile)
    finish_loss(partial, ntiles, 1.0f / (3.0f * float(P)), w_l1, w_ssim, 1, loss,
                reinterpret_cast<double(*)[256]>(&h[0][0][0]));
  const int lx = t % kLX, r0 = (t / kLX) * kRunV;
  for (; i < wk.end; i += wk.step) {
    const TileId id = tile_id(i, tx, ty);
    const int ox = id.ox, oy = id.oy, ch = id.ch;
    // every read of the previous tile's LDS planes is behind this barrier
    __syncthreads();
    stage_store<3>(st, &sm[0][0][0], kSY * kSXP);
    __syncthreads();
    if (i + wk.step < wk.end) {
      const TileId nx = tile_id(i + wk.step, tx, ty);
      const float* const src[3] = {maps + (3 * nx.ch) * P, maps + (3 * nx.ch + 1) * P, maps + (3 * nx.ch + 2) * P};
      stage_load<Ix, 3>(src, W, H, nx.ox, nx.oy, st);
    }
    if (t < kTasksH) {
      const int r = t / (kLX / kRunH), c0 = (t % (kLX / kRunH)) * kRunH;
#pragma unroll
      for (int m = 0; m < 3; ++m) {
        float in[kRunH + 10], o[kRunH];
        load_run(&sm[m][r][c0], in);
        taps<kRunH>(win, in, o);
        store_run(&h[m][r][c0], o);
      }
    }
    __syncthreads();
    const int x = ox + lx;
    const float* const imc = img + ch * P;
    const float* const tgc = tgt + ch * P;
    float* const dlc = dL + ch * P;
    // the output pixels' image and target values, loaded before the taps
    float xv[kRunV], yv[kRunV];
#pragma unroll
    for (int q = 0; q < kRunV; ++q) {
      const int y = oy + r0 + q;
      const bool in = x < W && y < H;
      const Ix pix = in ? Ix(y) * Ix(W) + Ix(x) : Ix(0);
      xv[q] = in ? elem<Ix>(imc, pix) : 0.0f;
      yv[q] = in ? elem<Ix>(tgc, pix) : 0.0f;
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
      const Ix pix = Ix(y) * Ix(W) + Ix(x);
      const float d = xv[q] - yv[q];
      const float sg = d > 0.0f ? 1.0f : (d < 0.0f ? -1.0f : 0.0f);
      elem<Ix>(dlc, pix) = w_l1 * inv * sg - w_ssim * inv * (b[0][q] + 2.0f * xv[q] * b[1][q] + yv[q] * b[2][q]);
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
  finish_loss(partial, nb, inv3p, w_l1, w_ssim, with_ssim, loss, sh);
}

// Workgroups of a persistent SSIM kernel: per_cu per compute unit, at most
// one per tile.
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
    // 39 KB / 40 KB of LDS per workgroup: four of each fit on a CU.  Twice
    // that many workgroups, each with half the tiles: where other kernels
    // still hold part of the CUs, the second half starts wherever slots free
    // up, so fewer tiles wait behind a late-starting workgroup
    const int nb = persistent_blocks(8, tiles);
    if (P < (int64_t(1) << 30)) {
      k_ssim_fwd<uint32_t><<<nb, 256, 0, st>>>(image, target, width, height, tx, ty, win, maps, partial);
      k_ssim_bwd<uint32_t><<<nb, 256, 0, st>>>(image, target, width, height, tx, ty, win, maps, w_l1, w_ssim,
                                               dL_dimage, partial, loss);
    } else {
      k_ssim_fwd<uint64_t><<<nb, 256, 0, st>>>(image, target, width, height, tx, ty, win, maps, partial);
      k_ssim_bwd<uint64_t><<<nb, 256, 0, st>>>(image, target, width, height, tx, ty, win, maps, w_l1, w_ssim,
                                               dL_dimage, partial, loss);
    }
  } else {
    const int64_t n3 = 3 * P;
    const int nb = int((n3 + 4095) / 4096);
    k_l1<<<nb, 256, 0, st>>>(image, target, n3, w_l1 * inv3p, dL_dimage, partial);
    k_finish<<<1, 256, 0, st>>>(partial, nb, inv3p, w_l1, 0.0f, 0, loss);
  }
  return hipGetLastError();
}

}  // namespace gs
