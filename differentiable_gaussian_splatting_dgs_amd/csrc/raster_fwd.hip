// Forward rasteriser: per 16x16 tile, front-to-back alpha compositing of
// the tile's depth-sorted Gaussians (the Grendel-GS notes' training
// pipeline: for each pixel, the covering Gaussians sorted by depth are
// alpha-composited).
//
// One workgroup per tile, 256 threads = 4 waves, each wave an 8x8 pixel
// block.  The tile's list is staged through LDS in batches of 256 records
// (one gather per thread).  Per (wave, Gaussian) a wave-uniform test
// against the Gaussian's alpha >= 1/255 footprint box skips blocks the
// Gaussian cannot reach; per pixel the canonical fp32 rule decides skip /
// composite / stop, so the image is bit-identical to the checker's.  A
// wave stops scanning when all its pixels have stopped, the workgroup when
// all 256 have.
#include "gs_device.hpp"

namespace gs {
namespace {

__global__ __launch_bounds__(kBlock) void k_render_fwd(const float4* __restrict__ proj, const int32_t* __restrict__ vals,
                                                       const uint32_t* __restrict__ ranges, int64_t num_pairs,
                                                       int W, int H, int TX, float* __restrict__ image,
                                                       float* __restrict__ T_final, uint32_t* __restrict__ last,
                                                       uint32_t* __restrict__ tile_processed) {
  __shared__ float4 s_q0[kBlock];   // u, v, -A/2, -B
  __shared__ float4 s_q1[kBlock];   // -C/2, opacity, r, g
  __shared__ float4 s_box[kBlock];  // u - ex, u + ex, v - ey, v + ey
  __shared__ float s_b[kBlock];     // b
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
  float T = 1.0f, C0 = 0.0f, C1 = 0.0f, C2 = 0.0f;
  uint32_t lastp = 0, read = end - start;
  bool done = !inside;
  if (t == 0) s_max = 0;
  for (uint32_t b0 = start; b0 < end; b0 += kBlock) {
    if (__syncthreads_count(done) == kBlock) break;
    const uint32_t j = b0 + t;
    if (j < end) {
      const int64_t g = vals[j];
      const float4 q0 = proj[4 * g], q1 = proj[4 * g + 1], q2 = proj[4 * g + 2];
      s_q0[t] = make_float4(q0.x, q0.y, -0.5f * q0.z, -q0.w);
      s_q1[t] = make_float4(-0.5f * q1.x, q1.y, q1.z, q1.w);
      s_b[t] = q2.x;
      s_box[t] = make_float4(q0.x - q2.y, q0.x + q2.y, q0.y - q2.z, q0.y + q2.z);
    }
    __syncthreads();
    const int cnt = int(min(end - b0, uint32_t(kBlock)));
    for (int k = 0; k < cnt; ++k) {
      if (__all(done)) break;
      const float4 box = s_box[k];
      if (box.y < bx0 || box.x > bx1 || box.w < by0 || box.z > by1) continue;
      if (done) continue;
      const float4 a = s_q0[k];
      const float4 c = s_q1[k];
      const float dx = pxc - a.x, dy = pyc - a.y;
      const float power = fmaf(dx, fmaf(a.z, dx, a.w * dy), (c.x * dy) * dy);
      // power < -5.6 gives alpha < e^-5.6 < 1/255 for any opacity <= 1
      if (power > 0.0f || power < -5.6f) continue;
      const float alpha = fminf(0.99f, c.y * pexp(power));
      if (alpha < 1.0f / 255.0f) continue;
      const float nt = T * (1.0f - alpha);
      if (nt < 0.0001f) {
        done = true;
        read = b0 + uint32_t(k) - start + 1;
        continue;
      }
      const float wgt = alpha * T;
      C0 = fmaf(c.z, wgt, C0);
      C1 = fmaf(c.w, wgt, C1);
      C2 = fmaf(s_b[k], wgt, C2);
      T = nt;
      lastp = b0 + uint32_t(k) - start + 1;
    }
  }
  if (inside) {
    const size_t pix = size_t(py) * W + px;
    const size_t P = size_t(W) * H;
    image[pix] = C0;
    image[P + pix] = C1;
    image[2 * P + pix] = C2;
    T_final[pix] = T;
    last[pix] = lastp;
  }
  if (tile_processed != nullptr) {
    __syncthreads();
    if (inside) atomicMax(&s_max, read);
    __syncthreads();
    if (t == 0) tile_processed[tile] = s_max;
  }
}

}  // namespace

hipError_t launch_render_fwd(const float* proj, const int32_t* vals, const uint32_t* ranges,
                             int64_t num_pairs, int32_t width, int32_t height, float* image,
                             float* T_final, uint32_t* last, uint32_t* tile_processed, hipStream_t st) {
  const int TX = (width + kTile - 1) / kTile, TY = (height + kTile - 1) / kTile;
  k_render_fwd<<<unsigned(TX * TY), kBlock, 0, st>>>(reinterpret_cast<const float4*>(proj), vals, ranges, num_pairs,
                                                     width, height, TX, image, T_final, last, tile_processed);
  return hipGetLastError();
}

}  // namespace gs
