// Forward rasteriser: per 16x16 tile, front-to-back alpha compositing of
// the tile's depth-sorted Gaussians (the Grendel-GS notes' training
// pipeline: for each pixel, the covering Gaussians sorted by depth are
// alpha-composited).
//
// Waves own 8x8 quarters of a tile (see raster_common.hpp).  Per pixel the
// canonical fp32 rule decides skip / composite / stop, evaluated without
// branches (selects), so the image and every decision are bit-identical to
// the checker's.  A wave ends at the first chunk boundary after all 64 of
// its pixels have stopped.
#include "raster_common.hpp"

namespace gs {
namespace {

__global__ __launch_bounds__(64) void k_fill(uint32_t* __restrict__ p, int n, uint32_t v) {
  const int i = int(blockIdx.x) * 64 + int(threadIdx.x);
  if (i < n) p[i] = v;
}

__global__ __launch_bounds__(64) void k_render_fwd(const float4* __restrict__ proj, const int32_t* __restrict__ vals,
                                                   const uint32_t* __restrict__ ranges,
                                                   const uint32_t* __restrict__ order, int64_t num_pairs, int W,
                                                   int H, int TX, int nT, float* __restrict__ image,
                                                   float* __restrict__ T_final, uint32_t* __restrict__ last,
                                                   uint32_t* __restrict__ tile_processed) {
  __shared__ float4 s_a[kChunk];
  __shared__ float4 s_c[kChunk];
  __shared__ float s_b[kChunk];
  int q0;
  const int tile = order_tile(order, nT, q0);
  if (tile < 0) return;
  const int lane = threadIdx.x;
  const int tx = tile % TX, ty = tile / TX;
  const int x0 = tx * kTile, y0 = ty * kTile;
  const float qx = float(x0 + (q0 & 1) * 8) + 0.5f, qy = float(y0 + (q0 >> 1) * 8) + 0.5f;
  uint32_t start = ranges[2 * tile], end = ranges[2 * tile + 1];
  if (end > uint64_t(num_pairs)) end = uint32_t(num_pairs);
  if (start > end) start = end;

  const int px = x0 + (q0 & 1) * 8 + (lane & 7), py = y0 + (q0 >> 1) * 8 + (lane >> 3);
  const float pxc = float(px) + 0.5f, pyc = float(py) + 0.5f;
  const bool inside = px < W && py < H;
  float T = 1.0f, C0 = 0.0f, C1 = 0.0f, C2 = 0.0f;
  uint32_t lastp = 0, read = end - start;
  bool live = inside;       // still compositing

  const uint32_t ul = uint32_t(lane);
  EntryRec cur = load_entry(proj, load_index(vals, start + ul, start + ul < end));
  int32_t gnext = load_index(vals, start + kChunk + ul, start + kChunk + ul < end);
  for (uint32_t cs = start; cs < end && __any(live); cs += kChunk) {
    const EntryRec nxt = load_entry(proj, gnext);
    const uint32_t j2 = cs + 2 * kChunk + ul;
    gnext = load_index(vals, j2, j2 < end);
    const bool hit = stage_entry(cur, qx, qy, s_a, s_c, s_b, nullptr, lane);
    cur = nxt;
    uint64_t active = __ballot(hit);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint32_t pos0 = cs - start + 1;   // list position + 1 of the chunk's entry 0
    while (active != 0) {
      const int k = __builtin_ctzll(active);
      active &= active - 1;
      const float4 a = s_a[k];
      const float4 c = s_c[k];
      const float dx = pxc - a.x, dy = pyc - a.y;
      const float power = fmaf(dx, fmaf(a.z, dx, a.w * dy), (c.x * dy) * dy);
      // power < -5.6 gives alpha < e^-5.6 < 1/255 for any opacity <= 1
      bool ok = live && !(power > 0.0f) && !(power < -5.6f);
      if (!__any(ok)) continue;
      const float cb = s_b[k];
      const float alpha = fminf(0.99f, c.y * pexp_core(power));
      ok = ok && !(alpha < 1.0f / 255.0f);
      const float nt = T * (1.0f - alpha);
      const bool stop = ok && nt < 0.0001f;
      const bool comp = ok && !stop;
      const uint32_t pos1 = pos0 + uint32_t(k);
      // a zero weight leaves the colour sums exactly as they are
      // (non-negative colours, sums from +0)
      const float wgt = comp ? alpha * T : 0.0f;
      C0 = fmaf(c.z, wgt, C0);
      C1 = fmaf(c.w, wgt, C1);
      C2 = fmaf(cb, wgt, C2);
      T = comp ? nt : T;
      lastp = comp ? pos1 : lastp;
      read = stop ? pos1 : read;
      live = live && !stop;
    }
    __builtin_amdgcn_wave_barrier();
  }

  if (inside) {
    const size_t P = size_t(W) * H;
    const size_t pix = size_t(py) * W + px;
    image[pix] = C0;
    image[P + pix] = C1;
    image[2 * P + pix] = C2;
    T_final[pix] = T;
    last[pix] = lastp;
  }
  if (tile_processed != nullptr) {
    const uint32_t rmax = wave_max_u32(inside ? read : 0u);
    if (lane == 0 && rmax != 0) atomicMax(tile_processed + tile, rmax);
  }
}

}  // namespace

hipError_t launch_render_fwd(const float* proj, const int32_t* vals, const uint32_t* ranges,
                             const uint32_t* tile_order, int64_t num_pairs, int32_t width, int32_t height,
                             float* image, float* T_final, uint32_t* last, uint32_t* tile_processed, hipStream_t st) {
  const int TX = (width + kTile - 1) / kTile, TY = (height + kTile - 1) / kTile;
  const int nT = TX * TY;
  if (tile_processed != nullptr) k_fill<<<unsigned((nT + 63) / 64), 64, 0, st>>>(tile_processed, nT, 0u);
  k_render_fwd<<<raster_grid(nT), 64, 0, st>>>(reinterpret_cast<const float4*>(proj), vals, ranges, tile_order,
                                              num_pairs, width, height, TX, nT, image, T_final, last,
                                              tile_processed);
  return hipGetLastError();
}

}  // namespace gs
