// Forward rasteriser: per 16x16 tile, front-to-back alpha compositing of
// the tile's depth-sorted Gaussians (the Grendel-GS notes' training
// pipeline: for each pixel, the covering Gaussians sorted by depth are
// alpha-composited).
//
// Waves own 8x8 quarters of a tile (see raster_common.hpp).  Per pixel the
// canonical fp32 rule decides skip / composite / stop, evaluated without
// branches (selects), so the image and every decision are bit-identical to
// the checker's.  A quarter whose 64 pixels have all stopped drops out of
// the masks; the wave ends when all of its quarters have.
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
  const float bx0 = float(x0) + 0.5f, by0 = float(y0) + 0.5f;
  uint32_t start = ranges[2 * tile], end = ranges[2 * tile + 1];
  if (end > uint64_t(num_pairs)) end = uint32_t(num_pairs);
  if (start > end) start = end;

  float pxc[kQPW], pyc[kQPW], T[kQPW], C0[kQPW], C1[kQPW], C2[kQPW];
  uint32_t lastp[kQPW], read[kQPW];
  bool done[kQPW], inside[kQPW];
  int qi[kQPW], pxi[kQPW], pyi[kQPW];
  uint32_t qlive = 0;       // wave-uniform: quarters with a pixel still compositing
#pragma unroll
  for (int i = 0; i < kQPW; ++i) {
    qi[i] = q0 + i;
    pxi[i] = x0 + (qi[i] & 1) * 8 + (lane & 7);
    pyi[i] = y0 + (qi[i] >> 1) * 8 + (lane >> 3);
    pxc[i] = float(pxi[i]) + 0.5f;
    pyc[i] = float(pyi[i]) + 0.5f;
    inside[i] = pxi[i] < W && pyi[i] < H;
    done[i] = !inside[i];
    T[i] = 1.0f;
    C0[i] = C1[i] = C2[i] = 0.0f;
    lastp[i] = 0;
    read[i] = end - start;
    qlive |= (__ballot(!done[i]) != 0 ? 1u : 0u) << i;
  }

  const uint32_t ul = uint32_t(lane);
  EntryRec cur = load_entry(proj, load_index(vals, start + ul, start + ul < end));
  int32_t gnext = load_index(vals, start + kChunk + ul, start + kChunk + ul < end);
  for (uint32_t cs = start; cs < end && qlive != 0; cs += kChunk) {
    const EntryRec nxt = load_entry(proj, gnext);
    const uint32_t j2 = cs + 2 * kChunk + ul;
    gnext = load_index(vals, j2, j2 < end);
    const uint32_t mq = stage_entry(cur, bx0, by0, s_a, s_c, s_b, nullptr, lane);
    cur = nxt;
    uint64_t m[kQPW];
    uint64_t active = 0;
#pragma unroll
    for (int i = 0; i < kQPW; ++i) {
      m[i] = ((qlive >> i) & 1u) ? uint64_t(__ballot((mq >> qi[i]) & 1u)) : 0ull;
      active |= m[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    while (active != 0) {
      const int k = __builtin_ctzll(active);
      active &= active - 1;
      const float4 a = s_a[k];
      const float4 c = s_c[k];
      const float cb = s_b[k];
      const uint32_t pos1 = cs + uint32_t(k) - start + 1;   // list position + 1
      bool stopped = false;
#pragma unroll
      for (int i = 0; i < kQPW; ++i) {
        if (!((m[i] >> k) & 1ull)) continue;
        const float dx = pxc[i] - a.x, dy = pyc[i] - a.y;
        const float power = fmaf(dx, fmaf(a.z, dx, a.w * dy), (c.x * dy) * dy);
        // power < -5.6 gives alpha < e^-5.6 < 1/255 for any opacity <= 1
        bool ok = !done[i] && !(power > 0.0f) && !(power < -5.6f);
        if (!__any(ok)) continue;
        const float alpha = fminf(0.99f, c.y * pexp_core(power));
        ok = ok && !(alpha < 1.0f / 255.0f);
        const float nt = T[i] * (1.0f - alpha);
        const bool stop = ok && nt < 0.0001f;
        const bool comp = ok && !stop;
        const float wgt = alpha * T[i];
        C0[i] = comp ? fmaf(c.z, wgt, C0[i]) : C0[i];
        C1[i] = comp ? fmaf(c.w, wgt, C1[i]) : C1[i];
        C2[i] = comp ? fmaf(cb, wgt, C2[i]) : C2[i];
        T[i] = comp ? nt : T[i];
        lastp[i] = comp ? pos1 : lastp[i];
        read[i] = stop ? pos1 : read[i];
        done[i] = done[i] || stop;
        stopped = stopped || stop;
      }
      if (__any(stopped)) {
        uint32_t ql = 0;
#pragma unroll
        for (int i = 0; i < kQPW; ++i) ql |= (__ballot(!done[i]) != 0 ? 1u : 0u) << i;
        if (ql != qlive) {
          qlive = ql;
          uint64_t keep = 0;
#pragma unroll
          for (int i = 0; i < kQPW; ++i) {
            if (!((qlive >> i) & 1u)) m[i] = 0;
            keep |= m[i];
          }
          active &= keep;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  const size_t P = size_t(W) * H;
  uint32_t rmax = 0;
#pragma unroll
  for (int i = 0; i < kQPW; ++i) {
    if (!inside[i]) continue;
    const size_t pix = size_t(pyi[i]) * W + pxi[i];
    image[pix] = C0[i];
    image[P + pix] = C1[i];
    image[2 * P + pix] = C2[i];
    T_final[pix] = T[i];
    last[pix] = lastp[i];
    rmax = read[i] > rmax ? read[i] : rmax;
  }
  if (tile_processed != nullptr) {
    rmax = wave_max_u32(rmax);
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
