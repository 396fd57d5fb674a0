// Densification (Grendel-GS notes, "training pipeline": clone or split the
// Gaussians whose screen position keeps being pulled, prune the transparent
// ones), on the [59][ld] parameter planes.
//
// The statistic is accumulated per view over the visible rows (fp32, one
// rounding per operation, as the decision depends on it).  The rebuild is
// a three-way stream compaction: every Gaussian is classified (kept,
// cloned, split, each unless pruned), per-block counts are scanned per
// class, and each Gaussian writes its columns -- itself, its clone, its two
// children -- at class base + block offset + rank in the block, so the
// output order (kept, clones, first children, second children; each in
// index order) needs no sort.
#include <algorithm>

#include "gs_internal.h"

namespace gs {
namespace {

constexpr int kDT = 256;   // Gaussians per block of the rebuild

enum : uint8_t { kKeep = 1, kClone = 2, kSplit = 4 };

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
}

__global__ __launch_bounds__(256) void k_dens_stats(const float* __restrict__ grad2d, const int32_t* __restrict__ vis,
                                                    const int64_t* __restrict__ vis_count, int64_t n,
                                                    float* __restrict__ accum, int32_t* __restrict__ denom) {
  int64_t V = vis_count[0];
  V = V < 0 ? 0 : (V > n ? n : V);
  for (int64_t k = int64_t(blockIdx.x) * 256 + threadIdx.x; k < V; k += int64_t(gridDim.x) * 256) {
    const int32_t i = vis[k];
    if (i < 0 || i >= n) continue;
    const float gu = grad2d[size_t(i) * 12], gv = grad2d[size_t(i) * 12 + 1];
    const float uu = gu * gu, vv = gv * gv;
    accum[i] = accum[i] + sqrtf(uu + vv);
    denom[i] = denom[i] + 1;
  }
}

struct DensArgs {
  float grad_threshold, log_scale_threshold, logit_threshold, log_shrink;
};

// class of Gaussian i (0: pruned)
__device__ __forceinline__ uint8_t classify(const float* __restrict__ p, int64_t ld, int64_t i, float acc, int32_t den,
                                            const DensArgs& a) {
  const float g = den > 0 ? acc / float(den) : 0.0f;
  const bool dense = g >= a.grad_threshold;
  const float maxls = fmaxf(fmaxf(p[3 * ld + i], p[4 * ld + i]), p[5 * ld + i]);
  const float s0 = p[3 * ld + i], s1 = p[4 * ld + i], s2 = p[5 * ld + i];
  // the largest log-scale, NaN-propagating like a comparison chain
  const bool any_nan = s0 != s0 || s1 != s1 || s2 != s2;
  const bool small = !any_nan && maxls <= a.log_scale_threshold;
  const bool big = !any_nan && maxls > a.log_scale_threshold;
  const bool low = !(p[10 * ld + i] >= a.logit_threshold);
  if (low) return 0;
  uint8_t c = (dense && big) ? 0 : kKeep;
  if (dense && small) c |= kClone;
  if (dense && big) c |= kSplit;
  return c;
}

// codes and per-block counts of each class (rows: keep, clone, split)
__global__ __launch_bounds__(kDT) void k_dens_classify(const float* __restrict__ p, int64_t n, int64_t ld,
                                                       const float* __restrict__ accum,
                                                       const int32_t* __restrict__ denom, DensArgs a, int nb,
                                                       uint8_t* __restrict__ codes, uint32_t* __restrict__ counts) {
  __shared__ uint32_t s_c[3][kDT / 64];
  const int64_t i = int64_t(blockIdx.x) * kDT + threadIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint8_t c = 0;
  if (i < n) {
    c = classify(p, ld, i, accum[i], denom[i], a);
    codes[i] = c;
  }
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const uint32_t cnt = uint32_t(__builtin_popcountll(__builtin_amdgcn_ballot_w64((c >> k) & 1u)));
    if (lane == 0) s_c[k][wave] = cnt;
  }
  __syncthreads();
  if (threadIdx.x < 3) {
    uint32_t t = 0;
    for (int w = 0; w < kDT / 64; ++w) t += s_c[threadIdx.x][w];
    counts[size_t(threadIdx.x) * nb + blockIdx.x] = t;
  }
}

// one workgroup per class: exclusive scan of its per-block counts, and the
// class total
__global__ __launch_bounds__(1024) void k_dens_scan(const uint32_t* __restrict__ counts, int nb,
                                                    uint32_t* __restrict__ offs, int64_t* __restrict__ totals) {
  __shared__ int64_t s[1024];
  const int t = threadIdx.x, k = blockIdx.x;
  const uint32_t* __restrict__ row = counts + size_t(k) * nb;
  const int chunk = (nb + 1023) / 1024;
  const int c0 = std::min(nb, t * chunk), c1 = std::min(nb, c0 + chunk);
  int64_t sum = 0;
  for (int b = c0; b < c1; ++b) sum += row[b];
  s[t] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int64_t add = t >= off ? s[t - off] : 0;
    __syncthreads();
    s[t] += add;
    __syncthreads();
  }
  int64_t run = s[t] - sum;
  for (int b = c0; b < c1; ++b) {
    offs[size_t(k) * nb + b] = uint32_t(run);
    run += row[b];
  }
  if (t == 1023) totals[k] = s[1023];
}

__device__ __forceinline__ void copy_column(const float* __restrict__ src, int64_t ld, int64_t i,
                                            float* __restrict__ dst, int64_t ld_out, int64_t pos) {
  for (int q = 0; q < 59; ++q) dst[q * ld_out + pos] = src[q * ld + i];
}

__device__ __forceinline__ void zero_column(float* __restrict__ dst, int64_t ld_out, int64_t pos) {
  for (int q = 0; q < 59; ++q) dst[q * ld_out + pos] = 0.0f;
}

__global__ __launch_bounds__(kDT) void k_dens_write(const float* __restrict__ p, const float* __restrict__ m,
                                                    const float* __restrict__ v, int64_t n, int64_t ld,
                                                    const float* __restrict__ normals, DensArgs a,
                                                    const uint8_t* __restrict__ codes, int nb,
                                                    const uint32_t* __restrict__ offs,
                                                    const int64_t* __restrict__ totals, float* __restrict__ op,
                                                    float* __restrict__ om, float* __restrict__ ov, int64_t ld_out,
                                                    int64_t* __restrict__ out_n) {
  __shared__ uint32_t s_w[3][kDT / 64];
  const int64_t i = int64_t(blockIdx.x) * kDT + threadIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint8_t c = i < n ? codes[i] : 0;
  uint32_t rank[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const uint64_t bal = __builtin_amdgcn_ballot_w64((c >> k) & 1u);
    rank[k] = lanes_below(bal);
    if (lane == 0) s_w[k][wave] = uint32_t(__builtin_popcountll(bal));
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 3; ++k)
    for (int w = 0; w < wave; ++w) rank[k] += s_w[k][w];
  const int64_t K = totals[0], C = totals[1], S = totals[2];
  if (blockIdx.x == 0 && threadIdx.x == 0) out_n[0] = K + C + 2 * S;
  if (c == 0) return;
  // the column is read once into registers and written from there to each
  // of its copies (a re-read would come from HBM: the writes of the other
  // copies stream through the cache in between)
  float col[59];
#pragma unroll
  for (int q = 0; q < 59; ++q) col[q] = p[q * ld + i];
  auto put = [&](int64_t pos) {
#pragma unroll
    for (int q = 0; q < 59; ++q) op[q * ld_out + pos] = col[q];
  };
  if (c & kKeep) {
    const int64_t pos = int64_t(offs[blockIdx.x]) + rank[0];
    if (pos < ld_out) {
      put(pos);
      copy_column(m, ld, i, om, ld_out, pos);
      copy_column(v, ld, i, ov, ld_out, pos);
    }
  }
  if (c & kClone) {
    const int64_t pos = K + int64_t(offs[size_t(nb) + blockIdx.x]) + rank[1];
    if (pos < ld_out) {
      put(pos);
      zero_column(om, ld_out, pos);
      zero_column(ov, ld_out, pos);
    }
  }
  if (c & kSplit) {
    const int64_t r = int64_t(offs[size_t(2) * nb + blockIdx.x]) + rank[2];
    // rotation of the normalised quaternion (w, x, y, z)
    const float qw = col[6], qx = col[7], qy = col[8], qz = col[9];
    const float inv = 1.0f / sqrtf(qw * qw + qx * qx + qy * qy + qz * qz);
    const float w = qw * inv, x = qx * inv, y = qy * inv, z = qz * inv;
    const float R[3][3] = {{1.0f - 2.0f * (y * y + z * z), 2.0f * (x * y - w * z), 2.0f * (x * z + w * y)},
                           {2.0f * (x * y + w * z), 1.0f - 2.0f * (x * x + z * z), 2.0f * (y * z - w * x)},
                           {2.0f * (x * z - w * y), 2.0f * (y * z + w * x), 1.0f - 2.0f * (x * x + y * y)}};
    const float sc[3] = {expf(col[3]), expf(col[4]), expf(col[5])};
    const float mu[3] = {col[0], col[1], col[2]}, ls[3] = {col[3], col[4], col[5]};
    for (int ch = 0; ch < 2; ++ch) {
      const int64_t pos = K + C + ch * S + r;
      if (pos >= ld_out) continue;
      float d[3];
      for (int j = 0; j < 3; ++j) d[j] = sc[j] * normals[(size_t(ch) * 3 + j) * size_t(n) + i];
      for (int j = 0; j < 3; ++j) {
        col[j] = mu[j] + (R[j][0] * d[0] + R[j][1] * d[1] + R[j][2] * d[2]);
        col[3 + j] = ls[j] - a.log_shrink;
      }
      put(pos);
      zero_column(om, ld_out, pos);
      zero_column(ov, ld_out, pos);
    }
  }
}

}  // namespace

size_t densify_ws_bytes(int64_t n) {
  const size_t nb = size_t(std::max<int64_t>(1, (n + kDT - 1) / kDT));   // the launch runs at least one block
  return align_up(size_t(n), 256) + 2 * align_up(sizeof(uint32_t) * 3 * nb, 256) + 256;
}

hipError_t launch_densify_stats(const float* grad2d, const int32_t* vis_idx, const int64_t* vis_count, int64_t n,
                                float* accum, int32_t* denom, hipStream_t st) {
  const unsigned grid = unsigned(std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 4096)));
  k_dens_stats<<<grid, 256, 0, st>>>(grad2d, vis_idx, vis_count, n, accum, denom);
  return hipGetLastError();
}

hipError_t launch_densify(const float* params, const float* m, const float* v, int64_t n, int64_t ld,
                          const float* accum, const int32_t* denom, const float* normals, float grad_threshold,
                          float log_scale_threshold, float logit_threshold, float log_shrink, float* out_params,
                          float* out_m, float* out_v, int64_t ld_out, int64_t* out_n, void* ws, hipStream_t st) {
  const int nb = int(std::max<int64_t>(1, (n + kDT - 1) / kDT));
  char* w = static_cast<char*>(ws);
  uint8_t* codes = reinterpret_cast<uint8_t*>(w);
  w += align_up(size_t(n), 256);
  uint32_t* counts = reinterpret_cast<uint32_t*>(w);
  w += align_up(sizeof(uint32_t) * 3 * size_t(nb), 256);
  uint32_t* offs = reinterpret_cast<uint32_t*>(w);
  w += align_up(sizeof(uint32_t) * 3 * size_t(nb), 256);
  int64_t* totals = reinterpret_cast<int64_t*>(w);
  const DensArgs a{grad_threshold, log_scale_threshold, logit_threshold, log_shrink};
  k_dens_classify<<<unsigned(nb), kDT, 0, st>>>(params, n, ld, accum, denom, a, nb, codes, counts);
  k_dens_scan<<<3, 1024, 0, st>>>(counts, nb, offs, totals);
  k_dens_write<<<unsigned(nb), kDT, 0, st>>>(params, m, v, n, ld, normals, a, codes, nb, offs, totals, out_params,
                                             out_m, out_v, ld_out, out_n);
  return hipGetLastError();
}

}  // namespace gs
