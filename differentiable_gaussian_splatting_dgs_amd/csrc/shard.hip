// One GPU's share of the Grendel-GS split (Grendel-GS notes, "hybrid
// parallel strategy", "sparse all-to-all communication" and "dynamic load
// balancing"): the image's tiles cut into K contiguous runs of tile ids of
// about equal cost, the records of a view's visible Gaussians packed per
// run for the forward all-to-all, and the gradient rows that come back
// added into the Gaussians' rows.
//
// A visible Gaussian goes to block d when its tile rectangle holds a tile
// whose id lies in [bounds[d], bounds[d+1]).  Row-major ids make a block a
// run of whole rows with a partial row at each end, so the test is a few
// comparisons per (Gaussian, block); the candidate blocks are those between
// the blocks of the rectangle's first and last tile.  K <= 64, so a
// Gaussian's blocks form one 64-bit mask and a wave ranks its 64 entries
// per block with one ballot: every block's list comes out in ascending
// Gaussian order with no sort.
#include <algorithm>

#include "gs_internal.h"

namespace gs {
namespace {

constexpr int kSegE = 512;   // visible entries per wave segment of the pack

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
}

// bounds[0] = 0, bounds[K] = T; for 0 < d < K the first t with
// K P(t) >= d total (P = exclusive prefix of the costs).  Tile t is the
// answer for the d in (K P(t-1) / total, K P(t) / total]; the thread that
// owns tile t - 1 writes them.  T <= 2^21 keeps K P below 2^59.
__global__ __launch_bounds__(1024) void k_partition(const uint32_t* __restrict__ cost, int T, int K,
                                                    int32_t* __restrict__ bounds) {
  __shared__ uint64_t s[1024];
  const int t = threadIdx.x;
  const int chunk = (T + 1023) / 1024;
  const int c0 = std::min(T, t * chunk), c1 = std::min(T, c0 + chunk);
  uint64_t sum = 0;
  for (int i = c0; i < c1; i += 8) {
    uint32_t v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = i + q < c1 ? cost[i + q] : 0u;
#pragma unroll
    for (int q = 0; q < 8; ++q) sum += v[q];
  }
  s[t] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const uint64_t add = t >= off ? s[t - off] : 0;
    __syncthreads();
    s[t] += add;
    __syncthreads();
  }
  const uint64_t total = s[1023];
  uint64_t P = s[t] - sum;   // exclusive prefix at c0
  if (t == 0) {
    bounds[0] = 0;
    bounds[K] = T;
  }
  if (total == 0) {
    for (int d = 1 + t; d < K; d += 1024) bounds[d] = 0;
    return;
  }
  const uint64_t k64 = uint64_t(K);
  for (int i0 = c0; i0 < c1; i0 += 8) {
    uint32_t v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = i0 + q < c1 ? cost[i0 + q] : 0u;
    for (int q = 0; q < 8 && i0 + q < c1; ++q) {
      const uint64_t Pn = P + v[q];
      // tile i + 1 answers d in [floor(K P / total) + 1, floor(K Pn / total)]
      const int64_t dlo = int64_t(k64 * P / total) + 1;
      const int64_t dhi = std::min<int64_t>(int64_t(k64 * Pn / total), K - 1);
      for (int64_t d = dlo; d <= dhi; ++d) bounds[d] = i0 + q + 1;
      P = Pn;
    }
  }
}

struct Blocks {
  const int32_t* b;   // K + 1 bounds (LDS)
  int K, TX;
};

// does block d (tiles [b, e)) hold a tile of the rectangle?
__device__ __forceinline__ bool block_meets(int b, int e, int TX, int x0, int y0, int x1, int y1) {
  if (b >= e) return false;
  const int rb = b / TX, re = (e - 1) / TX;
  const int lo = std::max(y0, rb), hi = std::min(y1 - 1, re);
  if (lo > hi) return false;
  if (std::max(lo, rb + 1) <= std::min(hi, re - 1)) return true;   // a whole row of the block
  // the partial rows at the block's two ends
  if (lo == rb) {
    const int cb = b % TX, ce = rb == re ? (e - 1) % TX + 1 : TX;
    if (std::max(cb, x0) < std::min(ce, x1)) return true;
  }
  if (hi == re && re != rb) {
    const int ce = (e - 1) % TX + 1;
    if (x0 < ce) return true;
  }
  return false;
}

// last d with b[d] <= id (d in [0, K - 1])
__device__ __forceinline__ int block_of(const Blocks& B, int id) {
  int lo = 0, hi = B.K - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (B.b[mid] <= id) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ uint64_t block_mask(const Blocks& B, uint32_t w13, uint32_t w14) {
  const int x0 = int(w13 & 0xFFFFu), x1 = int(w13 >> 16), y0 = int(w14 & 0xFFFFu), y1 = int(w14 >> 16);
  if (x0 >= x1 || y0 >= y1) return 0;
  const int d0 = block_of(B, y0 * B.TX + x0), d1 = block_of(B, (y1 - 1) * B.TX + x1 - 1);
  uint64_t m = 0;
  for (int d = d0; d <= d1; ++d)
    if (block_meets(B.b[d], B.b[d + 1], B.TX, x0, y0, x1, y1)) m |= uint64_t(1) << d;
  return m;
}

// Wave w of workgroup g takes segment s = 4 g + w: visible entries
// [s kSegE, (s + 1) kSegE), 64 per round.  Lane d keeps block d's count.
__global__ __launch_bounds__(256) void k_pack_count(const uint32_t* __restrict__ proj, const int32_t* __restrict__ vis,
                                                    const int64_t* __restrict__ vis_count, int64_t n,
                                                    const int32_t* __restrict__ bounds, int K, int TX, int nseg,
                                                    uint32_t* __restrict__ counts) {
  __shared__ int32_t s_b[kMaxTileBlocks + 1];
  for (int d = threadIdx.x; d <= K; d += 256) s_b[d] = bounds[d];
  __syncthreads();
  const Blocks B{s_b, K, TX};
  const int lane = threadIdx.x & 63;
  const int seg = int(blockIdx.x) * 4 + (int(threadIdx.x) >> 6);
  if (seg >= nseg) return;
  int64_t V = vis_count[0];
  V = V < 0 ? 0 : (V > n ? n : V);
  uint32_t cnt = 0;
  for (int r = 0; r < kSegE / 64; ++r) {
    const int64_t k = int64_t(seg) * kSegE + r * 64 + lane;
    uint64_t m = 0;
    if (k < V) {
      const int32_t i = vis[k];
      if (i >= 0 && i < n) m = block_mask(B, proj[size_t(i) * 16 + 13], proj[size_t(i) * 16 + 14]);
    }
    for (int d = 0; d < K; ++d) {
      const uint32_t c = uint32_t(__builtin_popcountll(__builtin_amdgcn_ballot_w64((m >> d) & 1u)));
      cnt += lane == d ? c : 0u;
    }
  }
  if (lane < K) counts[size_t(lane) * nseg + seg] = cnt;
}

// Exclusive scan of counts in (block, segment) order -> 64-bit offsets,
// one workgroup per block d: the counts of blocks before d summed
// (coalesced), then row d scanned.  send_offsets[d] = block d's first
// entry, send_offsets[K] = the total.
__global__ __launch_bounds__(1024) void k_pack_scan(const uint32_t* __restrict__ counts, int K, int nseg,
                                                    int64_t* __restrict__ offs, int64_t* __restrict__ send_offsets) {
  __shared__ int64_t s[1024];
  const int t = threadIdx.x;
  const int d = blockIdx.x;
  int64_t before = 0;
  for (int64_t e = t; e < int64_t(d) * nseg; e += 1024) before += counts[e];
  s[t] = before;
  __syncthreads();
  for (int off = 512; off > 0; off >>= 1) {
    if (t < off) s[t] += s[t + off];
    __syncthreads();
  }
  const int64_t base = s[0];
  __syncthreads();
  const uint32_t* __restrict__ row = counts + size_t(d) * nseg;
  const int chunk = (nseg + 1023) / 1024;
  const int c0 = std::min(nseg, t * chunk), c1 = std::min(nseg, c0 + chunk);
  int64_t sum = 0;
  for (int i = c0; i < c1; ++i) sum += row[i];
  s[t] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int64_t add = t >= off ? s[t - off] : 0;
    __syncthreads();
    s[t] += add;
    __syncthreads();
  }
  int64_t run = base + s[t] - sum;
  for (int i = c0; i < c1; ++i) {
    offs[size_t(d) * nseg + i] = run;
    run += row[i];
  }
  if (t == 0) send_offsets[d] = base;
  if (t == 1023 && d == K - 1) send_offsets[K] = base + s[1023];
}

// The count pass again, now writing: block d's entries of a round go to
// consecutive slots from the segment's offset, in lane (= list) order.
__global__ __launch_bounds__(256) void k_pack_write(const uint32_t* __restrict__ proj, const int32_t* __restrict__ vis,
                                                    const int64_t* __restrict__ vis_count, int64_t n,
                                                    const int32_t* __restrict__ bounds, int K, int TX, int nseg,
                                                    const int64_t* __restrict__ offs, int64_t capacity,
                                                    int32_t* __restrict__ send_idx, float4* __restrict__ send_rec) {
  __shared__ int32_t s_b[kMaxTileBlocks + 1];
  for (int d = threadIdx.x; d <= K; d += 256) s_b[d] = bounds[d];
  __syncthreads();
  const Blocks B{s_b, K, TX};
  const int lane = threadIdx.x & 63;
  const int seg = int(blockIdx.x) * 4 + (int(threadIdx.x) >> 6);
  if (seg >= nseg) return;
  int64_t V = vis_count[0];
  V = V < 0 ? 0 : (V > n ? n : V);
  int64_t next = lane < K ? offs[size_t(lane) * nseg + seg] : 0;   // lane d: block d's next slot
  const float4* __restrict__ rec4 = reinterpret_cast<const float4*>(proj);
  for (int r = 0; r < kSegE / 64; ++r) {
    const int64_t k = int64_t(seg) * kSegE + r * 64 + lane;
    uint64_t m = 0;
    int32_t i = -1;
    if (k < V) {
      i = vis[k];
      if (i >= 0 && i < n) m = block_mask(B, proj[size_t(i) * 16 + 13], proj[size_t(i) * 16 + 14]);
    }
    if (__builtin_amdgcn_ballot_w64(m != 0) == 0) continue;
    float4 q[4];
    if (m != 0 && send_rec != nullptr)
      for (int w = 0; w < 4; ++w) q[w] = rec4[size_t(i) * 4 + w];
    for (int d = 0; d < K; ++d) {
      const bool hit = (m >> d) & 1u;
      const uint64_t bal = __builtin_amdgcn_ballot_w64(hit);
      if (bal == 0) continue;
      const int64_t base = int64_t((uint64_t(__builtin_amdgcn_readlane(uint32_t(uint64_t(next) >> 32), d)) << 32) |
                                   uint64_t(__builtin_amdgcn_readlane(uint32_t(next), d)));
      const int64_t pos = base + lanes_below(bal);
      if (hit && pos < capacity) {
        send_idx[pos] = i;
        if (send_rec != nullptr)
          for (int w = 0; w < 4; ++w) send_rec[size_t(pos) * 4 + w] = q[w];
      }
      if (lane == d) next += __builtin_popcountll(bal);
    }
  }
}

// Block d's rows added into their Gaussians' rows (one launch per block, in
// order; a Gaussian appears once per block).
__global__ __launch_bounds__(256) void k_unpack(const float4* __restrict__ recv, const int64_t* __restrict__ offsets,
                                                const int32_t* __restrict__ idx, int d, int64_t capacity,
                                                int64_t n, float4* __restrict__ grad) {
  int64_t a = offsets[d], b = offsets[d + 1];
  a = std::min(std::max<int64_t>(a, 0), capacity);
  b = std::min(std::max<int64_t>(b, a), capacity);
  for (int64_t j = a + int64_t(blockIdx.x) * 256 + threadIdx.x; j < b; j += int64_t(gridDim.x) * 256) {
    const int32_t i = idx[j];
    if (i < 0 || i >= n) continue;
#pragma unroll
    for (int w = 0; w < 3; ++w) {
      const float4 g = grad[size_t(i) * 3 + w], r = recv[size_t(j) * 3 + w];
      grad[size_t(i) * 3 + w] = make_float4(g.x + r.x, g.y + r.y, g.z + r.z, g.w + r.w);
    }
  }
}

int64_t segments_of(int64_t n) { return (n + kSegE - 1) / kSegE; }

}  // namespace

size_t pack_ws_bytes(int64_t n, int32_t num_blocks) {
  // the launch runs at least one segment
  const size_t E = size_t(std::max<int64_t>(1, segments_of(n))) * size_t(std::max(num_blocks, 0));
  return align_up(sizeof(uint32_t) * E, 256) + align_up(sizeof(int64_t) * E, 256);
}

hipError_t launch_tile_partition(const uint32_t* cost, int32_t T, int32_t K, int32_t* bounds, hipStream_t st) {
  k_partition<<<1, 1024, 0, st>>>(cost, T, K, bounds);
  return hipGetLastError();
}

hipError_t launch_pack_records(const float* proj, int64_t n, const int32_t* vis_idx, const int64_t* vis_count,
                               int32_t tiles_x, const int32_t* bounds, int32_t K, int64_t capacity,
                               int64_t* send_offsets, int32_t* send_idx, float* send_rec, void* ws,
                               hipStream_t st) {
  const int64_t nseg = std::max<int64_t>(1, segments_of(n));
  const size_t E = size_t(nseg) * size_t(K);
  uint32_t* counts = static_cast<uint32_t*>(ws);
  int64_t* offs = reinterpret_cast<int64_t*>(static_cast<char*>(ws) + align_up(sizeof(uint32_t) * E, 256));
  const unsigned grid = unsigned((nseg + 3) / 4);
  const uint32_t* p32 = reinterpret_cast<const uint32_t*>(proj);
  k_pack_count<<<grid, 256, 0, st>>>(p32, vis_idx, vis_count, n, bounds, K, tiles_x, int(nseg), counts);
  k_pack_scan<<<unsigned(K), 1024, 0, st>>>(counts, K, int(nseg), offs, send_offsets);
  k_pack_write<<<grid, 256, 0, st>>>(p32, vis_idx, vis_count, n, bounds, K, tiles_x, int(nseg), offs, capacity,
                                     send_idx, reinterpret_cast<float4*>(send_rec));
  return hipGetLastError();
}

hipError_t launch_unpack_grads(const float* recv, const int64_t* send_offsets, const int32_t* send_idx, int32_t K,
                               int64_t capacity, float* grad2d, int64_t n, hipStream_t st) {
  const unsigned grid = unsigned(std::max<int64_t>(1, std::min<int64_t>((capacity + 255) / 256, 2048)));
  for (int d = 0; d < K; ++d)
    k_unpack<<<grid, 256, 0, st>>>(reinterpret_cast<const float4*>(recv), send_offsets, send_idx, d, capacity, n,
                                   reinterpret_cast<float4*>(grad2d));
  return hipGetLastError();
}

}  // namespace gs
