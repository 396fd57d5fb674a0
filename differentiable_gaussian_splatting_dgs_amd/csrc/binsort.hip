// Binning of Gaussian-tile pairs and their depth order (the Grendel-GS
// notes' training pipeline: for each pixel find the covering Gaussians and
// sort them by depth), then the range-extraction stage the Odin summary page
// lists first in its stage task graph.
//
// The sort order is the one of the keys (tile_id << 32 | bits(depth)) with
// ties in ascending Gaussian index.  It is produced in steps that give
// exactly that order with far less traffic than a 45-bit radix sort of
// all pairs:
//   1. the visible list (ascending indices) is radix-sorted stably by the
//      32 depth bits -- V elements, not M;
//   2. per block of depth ranks, its pairs in each tile column come from
//      the Gaussians' tile rectangles (a difference array over columns);
//   3. pairs are generated in depth order and written straight to their
//      place in tile-column order (column start + earlier blocks + stable
//      rank in the block), packed as row << 56 | index << 32 | depth bits;
//   4. a stable pass on the row writes the final (key, value), the column
//      coming from the pair's position (the column groups of step 3).
//   Column then row is tile-id order, and every placement keeps the depth
//   order (and the index order of equal depths) inside each tile.  Images
//   over 256 tiles wide or tall, or 2^24 or more Gaussians, use plain
//   stable LSD passes on 8-bit digits of the 64-bit keys instead.
// Radix passes are reduce-then-scan: per-block digit histograms, a scan of
// each digit row, then a scatter whose in-block rank comes from wave64
// ballot matching (8 ballots per digit) and per-wave running counts in LDS.
// No workgroup ever waits on another.
#include <algorithm>

#include "gs_scan.hpp"

namespace gs {
namespace {

constexpr int kRT = 256;                 // radix threads per block
constexpr int kRI = 16;                  // items per thread
constexpr int kRB = kRT * kRI;           // items per block
constexpr int kWaves = kRT / 64;
constexpr int kWaveItems = kRI * 64;

__device__ __forceinline__ uint32_t digit_of(uint16_t k, int shift) { return (uint32_t(k) >> shift) & 0xFFu; }
__device__ __forceinline__ uint32_t digit_of(uint32_t k, int shift) { return (k >> shift) & 0xFFu; }
__device__ __forceinline__ uint32_t digit_of(uint64_t k, int shift) { return uint32_t(k >> shift) & 0xFFu; }

__device__ __forceinline__ int64_t count_of(const int64_t* dev, int64_t host) {
  return dev != nullptr ? *dev : host;
}

// ---------------------------------------------------------------------------
// radix pass pieces
// ---------------------------------------------------------------------------
template <class K>
__global__ __launch_bounds__(kRT) void k_upsweep(const K* __restrict__ keys, const int64_t* count_dev,
                                                 int64_t count_host, int shift, uint32_t* __restrict__ H,
                                                 int nb) {
  __shared__ uint32_t hist[256];
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  hist[t] = 0;
  __syncthreads();
  const int64_t count = count_of(count_dev, count_host);
  const int64_t base = int64_t(blockIdx.x) * kRB + int64_t(w) * kWaveItems;
  // all loads first, so they are in flight together
  uint32_t dg[kRI];
#pragma unroll
  for (int it = 0; it < kRI; ++it) {
    const int64_t idx = base + it * 64 + lane;
    dg[it] = idx < count ? digit_of(keys[idx], shift) : 0u;
  }
#pragma unroll
  for (int it = 0; it < kRI; ++it) {
    if (base + it * 64 + lane < count) atomicAdd(&hist[dg[it]], 1u);
  }
  __syncthreads();
  H[size_t(t) * nb + blockIdx.x] = hist[t];
}

// grid = 256 blocks, one per digit: exclusive scan of H[d][0..nb) in place,
// row total to rowtot[d].
__global__ __launch_bounds__(kRT) void k_rowscan(uint32_t* __restrict__ H, int nb, uint32_t* __restrict__ rowtot) {
  __shared__ uint32_t sh[kRT / 64];
  uint32_t* row = H + size_t(blockIdx.x) * nb;
  uint32_t carry = 0;
  for (int base = 0; base < nb; base += kRT) {
    const int i = base + int(threadIdx.x);
    const uint32_t v = i < nb ? row[i] : 0u;
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan<kRT, uint32_t>(v, sh, tot);
    if (i < nb) row[i] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) rowtot[blockIdx.x] = carry;
}

struct RankSmem {
  uint32_t w[kWaves][256];     // per-wave running counts, then per-wave offsets
  uint32_t dstart[256];        // block-local start of each digit
  uint32_t dcnt[256];          // items of each digit in the chunk
  uint32_t gbase[256];         // global destination of each digit's first item
  uint32_t sc[kRT / 64];
};

// Stable ranking of one chunk of NI * 256 items by their 8-bit digit (256
// threads).  Item `it` of thread (wave w, lane l) is the chunk's item
// w * NI * 64 + it * 64 + l; absent items have valid[it] = false and sort
// after all present ones.  On return pos[it] is the item's place in the
// chunk's digit-sorted order, sm.dstart[d] / sm.dcnt[d] each digit's local
// start and count.  Ends with a barrier.
template <int NI>
__device__ __forceinline__ void rank_chunk(const uint32_t (&d)[NI], const bool (&valid)[NI], RankSmem& sm,
                                           uint32_t (&pos)[NI]) {
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) sm.w[k][t] = 0;
  __syncthreads();
  uint32_t rk[NI];
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const uint64_t act = ballot(valid[it]);
    const uint64_t peers = match_bits<8>(d[it], act);
    const uint32_t below = uint32_t(count_below(peers));
    const uint32_t prior = sm.w[w][d[it]];
    rk[it] = prior + below;
    __builtin_amdgcn_wave_barrier();
    if (valid[it] && below == 0) sm.w[w][d[it]] = prior + uint32_t(__popcll(peers));
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  // digit t: per-wave counts -> block-local offsets
  uint32_t c[kWaves], tot = 0;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) {
    c[k] = sm.w[k][t];
    tot += c[k];
  }
  uint32_t btot;
  const uint32_t ex = block_exclusive_scan<kRT, uint32_t>(tot, sm.sc, btot);
  sm.dstart[t] = ex;
  sm.dcnt[t] = tot;
  uint32_t run = ex;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) {
    sm.w[k][t] = run;
    run += c[k];
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < NI; ++it) pos[it] = sm.w[w][d[it]] + rk[it];
  __syncthreads();
}

// One radix block (kRI items per thread, input index base + it * 64 + lane
// for this thread, absent past `count`): rank_chunk plus each digit's
// global destination from the scanned histograms H / rowtot.
__device__ __forceinline__ void rank_block(const uint32_t (&d)[kRI], int64_t base, int64_t count,
                                           const uint32_t* __restrict__ H, const uint32_t* __restrict__ rowtot,
                                           int nb, RankSmem& sm, uint32_t (&pos)[kRI]) {
  const int t = threadIdx.x, lane = t & 63;
  bool valid[kRI];
#pragma unroll
  for (int it = 0; it < kRI; ++it) valid[it] = base + it * 64 + lane < count;
  rank_chunk<kRI>(d, valid, sm, pos);
  uint32_t rtot;
  const uint32_t rex = block_exclusive_scan<kRT, uint32_t>(rowtot[t], sm.sc, rtot);
  sm.gbase[t] = rex + H[size_t(t) * nb + blockIdx.x];
  __syncthreads();
}

// Plain stable pass: (key, value) -> (key, value) ordered by the digit at
// `shift`.
template <class K>
__global__ __launch_bounds__(kRT) void k_scatter(const K* __restrict__ kin, const uint32_t* __restrict__ vin,
                                                 K* __restrict__ kout, uint32_t* __restrict__ vout,
                                                 const int64_t* count_dev, int64_t count_host, int shift,
                                                 const uint32_t* __restrict__ H,
                                                 const uint32_t* __restrict__ rowtot, int nb) {
  __shared__ RankSmem sm;
  __shared__ K s_key[kRB];
  __shared__ uint32_t s_val[kRB];
  const int64_t count = count_of(count_dev, count_host);
  const int64_t bbase = int64_t(blockIdx.x) * kRB;
  if (bbase >= count) return;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  K key[kRI];
  uint32_t val[kRI], d[kRI], pos[kRI];
  const int64_t base = bbase + int64_t(w) * kWaveItems;
  // all loads first, so they are in flight together
#pragma unroll
  for (int it = 0; it < kRI; ++it) {
    const int64_t idx = base + it * 64 + lane;
    const bool valid = idx < count;
    key[it] = valid ? kin[idx] : K(0);
    val[it] = valid ? vin[idx] : 0u;
  }
#pragma unroll
  for (int it = 0; it < kRI; ++it) d[it] = digit_of(key[it], shift);
  rank_block(d, base, count, H, rowtot, nb, sm, pos);
#pragma unroll
  for (int it = 0; it < kRI; ++it) {
    if (base + it * 64 + lane < count) {
      s_key[pos[it]] = key[it];
      s_val[pos[it]] = val[it];
    }
  }
  __syncthreads();
  const int nvalid = int(count - bbase < kRB ? count - bbase : kRB);
  for (int j = t; j < nvalid; j += kRT) {
    const K k = s_key[j];
    const uint32_t dg = digit_of(k, shift);
    const uint32_t g = sm.gbase[dg] + (uint32_t(j) - sm.dstart[dg]);
    kout[g] = k;
    vout[g] = s_val[j];
  }
}

// Row pass: row << 56 | index << 32 | depth bits, grouped by column (group
// c starts at the exclusive scan of the column pass's digit totals
// col_tot), -> final (tile << 32 | depth bits, Gaussian index) ordered by
// row.  Each run of one tile in the block's sorted items also extends the
// tile's range ([min start, max end) by atomics on a range array holding
// (UINT_MAX, 0) beforehand).
__global__ __launch_bounds__(kRT) void k_scatter_row(const uint64_t* __restrict__ pin, const int64_t* count_dev,
                                                     int64_t count_host, const uint32_t* __restrict__ H,
                                                     const uint32_t* __restrict__ rowtot, int nb,
                                                     const uint32_t* __restrict__ col_tot, int32_t tiles_x,
                                                     uint64_t* __restrict__ keys, uint32_t* __restrict__ vals,
                                                     uint32_t* __restrict__ ranges) {
  __shared__ RankSmem sm;
  __shared__ uint32_t s_col[256];
  __shared__ uint64_t s_p[kRB];
  __shared__ uint8_t s_c[kRB];
  const int64_t count = count_of(count_dev, count_host);
  const int64_t bbase = int64_t(blockIdx.x) * kRB;
  if (bbase >= count) return;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  {
    uint32_t tot;
    s_col[t] = block_exclusive_scan<kRT, uint32_t>(t < tiles_x ? col_tot[t] : 0u, sm.sc, tot);
  }
  __syncthreads();
  uint64_t p[kRI];
  uint32_t d[kRI], pos[kRI], cc[kRI];
  const int64_t base = bbase + int64_t(w) * kWaveItems;
#pragma unroll
  for (int it = 0; it < kRI; ++it) {
    const int64_t idx = base + it * 64 + lane;
    p[it] = idx < count ? pin[idx] : 0ull;
    d[it] = uint32_t(p[it] >> 56);
  }
  // column group of each item: the last c with s_col[c] <= idx (empty
  // groups share their start with the next one, so the last such c is
  // non-empty).  A thread's indices increase with `it`: one search for the
  // first, a forward walk for the rest.
  {
    int c = 0;
#pragma unroll
    for (int step = 128; step >= 1; step >>= 1) c = int64_t(s_col[c + step]) <= base + lane ? c + step : c;
#pragma unroll
    for (int it = 0; it < kRI; ++it) {
      const int64_t idx = base + it * 64 + lane;
      while (c < 255 && int64_t(s_col[c + 1]) <= idx) ++c;
      cc[it] = uint32_t(c);
    }
  }
  rank_block(d, base, count, H, rowtot, nb, sm, pos);
#pragma unroll
  for (int it = 0; it < kRI; ++it) {
    if (base + it * 64 + lane < count) {
      s_p[pos[it]] = p[it];
      s_c[pos[it]] = uint8_t(cc[it]);
    }
  }
  __syncthreads();
  const int nvalid = int(count - bbase < kRB ? count - bbase : kRB);
  auto tile_at = [&](int j) { return uint32_t(s_p[j] >> 56) * uint32_t(tiles_x) + s_c[j]; };
  for (int j = t; j < nvalid; j += kRT) {
    const uint64_t pj = s_p[j];
    const uint32_t row = uint32_t(pj >> 56);
    const uint32_t g = sm.gbase[row] + (uint32_t(j) - sm.dstart[row]);
    const uint32_t tile = row * uint32_t(tiles_x) + s_c[j];
    keys[g] = (uint64_t(tile) << 32) | (pj & 0xFFFFFFFFull);
    vals[g] = uint32_t(pj >> 32) & 0xFFFFFFu;
    if (j == 0 || tile_at(j - 1) != tile) atomicMin(ranges + 2 * size_t(tile), g);
    if (j == nvalid - 1 || tile_at(j + 1) != tile) atomicMax(ranges + 2 * size_t(tile) + 1, g + 1);
  }
}

// Range array before the row pass: (UINT_MAX, 0) per tile.
__global__ __launch_bounds__(256) void k_init_ranges(uint32_t* __restrict__ ranges, int T) {
  const int i = int(blockIdx.x) * 256 + int(threadIdx.x);
  if (i < T) {
    ranges[2 * i] = 0xFFFFFFFFu;
    ranges[2 * i + 1] = 0u;
  }
}

// After it: tiles no pair reached get [0, 0).
__global__ __launch_bounds__(256) void k_fix_ranges(uint32_t* __restrict__ ranges, int T) {
  const int i = int(blockIdx.x) * 256 + int(threadIdx.x);
  if (i < T && ranges[2 * i] == 0xFFFFFFFFu) ranges[2 * i] = 0u;
}

// ---------------------------------------------------------------------------
// pipeline kernels
// ---------------------------------------------------------------------------

// depth keys of the visible list (in ascending index order)
__global__ __launch_bounds__(256) void k_depth_gather(const float4* __restrict__ proj,
                                                      const int32_t* __restrict__ vis,
                                                      const int64_t* __restrict__ vis_count,
                                                      uint32_t* __restrict__ keys, uint32_t* __restrict__ vals) {
  const int64_t r = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (r >= *vis_count) return;
  const int32_t g = vis[r];
  keys[r] = __builtin_bit_cast(uint32_t, proj[4 * int64_t(g) + 3].x);
  vals[r] = uint32_t(g);
}

// Duplication works on blocks of kDB consecutive depth ranks.
constexpr int kDT = 256;                 // threads
constexpr int kDI = 4;                   // Gaussians per thread
constexpr int kDB = kDT * kDI;           // Gaussians per block

// Last i in [0, kDB) with off[i] <= o, for non-decreasing off with off[0] = 0
// (Gaussians without pairs share the next one's offset, so the last such i
// has pairs); fixed depth and branch-free, so several searches overlap.
__device__ __forceinline__ int last_at_or_below(const uint32_t* off, uint32_t o) {
  int lo = 0;
#pragma unroll
  for (int step = kDB / 2; step >= 1; step >>= 1) lo = off[lo + step] <= o ? lo + step : lo;
  return lo;
}

// per-block sums of tiles_touched in depth order
__global__ __launch_bounds__(kDT) void k_tilesum(const float4* __restrict__ proj, const uint32_t* __restrict__ order,
                                                 const int64_t* __restrict__ vis_count,
                                                 int64_t* __restrict__ block_sums) {
  __shared__ int64_t sh[kDT / 64];
  const int64_t V = *vis_count;
  const int64_t start = int64_t(blockIdx.x) * kDB + int64_t(threadIdx.x) * kDI;
  int64_t s = 0;
#pragma unroll
  for (int k = 0; k < kDI; ++k) {
    const int64_t r = start + k;
    if (r < V) s += __builtin_bit_cast(uint32_t, proj[4 * int64_t(order[r]) + 3].w);
  }
  int64_t tot;
  block_exclusive_scan<kDT, int64_t>(s, sh, tot);
  if (threadIdx.x == 0) block_sums[blockIdx.x] = tot;
}

__global__ __launch_bounds__(1024) void k_scan_sums(int64_t* __restrict__ sums, int nb, int64_t* __restrict__ total) {
  __shared__ int64_t sh[16];
  __shared__ int64_t carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < nb; base += 1024) {
    const int i = base + int(threadIdx.x);
    const int64_t v = i < nb ? sums[i] : 0;
    int64_t tot;
    const int64_t ex = block_exclusive_scan<1024, int64_t>(v, sh, tot);
    if (i < nb) sums[i] = carry + ex;
    __syncthreads();
    if (threadIdx.x == 0) carry += tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) *total = carry;
}

// Pairs in depth order: for each visible Gaussian (depth rank r), one pair
// per tile of its rectangle, row-major.  Load-balanced: the block's
// Gaussians and their exclusive pair offsets go to LDS, then the block's
// threads write its output range round-robin (coalesced), each locating
// its Gaussian by binary search over the offsets.
__global__ __launch_bounds__(kDT) void k_duplicate(const float4* __restrict__ proj, const uint32_t* __restrict__ order,
                                                   const int64_t* __restrict__ vis_count,
                                                   const int64_t* __restrict__ block_offsets, int32_t tiles_x,
                                                   const int64_t* __restrict__ m_eff, uint64_t* __restrict__ keys,
                                                   uint32_t* __restrict__ vals) {
  __shared__ int64_t sh[kDT / 64];
  __shared__ uint32_t s_off[kDB];        // exclusive pair offset within the block
  __shared__ uint32_t s_rx[kDB];         // x0 | width << 16
  __shared__ uint32_t s_y0[kDB];
  __shared__ uint32_t s_dep[kDB];
  __shared__ uint32_t s_g[kDB];
  if (m_eff != nullptr && *m_eff == 0) return;        // no pairs, or more than the buffers hold
  const int64_t V = *vis_count;
  const int64_t r0 = int64_t(blockIdx.x) * kDB;
  const int t = threadIdx.x;
  uint32_t cnt[kDI];
  uint32_t s = 0;
#pragma unroll
  for (int k = 0; k < kDI; ++k) {
    const int64_t r = r0 + t * kDI + k;
    cnt[k] = 0;
    if (r < V) {
      const uint32_t g = order[r];
      const float4 q3 = proj[4 * int64_t(g) + 3];
      const uint32_t rx = __builtin_bit_cast(uint32_t, q3.y), ry = __builtin_bit_cast(uint32_t, q3.z);
      const uint32_t x0 = rx & 0xFFFFu, x1 = rx >> 16;
      cnt[k] = __builtin_bit_cast(uint32_t, q3.w);
      s_rx[t * kDI + k] = x0 | ((x1 - x0) << 16);
      s_y0[t * kDI + k] = ry & 0xFFFFu;
      s_dep[t * kDI + k] = __builtin_bit_cast(uint32_t, q3.x);
      s_g[t * kDI + k] = g;
    }
    s += cnt[k];
  }
  int64_t tot;
  uint32_t off = uint32_t(block_exclusive_scan<kDT, int64_t>(int64_t(s), sh, tot));
#pragma unroll
  for (int k = 0; k < kDI; ++k) {
    // absent entries (past the visible count) get an offset no pair reaches
    s_off[t * kDI + k] = r0 + t * kDI + k < V ? off : 0xFFFFFFFFu;
    off += cnt[k];
  }
  __syncthreads();
  const int64_t base = block_offsets[blockIdx.x];
  const int nvalid = int(V - r0 < kDB ? V - r0 : kDB);
  const uint32_t total = uint32_t(tot);
  for (uint32_t o0 = uint32_t(t); o0 < total; o0 += 4 * kDT) {
#pragma unroll
   for (int u = 0; u < 4; ++u) {
    const uint32_t o = o0 + uint32_t(u * kDT);
    if (o >= total) break;
    const int lo = last_at_or_below(s_off, o);
    const uint32_t local = o - s_off[lo];
    const uint32_t rx = s_rx[lo];
    const uint32_t w = rx >> 16;
    const uint32_t ty = s_y0[lo] + local / w, tx = (rx & 0xFFFFu) + local % w;
    keys[base + o] = (uint64_t(ty * uint32_t(tiles_x) + tx) << 32) | s_dep[lo];
    vals[base + o] = s_g[lo];
   }
  }
}

// ---------------------------------------------------------------------------
// exact placement of the pairs (images up to 256 x 256 tiles, < 2^24
// Gaussians): tile-column then tile-row order without histogram passes
// ---------------------------------------------------------------------------
constexpr int kMaxT = 256;               // tile columns / rows this path handles
constexpr int kPI = 4;                   // pairs per thread per chunk of the column placement

// Per block of kDB Gaussians in depth order: its pair total (block_sums)
// and its pairs in each tile column (colcnt[c][b], from a difference array
// over columns: a rectangle adds its row count on [x0, x1)); block 0 also
// clears the total slot colcnt[c][nbv].
__global__ __launch_bounds__(kDT) void k_count_pairs(const float4* __restrict__ proj,
                                                     const uint32_t* __restrict__ order,
                                                     const int64_t* __restrict__ vis_count, int nbv, int tiles_x,
                                                     int64_t* __restrict__ block_sums, uint32_t* __restrict__ colcnt) {
  __shared__ int64_t sh[kDT / 64];
  __shared__ uint32_t s_sc[kDT / 64];
  __shared__ int32_t s_cd[kMaxT + 1];
  const int t = threadIdx.x;
  for (int i = t; i <= kMaxT; i += kDT) s_cd[i] = 0;
  __syncthreads();
  const int64_t V = *vis_count;
  const int64_t r0 = int64_t(blockIdx.x) * kDB;
  int64_t s = 0;
#pragma unroll
  for (int k = 0; k < kDI; ++k) {
    const int64_t r = r0 + t * kDI + k;
    if (r < V) {
      const float4 q3 = proj[4 * int64_t(order[r]) + 3];
      const uint32_t rx = __builtin_bit_cast(uint32_t, q3.y), ry = __builtin_bit_cast(uint32_t, q3.z);
      const int x0 = int(rx & 0xFFFFu), x1 = int(rx >> 16), y0 = int(ry & 0xFFFFu), y1 = int(ry >> 16);
      s += __builtin_bit_cast(uint32_t, q3.w);
      const int h = y1 - y0;
      atomicAdd(&s_cd[x0], h);
      atomicAdd(&s_cd[x1], -h);
    }
  }
  int64_t tot;
  block_exclusive_scan<kDT, int64_t>(s, sh, tot);
  if (t == 0) block_sums[blockIdx.x] = tot;
  // column counts: inclusive prefix of the column differences (mod 2^32)
  const uint32_t v = uint32_t(s_cd[t]);
  uint32_t vt;
  const uint32_t incl = block_exclusive_scan<kDT, uint32_t>(v, s_sc, vt) + v;
  if (t < tiles_x) {
    colcnt[size_t(t) * (nbv + 1) + blockIdx.x] = incl;
    if (blockIdx.x == 0) colcnt[size_t(t) * (nbv + 1) + nbv] = 0u;
  }
}

// Pairs of a block of kDB Gaussians (depth order) straight into tile-column
// order: generated in order (depth rank, rectangle row-major) in chunks of
// kDT * kPI, ranked stably by column, and written at col_start[c] +
// colcnt[c][b] (pairs of c in earlier blocks) + pairs of c in earlier
// chunks + rank, each as row << 56 | Gaussian index << 32 | depth bits.
__global__ __launch_bounds__(kDT) void k_dup_col(const float4* __restrict__ proj, const uint32_t* __restrict__ order,
                                                 const int64_t* __restrict__ vis_count,
                                                 const uint32_t* __restrict__ colcnt,
                                                 const uint32_t* __restrict__ coltot, int nbv, int tiles_x,
                                                 const int64_t* __restrict__ m_eff, uint64_t* __restrict__ out) {
  __shared__ int64_t sh[kDT / 64];
  __shared__ uint32_t s_off[kDB];        // exclusive pair offset within the block
  __shared__ uint32_t s_rx[kDB];         // x0 | width << 16
  __shared__ uint32_t s_y0[kDB];
  __shared__ uint32_t s_g[kDB];
  __shared__ uint32_t s_dep[kDB];
  __shared__ uint32_t s_cb[kMaxT];       // running destination of each column
  __shared__ RankSmem sm;
  __shared__ uint64_t s_p[kDT * kPI];
  __shared__ uint8_t s_d[kDT * kPI];
  if (m_eff != nullptr && *m_eff == 0) return;        // no pairs, or more than the buffers hold
  const int64_t V = *vis_count;
  const int64_t r0 = int64_t(blockIdx.x) * kDB;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  uint32_t cnt[kDI];
  uint32_t s = 0;
#pragma unroll
  for (int k = 0; k < kDI; ++k) {
    const int64_t r = r0 + t * kDI + k;
    cnt[k] = 0;
    if (r < V) {
      const uint32_t g = order[r];
      const float4 q3 = proj[4 * int64_t(g) + 3];
      const uint32_t rx = __builtin_bit_cast(uint32_t, q3.y), ry = __builtin_bit_cast(uint32_t, q3.z);
      const uint32_t x0 = rx & 0xFFFFu, x1 = rx >> 16;
      cnt[k] = __builtin_bit_cast(uint32_t, q3.w);
      s_rx[t * kDI + k] = x0 | ((x1 - x0) << 16);
      s_y0[t * kDI + k] = ry & 0xFFFFu;
      s_dep[t * kDI + k] = __builtin_bit_cast(uint32_t, q3.x);
      s_g[t * kDI + k] = g;
    }
    s += cnt[k];
  }
  int64_t tot;
  uint32_t off = uint32_t(block_exclusive_scan<kDT, int64_t>(int64_t(s), sh, tot));
#pragma unroll
  for (int k = 0; k < kDI; ++k) {
    // absent entries (past the visible count) get an offset no pair reaches
    s_off[t * kDI + k] = r0 + t * kDI + k < V ? off : 0xFFFFFFFFu;
    off += cnt[k];
  }
  {
    uint32_t ct;
    const uint32_t cstart = block_exclusive_scan<kDT, uint32_t>(t < tiles_x ? coltot[t] : 0u, sm.sc, ct);
    s_cb[t] = t < tiles_x ? cstart + colcnt[size_t(t) * (nbv + 1) + blockIdx.x] : 0u;
  }
  __syncthreads();
  const uint32_t total = uint32_t(tot);
  for (uint32_t c0 = 0; c0 < total; c0 += kDT * kPI) {
    uint32_t d[kPI], pos[kPI];
    bool valid[kPI];
    uint64_t pk[kPI];
#pragma unroll
    for (int it = 0; it < kPI; ++it) {
      const uint32_t o = c0 + uint32_t(w * kPI * 64 + it * 64 + lane);
      valid[it] = o < total;
      d[it] = 0;
      pk[it] = 0;
      if (valid[it]) {
        const int lo = last_at_or_below(s_off, o);
        const uint32_t local = o - s_off[lo];
        const uint32_t rx = s_rx[lo];
        const uint32_t wd = rx >> 16;
        const uint32_t ty = s_y0[lo] + local / wd, tx = (rx & 0xFFFFu) + local % wd;
        d[it] = tx;
        pk[it] = (uint64_t(ty) << 56) | (uint64_t(s_g[lo]) << 32) | s_dep[lo];
      }
    }
    rank_chunk<kPI>(d, valid, sm, pos);
#pragma unroll
    for (int it = 0; it < kPI; ++it) {
      if (valid[it]) {
        s_p[pos[it]] = pk[it];
        s_d[pos[it]] = uint8_t(d[it]);
      }
    }
    __syncthreads();
    const int nvalid = int(total - c0 < uint32_t(kDT * kPI) ? total - c0 : uint32_t(kDT * kPI));
    for (int j = t; j < nvalid; j += kDT) {
      const uint32_t dd = s_d[j];
      out[s_cb[dd] + (uint32_t(j) - sm.dstart[dd])] = s_p[j];
    }
    __syncthreads();
    s_cb[t] += sm.dcnt[t];
    __syncthreads();
  }
}

// The pair count the second half of the binning works with: M, or 0 when
// M exceeds the capacity (nothing is then written but empty ranges).
// Also copies M to the caller's device slot m_out (if any).
__global__ __launch_bounds__(64) void k_eff_count(const int64_t* __restrict__ m_dev, int64_t cap,
                                                  int64_t* __restrict__ m_eff, int64_t* __restrict__ m_out) {
  if (threadIdx.x == 0) {
    const int64_t M = *m_dev;
    *m_eff = M <= cap ? M : 0;
    if (m_out != nullptr) *m_out = M;
  }
}

__global__ __launch_bounds__(256) void k_fill_u32(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ __launch_bounds__(256) void k_ranges(const uint64_t* __restrict__ keys, const int64_t* count_dev,
                                                int64_t count_host, uint32_t* __restrict__ ranges) {
  const int64_t M = count_of(count_dev, count_host);
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= M) return;
  const uint32_t t = uint32_t(keys[i] >> 32);
  if (i == 0 || uint32_t(keys[i - 1] >> 32) != t) ranges[2 * size_t(t)] = uint32_t(i);
  if (i == M - 1 || uint32_t(keys[i + 1] >> 32) != t) ranges[2 * size_t(t) + 1] = uint32_t(i + 1);
}

// Launch order of the tiles for the rasterisers: stable counting sort of
// the tiles by descending bucket of their pair count (bucket = bit length
// of the count), so the longest lists start first and short ones fill the
// gaps.  One workgroup; deterministic (wave ballot ranking, no atomics
// whose order matters).
__global__ __launch_bounds__(1024) void k_tile_order(const uint32_t* __restrict__ ranges, int nT,
                                                     uint32_t* __restrict__ order) {
  constexpr int kB = 33;                     // buckets: bit length 0..32
  __shared__ uint32_t s_cnt[kB];
  __shared__ uint32_t s_base[kB];
  __shared__ uint32_t s_w[16][kB];           // per-wave counts of the current round
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  if (t < kB) s_cnt[t] = 0;
  __syncthreads();
  auto bucket_of = [&](int tile) -> uint32_t {       // 0 = longest lists
    const uint32_t len = ranges[2 * tile + 1] - ranges[2 * tile];
    const uint32_t bits = len != 0 ? 32u - uint32_t(__builtin_clz(len)) : 0u;
    return 32u - bits;
  };
  for (int base = 0; base < nT; base += 1024) {
    const int tile = base + t;
    if (tile < nT) atomicAdd(&s_cnt[bucket_of(tile)], 1u);
  }
  __syncthreads();
  if (t == 0) {
    uint32_t run = 0;
    for (int b = 0; b < kB; ++b) {
      s_base[b] = run;
      run += s_cnt[b];
    }
  }
  __syncthreads();
  for (int base = 0; base < nT; base += 1024) {
    const int tile = base + t;
    const bool valid = tile < nT;
    const uint32_t b = valid ? bucket_of(tile) : 0u;
    const uint64_t act = ballot(valid);
    const uint64_t peers = match_bits<6>(b, act);
    const uint32_t below = uint32_t(count_below(peers));
    if (t < 16 * kB) (&s_w[0][0])[t] = 0;
    __syncthreads();
    if (valid && below == 0) s_w[w][b] = uint32_t(__popcll(peers));
    __syncthreads();
    if (valid) {
      uint32_t off = s_base[b] + below;
      for (int k = 0; k < w; ++k) off += s_w[k][b];
      order[off] = uint32_t(tile);
    }
    __syncthreads();
    if (t < kB) {
      uint32_t add = 0;
      for (int k = 0; k < 16; ++k) add += s_w[k][t];
      s_base[t] += add;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// workspace layout
// ---------------------------------------------------------------------------
struct Ws {
  uint32_t *dkA, *dvA, *dkB, *dvB;   // depth sort ping-pong [n]
  uint32_t* H;                       // radix histograms [256][nb]
  uint32_t* rowtot;                  // [256]
  uint32_t* coltot;                  // [256], pairs per tile column
  int64_t* bsums;                    // per-block tile sums [nbv + 1]
  int64_t* m_dev;                    // pair count
  int64_t* m_eff;                    // pair count if within capacity, else 0
  uint32_t* colcnt;                  // [kMaxT][nbv + 1], pairs per (column, block), then scanned
  uint64_t* pk;                      // pair keys scratch [cap]
  uint32_t* pv;                      // pair values scratch [cap]
};

inline int64_t nblocks(int64_t count) { return (count + kRB - 1) / kRB; }
inline int64_t dup_blocks(int64_t n) { return (n + kDB - 1) / kDB; }

// Workspace layout; with ws == nullptr only the size is computed.
Ws carve(void* ws, int64_t n, int64_t cap, size_t* bytes = nullptr) {
  Ws w;
  char* base = static_cast<char*>(ws);
  size_t at = 0;
  auto take = [&](size_t b) { char* q = base != nullptr ? base + at : nullptr; at += align_up(b, 256); return q; };
  const int64_t nbh = std::max<int64_t>(1, std::max(nblocks(n), nblocks(cap)));
  const int64_t nbv = dup_blocks(n);
  w.dkA = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * size_t(n)));
  w.dvA = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * size_t(n)));
  w.dkB = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * size_t(n)));
  w.dvB = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * size_t(n)));
  w.H = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * 256 * size_t(nbh)));
  w.rowtot = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * 256));
  w.coltot = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * 256));
  w.bsums = reinterpret_cast<int64_t*>(take(sizeof(int64_t) * size_t(nbv + 1)));
  w.m_dev = reinterpret_cast<int64_t*>(take(sizeof(int64_t)));
  w.m_eff = reinterpret_cast<int64_t*>(take(sizeof(int64_t)));
  w.colcnt = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * kMaxT * size_t(nbv + 1)));
  w.pk = reinterpret_cast<uint64_t*>(take(sizeof(uint64_t) * size_t(cap)));
  w.pv = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * size_t(cap)));
  if (bytes != nullptr) *bytes = at;
  return w;
}

size_t carve_bytes(int64_t n, int64_t cap) {
  size_t b = 0;
  carve(nullptr, n, cap, &b);
  return b;
}

// The exact-placement path: column and row fit a byte, Gaussian indices 24 bits.
inline bool exact_path(int64_t n, int32_t tiles_x, int32_t tiles_y) {
  return tiles_x <= kMaxT && tiles_y <= kMaxT && n < (int64_t(1) << 24);
}

template <class K>
void radix_pass(const K* kin, const uint32_t* vin, K* kout, uint32_t* vout, const int64_t* count_dev,
                int64_t count_host, int64_t count_bound, int shift, const Ws& w, hipStream_t st) {
  const int nb = int(std::max<int64_t>(1, nblocks(count_bound)));
  k_upsweep<K><<<nb, kRT, 0, st>>>(kin, count_dev, count_host, shift, w.H, nb);
  k_rowscan<<<256, kRT, 0, st>>>(w.H, nb, w.rowtot);
  k_scatter<K><<<nb, kRT, 0, st>>>(kin, vin, kout, vout, count_dev, count_host, shift, w.H, w.rowtot, nb);
}

}  // namespace

size_t binsort_ws_bytes(int64_t n, int64_t pair_capacity) { return carve_bytes(n, pair_capacity); }

int64_t* binsort_count_ptr(void* ws, int64_t n, int64_t pair_capacity) {
  return carve(ws, n, pair_capacity).m_dev;
}

hipError_t launch_binsort_stage1(const float* proj, int64_t n, const int32_t* vis_idx,
                                 const int64_t* vis_count, int32_t tiles_x, int32_t tiles_y, void* ws,
                                 int64_t pair_capacity, hipStream_t st) {
  Ws w = carve(ws, n, pair_capacity);
  int64_t* m_dev = w.m_dev;
  const float4* P = reinterpret_cast<const float4*>(proj);
  if (n > 0) {
    k_depth_gather<<<unsigned((n + 255) / 256), 256, 0, st>>>(P, vis_idx, vis_count, w.dkA, w.dvA);
    // stable LSD radix on the 32 depth bits: A -> B -> A -> B -> A
    for (int pass = 0; pass < 4; ++pass) {
      const bool even = (pass & 1) == 0;
      radix_pass<uint32_t>(even ? w.dkA : w.dkB, even ? w.dvA : w.dvB, even ? w.dkB : w.dkA,
                           even ? w.dvB : w.dvA, vis_count, 0, n, 8 * pass, w, st);
    }
  }
  const int nbv = int(dup_blocks(n));
  if (nbv > 0 && exact_path(n, tiles_x, tiles_y)) {
    // pair totals and per-(column, block) counts
    k_count_pairs<<<nbv, kDT, 0, st>>>(P, w.dvA, vis_count, nbv, tiles_x, w.bsums, w.colcnt);
    k_rowscan<<<unsigned(tiles_x), kRT, 0, st>>>(w.colcnt, nbv + 1, w.coltot);
  } else if (nbv > 0) {
    k_tilesum<<<nbv, kDT, 0, st>>>(P, w.dvA, vis_count, w.bsums);
  }
  k_scan_sums<<<1, 1024, 0, st>>>(w.bsums, nbv, m_dev);
  return hipGetLastError();
}

// Second half.  M_host >= 0: the pair count read by the caller (<= the
// capacity).  M_host < 0: the count stays on the device (nothing blocks);
// grids are sized for the capacity and every kernel reads the effective
// count (0 when M exceeds the capacity: then only empty ranges are written).
hipError_t launch_binsort_stage2(const float* proj, int64_t n, const int32_t* vis_idx,
                                 const int64_t* vis_count, int64_t M_host, int32_t tiles_x, int32_t tiles_y,
                                 uint64_t* keys, int32_t* vals, uint32_t* ranges, uint32_t* tile_order,
                                 int64_t* num_pairs_dev, void* ws, int64_t pair_capacity, hipStream_t st) {
  (void)vis_idx;
  Ws w = carve(ws, n, pair_capacity);
  const float4* P = reinterpret_cast<const float4*>(proj);
  const int64_t T = int64_t(tiles_x) * tiles_y;
  uint32_t* uvals = reinterpret_cast<uint32_t*>(vals);
  const int nbv = int(dup_blocks(n));
  const bool on_device = M_host < 0;
  const int64_t* m_dev = nullptr;
  int64_t bound = M_host;                       // upper bound of the count, for grid sizes
  if (on_device) {
    k_eff_count<<<1, 64, 0, st>>>(w.m_dev, pair_capacity, w.m_eff, num_pairs_dev);
    m_dev = w.m_eff;
    bound = pair_capacity;
  }
  if (!on_device && M_host == 0) {
    k_fill_u32<<<unsigned((2 * T + 255) / 256), 256, 0, st>>>(ranges, 2 * T, 0u);
  } else if (exact_path(n, tiles_x, tiles_y)) {
    // pairs straight into tile-column order, then a stable pass on the row
    const int nb = int(std::max<int64_t>(1, nblocks(bound)));
    if (nbv > 0) k_dup_col<<<nbv, kDT, 0, st>>>(P, w.dvA, vis_count, w.colcnt, w.coltot, nbv, tiles_x, m_dev, w.pk);
    k_upsweep<uint64_t><<<nb, kRT, 0, st>>>(w.pk, m_dev, M_host, 56, w.H, nb);
    k_rowscan<<<256, kRT, 0, st>>>(w.H, nb, w.rowtot);
    k_init_ranges<<<unsigned((T + 255) / 256), 256, 0, st>>>(ranges, int(T));
    k_scatter_row<<<nb, kRT, 0, st>>>(w.pk, m_dev, M_host, w.H, w.rowtot, nb, w.coltot, tiles_x, keys, uvals,
                                      ranges);
    k_fix_ranges<<<unsigned((T + 255) / 256), 256, 0, st>>>(ranges, int(T));
  } else {
    // number of 8-bit passes over the tile bits
    int tbits = 0;
    while ((int64_t(1) << tbits) < T) ++tbits;
    const int passes = std::max(1, (tbits + 7) / 8);
    // duplicate into the buffer that makes the last pass land in (keys, vals)
    uint64_t* bufk[2] = {keys, w.pk};
    uint32_t* bufv[2] = {uvals, w.pv};
    int cur = (passes & 1) ? 1 : 0;
    if (nbv > 0)
      k_duplicate<<<nbv, kDT, 0, st>>>(P, w.dvA, vis_count, w.bsums, tiles_x, m_dev, bufk[cur], bufv[cur]);
    for (int pass = 0; pass < passes; ++pass) {
      radix_pass<uint64_t>(bufk[cur], bufv[cur], bufk[cur ^ 1], bufv[cur ^ 1], m_dev, M_host, bound,
                           32 + 8 * pass, w, st);
      cur ^= 1;
    }
    k_fill_u32<<<unsigned((2 * T + 255) / 256), 256, 0, st>>>(ranges, 2 * T, 0u);
    k_ranges<<<unsigned((std::max<int64_t>(bound, 1) + 255) / 256), 256, 0, st>>>(keys, m_dev, M_host, ranges);
  }
  if (tile_order != nullptr) k_tile_order<<<1, 1024, 0, st>>>(ranges, int(T), tile_order);
  return hipGetLastError();
}

}  // namespace gs
