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
//      32 depth bits -- V elements, not M.  Each visible Gaussian's compact
//      record (index, tile rectangle, depth: 16 bytes) is gathered once, in
//      ascending index order, and the sort carries its rank in that list;
//      the last pass writes the records themselves in depth order, so the
//      steps below read them contiguously instead of gathering 64-byte
//      projection records at random twice;
//   2. each Gaussian becomes one entry per super-tile (block of 8 x 8 or
//      16 x 16 tiles) its tile rectangle meets, placed stably by super-tile,
//      so every super-tile holds its entries in depth order;
//   3. per chunk of a super-tile's list, each entry's covered tiles as a
//      64-bit mask, transposed across a wave into per-tile bit columns: the
//      pairs of a tile leave in depth order at exact slots (tile starts
//      from per-chunk tile counts scanned in tile-id order).
//   Images over 256 tiles wide or tall use plain stable LSD passes on 8-bit
//   digits of the 64-bit keys instead.
// Radix passes are reduce-then-scan: per-block digit histograms, a scan of
// each digit row, then a scatter whose in-block rank comes from wave64
// ballot matching (8 ballots per digit) and per-wave running counts in LDS.
// No workgroup ever waits on another.
#include <algorithm>

#include "gs_scan.hpp"

namespace gs {
namespace {

// Issue priority of the binning's few-workgroup kernels (scans, the stage
// tail, tile ranges): beside the rasterisers (priority 2) on another stream
// their handful of waves would otherwise wait behind them, and the next
// view's binning, which the caller's stream will wait for, stretches.  Few
// waves: the rasterisers lose little.
constexpr int kFewPrio = 3;

constexpr int kRT = 256;                 // radix threads per block
constexpr int kRI = 8;                   // items per thread (blocks of 2048 items)
constexpr int kRIBig = 16;               // items per thread of a large sort
constexpr int kRB = kRT * kRI;           // items per block: the most blocks a sort uses
constexpr int kWaves = kRT / 64;
// Sorts of at least this many items (an upper bound known on the host) take
// kRIBig items per thread: half the blocks, so half the digit histograms to
// write, scan and read back, and still >= 1024 blocks for 256 CUs.  Below it
// the smaller blocks keep the device full (a 1M-item sort is 489 blocks).
constexpr int64_t kBigSort = int64_t(1) << 22;

__device__ __forceinline__ uint32_t digit_of(uint16_t k, int shift) { return (uint32_t(k) >> shift) & 0xFFu; }
__device__ __forceinline__ uint32_t digit_of(uint32_t k, int shift) { return (k >> shift) & 0xFFu; }
__device__ __forceinline__ uint32_t digit_of(uint64_t k, int shift) { return uint32_t(k >> shift) & 0xFFu; }

__device__ __forceinline__ int64_t count_of(const int64_t* dev, int64_t host) {
  return dev != nullptr ? *dev : host;
}

// ---------------------------------------------------------------------------
// radix pass pieces
// ---------------------------------------------------------------------------
template <class K, int NI>
__global__ __launch_bounds__(kRT) void k_upsweep(const K* __restrict__ keys, const int64_t* count_dev,
                                                 int64_t count_host, int shift, uint32_t* __restrict__ H,
                                                 int nb) {
  __shared__ uint32_t hist[256];
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  hist[t] = 0;
  __syncthreads();
  const int64_t count = count_of(count_dev, count_host);
  const int64_t base = int64_t(blockIdx.x) * (kRT * NI) + int64_t(w) * (NI * 64);
  // all loads first, so they are in flight together
  uint32_t dg[NI];
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int64_t idx = base + it * 64 + lane;
    dg[it] = idx < count ? digit_of(keys[idx], shift) : 0u;
  }
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    if (base + it * 64 + lane < count) atomicAdd(&hist[dg[it]], 1u);
  }
  __syncthreads();
  H[size_t(t) * nb + blockIdx.x] = hist[t];
}

// grid = 256 blocks, one per digit: exclusive scan of H[d][0..nb) in place,
// row total to rowtot[d].
__global__ __launch_bounds__(kRT) void k_rowscan(uint32_t* __restrict__ H, int nb, uint32_t* __restrict__ rowtot) {
  __builtin_amdgcn_s_setprio(kFewPrio);
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

// One radix block (NI items per thread, input index base + it * 64 + lane
// for this thread, absent past `count`): rank_chunk plus each digit's
// global destination from the scanned histograms H / rowtot.
template <int NI>
__device__ __forceinline__ void rank_block(const uint32_t (&d)[NI], int64_t base, int64_t count,
                                           const uint32_t* __restrict__ H, const uint32_t* __restrict__ rowtot,
                                           int nb, RankSmem& sm, uint32_t (&pos)[NI]) {
  const int t = threadIdx.x, lane = t & 63;
  bool valid[NI];
#pragma unroll
  for (int it = 0; it < NI; ++it) valid[it] = base + it * 64 + lane < count;
  rank_chunk<NI>(d, valid, sm, pos);
  uint32_t rtot;
  const uint32_t rex = block_exclusive_scan<kRT, uint32_t>(rowtot[t], sm.sc, rtot);
  sm.gbase[t] = rex + H[size_t(t) * nb + blockIdx.x];
  __syncthreads();
}

// Plain stable pass: (key, value) -> (key, value) ordered by the digit at
// `shift`.
template <class K, int NI>
__global__ __launch_bounds__(kRT) void k_scatter(const K* __restrict__ kin, const uint32_t* __restrict__ vin,
                                                 K* __restrict__ kout, uint32_t* __restrict__ vout,
                                                 const int64_t* count_dev, int64_t count_host, int shift,
                                                 const uint32_t* __restrict__ H,
                                                 const uint32_t* __restrict__ rowtot, int nb) {
  __shared__ RankSmem sm;
  __shared__ K s_key[(kRT * NI)];
  __shared__ uint32_t s_val[(kRT * NI)];
  const int64_t count = count_of(count_dev, count_host);
  const int64_t bbase = int64_t(blockIdx.x) * (kRT * NI);
  if (bbase >= count) return;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  K key[NI];
  uint32_t val[NI], d[NI], pos[NI];
  const int64_t base = bbase + int64_t(w) * (NI * 64);
  // all loads first, so they are in flight together
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int64_t idx = base + it * 64 + lane;
    const bool valid = idx < count;
    key[it] = valid ? kin[idx] : K(0);
    val[it] = valid ? vin[idx] : 0u;
  }
#pragma unroll
  for (int it = 0; it < NI; ++it) d[it] = digit_of(key[it], shift);
  rank_block(d, base, count, H, rowtot, nb, sm, pos);
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    if (base + it * 64 + lane < count) {
      s_key[pos[it]] = key[it];
      s_val[pos[it]] = val[it];
    }
  }
  __syncthreads();
  const int nvalid = int(count - bbase < (kRT * NI) ? count - bbase : (kRT * NI));
  for (int j = t; j < nvalid; j += kRT) {
    const K k = s_key[j];
    const uint32_t dg = digit_of(k, shift);
    const uint32_t g = sm.gbase[dg] + (uint32_t(j) - sm.dstart[dg]);
    kout[g] = k;
    vout[g] = s_val[j];
  }
}

// The depth sort's last pass: as k_scatter, but each item's compact record
// crec[value] (gathered as the block loads its items, so the random reads
// overlap the ranking) is written at its sorted place instead of the key
// and value.
template <int NI>
__global__ __launch_bounds__(kRT) void k_scatter_rec(const uint32_t* __restrict__ kin,
                                                     const uint32_t* __restrict__ vin,
                                                     const uint4* __restrict__ crec, uint4* __restrict__ rout,
                                                     const int64_t* count_dev, int shift,
                                                     const uint32_t* __restrict__ H,
                                                     const uint32_t* __restrict__ rowtot, int nb) {
  __shared__ RankSmem sm;
  __shared__ uint4 s_rec[(kRT * NI)];
  const int64_t count = *count_dev;
  const int64_t bbase = int64_t(blockIdx.x) * (kRT * NI);
  if (bbase >= count) return;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  uint32_t d[NI], pos[NI];
  uint4 rec[NI];
  const int64_t base = bbase + int64_t(w) * (NI * 64);
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int64_t idx = base + it * 64 + lane;
    const bool valid = idx < count;
    d[it] = valid ? digit_of(kin[idx], shift) : 0u;
    rec[it] = valid ? crec[vin[idx]] : make_uint4(0u, 0u, 0u, 0u);
  }
  rank_block(d, base, count, H, rowtot, nb, sm, pos);
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    if (base + it * 64 + lane < count) s_rec[pos[it]] = rec[it];
  }
  __syncthreads();
  const int nvalid = int(count - bbase < (kRT * NI) ? count - bbase : (kRT * NI));
  for (int j = t; j < nvalid; j += kRT) {
    const uint4 e = s_rec[j];
    const uint32_t dg = digit_of(e.w, shift);
    rout[sm.gbase[dg] + (uint32_t(j) - sm.dstart[dg])] = e;
  }
}

// ---------------------------------------------------------------------------
// pipeline kernels
// ---------------------------------------------------------------------------

// Visible rank r (ascending index order): depth key, the rank itself as
// the sort's value, and the compact record (index, x0 | x1 << 16,
// y0 | y1 << 16, depth bits) from the projection record's last word.
// (bin: NULL, or the records' last four words again, densely [n][4]: 16
// bytes per Gaussian fetched instead of a 64-byte record's)
__global__ __launch_bounds__(256) void k_depth_gather(const float4* __restrict__ proj,
                                                      const float4* __restrict__ bin,
                                                      const int32_t* __restrict__ vis,
                                                      const int64_t* __restrict__ vis_count,
                                                      uint32_t* __restrict__ keys, uint32_t* __restrict__ vals,
                                                      uint4* __restrict__ crec) {
  const int64_t r = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (r >= *vis_count) return;
  const int32_t g = vis[r];
  const float4 q3 = bin != nullptr ? bin[g] : proj[4 * int64_t(g) + 3];
  const uint32_t d = __builtin_bit_cast(uint32_t, q3.x);
  keys[r] = d;
  vals[r] = uint32_t(r);
  crec[r] = make_uint4(uint32_t(g), __builtin_bit_cast(uint32_t, q3.y), __builtin_bit_cast(uint32_t, q3.z), d);
}

// Tiles of a compact record's rectangle (0 for an empty one).
__device__ __forceinline__ uint32_t rec_tiles(const uint4& e) {
  return ((e.y >> 16) - (e.y & 0xFFFFu)) * ((e.z >> 16) - (e.z & 0xFFFFu));
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
__global__ __launch_bounds__(kDT) void k_tilesum(const uint4* __restrict__ srec,
                                                 const int64_t* __restrict__ vis_count,
                                                 int64_t* __restrict__ block_sums) {
  __shared__ int64_t sh[kDT / 64];
  const int64_t V = *vis_count;
  const int64_t start = int64_t(blockIdx.x) * kDB + int64_t(threadIdx.x) * kDI;
  int64_t s = 0;
#pragma unroll
  for (int k = 0; k < kDI; ++k) {
    const int64_t r = start + k;
    if (r < V) s += rec_tiles(srec[r]);
  }
  int64_t tot;
  block_exclusive_scan<kDT, int64_t>(s, sh, tot);
  if (threadIdx.x == 0) block_sums[blockIdx.x] = tot;
}


// Pairs in depth order: for each visible Gaussian (depth rank r), one pair
// per tile of its rectangle, row-major.  Load-balanced: the block's
// Gaussians and their exclusive pair offsets go to LDS, then the block's
// threads write its output range round-robin (coalesced), each locating
// its Gaussian by binary search over the offsets.
__global__ __launch_bounds__(kDT) void k_duplicate(const uint4* __restrict__ srec,
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
      const uint4 e = srec[r];
      const uint32_t rx = e.y, ry = e.z;
      const uint32_t x0 = rx & 0xFFFFu, x1 = rx >> 16;
      cnt[k] = rec_tiles(e);
      s_rx[t * kDI + k] = x0 | ((x1 - x0) << 16);
      s_y0[t * kDI + k] = ry & 0xFFFFu;
      s_dep[t * kDI + k] = e.w;
      s_g[t * kDI + k] = e.x;
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
// exact placement through super-tiles (images up to 256 x 256 tiles)
// ---------------------------------------------------------------------------
// A super-tile is an S x S block of tiles (S = 8, or 16 where an 8 grid
// would exceed 256 blocks); the image holds SX x SY <= 256 of them.
//   a. per block of kDB Gaussians in depth order: its entries in each
//      super-tile (one entry per super-tile a tile rectangle meets; a
//      difference array over the super-tile grid), and its pair total;
//   b. entries generated in depth order and placed stably by super-tile
//      (wave-ballot ranking on the 8-bit super-tile id), so each
//      super-tile's list is in depth order; an entry holds the Gaussian,
//      its depth bits and its rectangle clipped to the super-tile;
//   c. each list is cut in chunks of kQ entries; per chunk its pairs in
//      each of the S x S tiles (difference array), scanned over the
//      super-tile's chunks, then over all tiles in tile-id order: every
//      tile's range and each chunk's first slot in each tile;
//   d. per chunk, thread (part p, tile t) walks part p of the chunk's
//      entries in order and writes the pair of each entry that covers t at
//      t's next slot.
// Every step keeps the depth order inside a tile, and equal depths stay in
// index order (the depth sort is stable over the ascending visible list).
constexpr int kMaxT = 256;               // tile columns / rows this path handles
constexpr int kQ = 512;                  // entries per chunk
constexpr int kEI = 4;                   // entries per thread per round of step b
constexpr int kMaxSide = 33;             // super-tile grid side + 1, at most

struct StGrid {
  int shift;     // S = 1 << shift tiles per super-tile side
  int sx, sy;    // super-tiles across, down
  int tx, ty;    // tiles across, down
};

// Step a.  block_sums[b]: pairs of block b; stcnt[s][b]: its entries in
// super-tile s (block 0 also clears the total slot stcnt[s][nbv]).
__global__ __launch_bounds__(kDT) void k_count_st(const uint4* __restrict__ srec,
                                                  const int64_t* __restrict__ vis_count, int nbv, StGrid sg,
                                                  int64_t* __restrict__ block_sums, uint32_t* __restrict__ stcnt) {
  __shared__ int64_t sh[kDT / 64];
  __shared__ int32_t s_cd[kMaxSide * kMaxSide];
  const int t = threadIdx.x;
  const int W = sg.sx + 1;
  for (int i = t; i < kMaxSide * kMaxSide; i += kDT) s_cd[i] = 0;
  __syncthreads();
  const int64_t V = *vis_count;
  const int64_t r0 = int64_t(blockIdx.x) * kDB;
  int64_t s = 0;
#pragma unroll
  for (int k = 0; k < kDI; ++k) {
    const int64_t r = r0 + t * kDI + k;
    if (r < V) {
      const uint4 e = srec[r];
      const uint32_t tiles = rec_tiles(e);
      s += tiles;
      if (tiles != 0) {
        const uint32_t rx = e.y, ry = e.z;
        const int a0 = int(rx & 0xFFFFu) >> sg.shift, a1 = (int((rx >> 16) - 1u) >> sg.shift) + 1;
        const int b0 = int(ry & 0xFFFFu) >> sg.shift, b1 = (int((ry >> 16) - 1u) >> sg.shift) + 1;
        atomicAdd(&s_cd[b0 * W + a0], 1);
        atomicAdd(&s_cd[b0 * W + a1], -1);
        atomicAdd(&s_cd[b1 * W + a0], -1);
        atomicAdd(&s_cd[b1 * W + a1], 1);
      }
    }
  }
  int64_t tot;
  block_exclusive_scan<kDT, int64_t>(s, sh, tot);
  if (t == 0) block_sums[blockIdx.x] = tot;
  // 2-D inclusive prefix of the differences: rows, then columns
  if (t < sg.sy) {
    int acc = 0;
    for (int x = 0; x < sg.sx; ++x) s_cd[t * W + x] = acc += s_cd[t * W + x];
  }
  __syncthreads();
  if (t < sg.sx) {
    int acc = 0;
    for (int y = 0; y < sg.sy; ++y) s_cd[y * W + t] = acc += s_cd[y * W + t];
  }
  __syncthreads();
  if (t < sg.sx * sg.sy) {
    stcnt[size_t(t) * (nbv + 1) + blockIdx.x] = uint32_t(s_cd[(t / sg.sx) * W + t % sg.sx]);
    if (blockIdx.x == 0) stcnt[size_t(t) * (nbv + 1) + nbv] = 0u;
  }
}

// End of stage 1, one workgroup: the per-block pair sums scanned in place
// (exclusive), the pair count M to m_dev (and m_out if given), the
// effective count m_eff = M, or 0 when M exceeds the capacity; with sttot,
// the super-tile list starts st_start[s] (exclusive scan of the entry
// totals) and chunk numbering chunk_base[s] (exclusive scan of
// ceil(sttot / kQ)), chunk_base[ns] = number of chunks.
__global__ __launch_bounds__(1024) void k_stage1_tail(int64_t* __restrict__ sums, int nb, int64_t cap,
                                                      int64_t* __restrict__ m_dev, int64_t* __restrict__ m_eff,
                                                      int64_t* __restrict__ m_out, const uint32_t* __restrict__ sttot,
                                                      int ns, uint32_t* __restrict__ st_start,
                                                      uint32_t* __restrict__ chunk_base) {
  __builtin_amdgcn_s_setprio(kFewPrio);
  __shared__ int64_t sh[16];
  __shared__ uint32_t sh32[16];
  __shared__ int64_t carry;
  const int t = threadIdx.x;
  if (t == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < nb; base += 1024) {
    const int i = base + t;
    const int64_t v = i < nb ? sums[i] : 0;
    int64_t tot;
    const int64_t ex = block_exclusive_scan<1024, int64_t>(v, sh, tot);
    if (i < nb) sums[i] = carry + ex;
    __syncthreads();
    if (t == 0) carry += tot;
    __syncthreads();
  }
  if (t == 0) {
    const int64_t M = carry;
    *m_dev = M;
    *m_eff = M <= cap ? M : 0;
    if (m_out != nullptr) *m_out = M;
  }
  if (sttot != nullptr) {
    const uint32_t c = t < ns ? sttot[t] : 0u;
    uint32_t tot, ctot;
    const uint32_t ex = block_exclusive_scan<1024, uint32_t>(c, sh32, tot);
    const uint32_t cex = block_exclusive_scan<1024, uint32_t>((c + kQ - 1) / kQ, sh32, ctot);
    if (t < ns) {
      st_start[t] = ex;
      chunk_base[t] = cex;
    }
    if (t == 0) chunk_base[ns] = ctot;
  }
}

// Step b.  Entries of a block of kDB Gaussians (depth order) in order
// (depth rank, super-tiles of the rectangle row-major), in chunks of
// kDT * kEI, ranked stably by super-tile and written at st_start[s] +
// stcnt[s][b] (entries of s in earlier blocks) + entries of s in earlier
// chunks + rank.  Entry: Gaussian index, depth bits, clipped rectangle
// x0 | (w - 1) << 4 | y0 << 8 | (h - 1) << 12 in tiles of the super-tile.
__global__ __launch_bounds__(kDT) void k_dup_st(const uint4* __restrict__ srec,
                                                const int64_t* __restrict__ vis_count,
                                                const uint32_t* __restrict__ stcnt,
                                                const uint32_t* __restrict__ st_start, int nbv, StGrid sg,
                                                const int64_t* __restrict__ m_eff, uint32_t* __restrict__ e_g,
                                                uint32_t* __restrict__ e_d, uint32_t* __restrict__ e_r) {
  __shared__ int64_t sh[kDT / 64];
  __shared__ uint32_t s_off[kDB];        // exclusive entry offset within the block
  __shared__ uint32_t s_rx[kDB];         // x0 | x1 << 16 (tiles)
  __shared__ uint32_t s_ry[kDB];         // y0 | y1 << 16
  __shared__ uint32_t s_g[kDB];
  __shared__ uint32_t s_dep[kDB];
  __shared__ uint32_t s_cb[256];         // running destination of each super-tile
  __shared__ RankSmem sm;
  __shared__ uint16_t s_pl[kDT * kEI];   // staged entries in super-tile order: Gaussian slot,
  __shared__ uint16_t s_pr[kDT * kEI];   // clipped rectangle,
  __shared__ uint8_t s_ps[kDT * kEI];    // super-tile
  if (*m_eff == 0) return;               // no pairs, or more than the buffers hold
  const int64_t V = *vis_count;
  const int64_t r0 = int64_t(blockIdx.x) * kDB;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  const int S = 1 << sg.shift;
  uint32_t cnt[kDI];
  uint32_t s = 0;
#pragma unroll
  for (int k = 0; k < kDI; ++k) {
    const int64_t r = r0 + t * kDI + k;
    cnt[k] = 0;
    if (r < V) {
      const uint4 e = srec[r];
      const uint32_t rx = e.y, ry = e.z;
      if (rec_tiles(e) != 0u) {
        const uint32_t a0 = (rx & 0xFFFFu) >> sg.shift, a1 = (((rx >> 16) - 1u) >> sg.shift) + 1u;
        const uint32_t b0 = (ry & 0xFFFFu) >> sg.shift, b1 = (((ry >> 16) - 1u) >> sg.shift) + 1u;
        cnt[k] = (a1 - a0) * (b1 - b0);
      }
      s_rx[t * kDI + k] = rx;
      s_ry[t * kDI + k] = ry;
      s_dep[t * kDI + k] = e.w;
      s_g[t * kDI + k] = e.x;
    }
    s += cnt[k];
  }
  int64_t tot;
  uint32_t off = uint32_t(block_exclusive_scan<kDT, int64_t>(int64_t(s), sh, tot));
#pragma unroll
  for (int k = 0; k < kDI; ++k) {
    // absent entries (past the visible count) get an offset no entry reaches
    s_off[t * kDI + k] = r0 + t * kDI + k < V ? off : 0xFFFFFFFFu;
    off += cnt[k];
  }
  const int ns = sg.sx * sg.sy;
  s_cb[t] = t < ns ? st_start[t] + stcnt[size_t(t) * (nbv + 1) + blockIdx.x] : 0u;
  __syncthreads();
  const uint32_t total = uint32_t(tot);
  for (uint32_t c0 = 0; c0 < total; c0 += kDT * kEI) {
    uint32_t d[kEI], pos[kEI], rect[kEI], slot[kEI];
    bool valid[kEI];
#pragma unroll
    for (int it = 0; it < kEI; ++it) {
      const uint32_t o = c0 + uint32_t(w * kEI * 64 + it * 64 + lane);
      valid[it] = o < total;
      d[it] = 0;
      rect[it] = 0;
      slot[it] = 0;
      if (valid[it]) {
        const int lo = last_at_or_below(s_off, o);
        const uint32_t local = o - s_off[lo];
        const uint32_t rx = s_rx[lo], ry = s_ry[lo];
        const uint32_t x0 = rx & 0xFFFFu, x1 = rx >> 16, y0 = ry & 0xFFFFu, y1 = ry >> 16;
        const uint32_t a0 = x0 >> sg.shift, na = (((x1 - 1u) >> sg.shift) + 1u) - a0;
        const uint32_t ea = a0 + local % na, eb = (y0 >> sg.shift) + local / na;
        const uint32_t bx = ea << sg.shift, by = eb << sg.shift;
        const uint32_t lx0 = (x0 > bx ? x0 : bx) - bx, lx1 = (x1 < bx + S ? x1 : bx + S) - bx;
        const uint32_t ly0 = (y0 > by ? y0 : by) - by, ly1 = (y1 < by + S ? y1 : by + S) - by;
        d[it] = eb * uint32_t(sg.sx) + ea;
        rect[it] = lx0 | ((lx1 - lx0 - 1u) << 4) | (ly0 << 8) | ((ly1 - ly0 - 1u) << 12);
        slot[it] = uint32_t(lo);
      }
    }
    rank_chunk<kEI>(d, valid, sm, pos);
#pragma unroll
    for (int it = 0; it < kEI; ++it) {
      if (valid[it]) {
        s_pl[pos[it]] = uint16_t(slot[it]);
        s_pr[pos[it]] = uint16_t(rect[it]);
        s_ps[pos[it]] = uint8_t(d[it]);
      }
    }
    __syncthreads();
    const int nvalid = int(total - c0 < uint32_t(kDT * kEI) ? total - c0 : uint32_t(kDT * kEI));
    for (int j = t; j < nvalid; j += kDT) {
      const uint32_t st = s_ps[j];
      const uint32_t dst = s_cb[st] + (uint32_t(j) - sm.dstart[st]);
      const uint32_t lo = s_pl[j];
      e_g[dst] = s_g[lo];
      e_d[dst] = s_dep[lo];
      e_r[dst] = s_pr[j];
    }
    __syncthreads();
    s_cb[t] += sm.dcnt[t];
    __syncthreads();
  }
}

// Super-tile s of chunk c and its entry span [e0, e1).
__device__ __forceinline__ void chunk_span(const uint32_t* __restrict__ chunk_base,
                                           const uint32_t* __restrict__ st_start,
                                           const uint32_t* __restrict__ sttot, int ns, uint32_t c, int& s,
                                           uint32_t& e0, uint32_t& e1) {
  // the last s with chunk_base[s] <= c (super-tiles without chunks share
  // the next one's base, so the last such s has chunks)
  int lo = 0;
#pragma unroll
  for (int step = 128; step >= 1; step >>= 1) lo = (lo + step < ns && chunk_base[lo + step] <= c) ? lo + step : lo;
  s = lo;
  e0 = st_start[lo] + (c - chunk_base[lo]) * uint32_t(kQ);
  const uint32_t end = st_start[lo] + sttot[lo];
  e1 = e0 + uint32_t(kQ) < end ? e0 + uint32_t(kQ) : end;
}

// Step c, first half: pairs of chunk c in local tile t (ly * S + lx) to
// cc[c][t] (a difference array over the S x S tiles).
__global__ __launch_bounds__(256) void k_count_chunk(const uint32_t* __restrict__ chunk_base,
                                                     const uint32_t* __restrict__ st_start,
                                                     const uint32_t* __restrict__ sttot, int ns,
                                                     const uint32_t* __restrict__ e_r, StGrid sg,
                                                     const int64_t* __restrict__ m_eff, uint32_t* __restrict__ cc) {
  __shared__ int32_t s_cd[17 * 17];
  if (*m_eff == 0) return;
  const int t = threadIdx.x;
  const int S = 1 << sg.shift, W = S + 1;
  const uint32_t C = chunk_base[ns];
  for (uint32_t c = blockIdx.x; c < C; c += gridDim.x) {
    for (int i = t; i < W * W; i += 256) s_cd[i] = 0;
    __syncthreads();
    int s;
    uint32_t e0, e1;
    chunk_span(chunk_base, st_start, sttot, ns, c, s, e0, e1);
    for (uint32_t e = e0 + uint32_t(t); e < e1; e += 256) {
      const uint32_t r = e_r[e];
      const int x0 = int(r & 15u), x1 = x0 + int((r >> 4) & 15u) + 1;
      const int y0 = int((r >> 8) & 15u), y1 = y0 + int(r >> 12) + 1;
      atomicAdd(&s_cd[y0 * W + x0], 1);
      atomicAdd(&s_cd[y0 * W + x1], -1);
      atomicAdd(&s_cd[y1 * W + x0], -1);
      atomicAdd(&s_cd[y1 * W + x1], 1);
    }
    __syncthreads();
    if (t < S) {
      int acc = 0;
      for (int x = 0; x < S; ++x) s_cd[t * W + x] = acc += s_cd[t * W + x];
    }
    __syncthreads();
    if (t < S) {
      int acc = 0;
      for (int y = 0; y < S; ++y) s_cd[y * W + t] = acc += s_cd[y * W + t];
    }
    __syncthreads();
    if (t < S * S) cc[size_t(c) * 256 + t] = uint32_t(s_cd[(t >> sg.shift) * W + (t & (S - 1))]);
    __syncthreads();
  }
}

// Step c, second half: per super-tile (one block each), cc scanned over its
// chunks for each local tile (exclusive, in place); each tile's pair count
// to tcount[tile] (k_tile_ranges_order turns the counts into ranges).
// 256 / (S x S) threads per tile, each scanning a contiguous run of the
// chunks from the sum of the runs before it.
__global__ __launch_bounds__(256) void k_scan_chunks(const uint32_t* __restrict__ chunk_base, StGrid sg,
                                                     const int64_t* __restrict__ m_eff, uint32_t* __restrict__ cc,
                                                     uint32_t* __restrict__ tcount) {
  __builtin_amdgcn_s_setprio(kFewPrio);
  __shared__ uint32_t s_sum[256];
  const int s = blockIdx.x, t = threadIdx.x;
  const int S = 1 << sg.shift, L = S * S, np = 256 / L;
  const int lt = t & (L - 1), part = t / L;
  const bool live = *m_eff != 0;
  const uint32_t c0 = live ? chunk_base[s] : 0u, c1 = live ? chunk_base[s + 1] : 0u;
  const uint32_t len = (c1 - c0 + uint32_t(np) - 1u) / uint32_t(np);
  const uint32_t a = c0 + uint32_t(part) * len < c1 ? c0 + uint32_t(part) * len : c1;
  const uint32_t b = a + len < c1 ? a + len : c1;
  // sixteen chunks' counts loaded together
  uint32_t sum = 0;
  for (uint32_t cb = a; cb < b; cb += 16) {
    uint32_t v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = cb + uint32_t(k) < b ? cc[size_t(cb + uint32_t(k)) * 256 + lt] : 0u;
#pragma unroll
    for (int k = 0; k < 16; ++k) sum += v[k];
  }
  s_sum[t] = sum;
  __syncthreads();
  uint32_t run = 0, total = 0;
  for (int p = 0; p < np; ++p) {
    const uint32_t v = s_sum[p * L + lt];
    run += p < part ? v : 0u;
    total += v;
  }
  for (uint32_t cb = a; cb < b; cb += 16) {
    uint32_t v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = cb + uint32_t(k) < b ? cc[size_t(cb + uint32_t(k)) * 256 + lt] : 0u;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (cb + uint32_t(k) < b) cc[size_t(cb + uint32_t(k)) * 256 + lt] = run;
      run += v[k];
    }
  }
  const int tx = (s % sg.sx) * S + (lt & (S - 1)), ty = (s / sg.sx) * S + (lt >> sg.shift);
  if (part == 0 && tx < sg.tx && ty < sg.ty) tcount[ty * sg.tx + tx] = total;
}

// 64 x 64 bit transpose across a wave: lane r holds row r (bit c = element
// (r, c)); on return lane c holds column c (bit r = element (r, c)).  Six
// stages, each exchanging the off-diagonal j x j blocks of every 2j x 2j
// block with the partner lane r ^ j.
__device__ __forceinline__ uint64_t wave_transpose64(uint64_t x, uint32_t lane) {
  constexpr uint64_t kHi[6] = {0xFFFFFFFF00000000ull, 0xFFFF0000FFFF0000ull, 0xFF00FF00FF00FF00ull,
                               0xF0F0F0F0F0F0F0F0ull, 0xCCCCCCCCCCCCCCCCull, 0xAAAAAAAAAAAAAAAAull};
#pragma unroll
  for (int st = 0; st < 6; ++st) {
    const int j = 32 >> st;
    const uint32_t lo = uint32_t(x), hi = uint32_t(x >> 32);
    const uint64_t y = uint64_t(uint32_t(__shfl_xor(int(lo), j, 64))) |
                       (uint64_t(uint32_t(__shfl_xor(int(hi), j, 64))) << 32);
    x = (lane & uint32_t(j)) == 0 ? (x & ~kHi[st]) | ((y & ~kHi[st]) << j) : (x & kHi[st]) | ((y & kHi[st]) >> j);
  }
  return x;
}

// Step d, one block per (chunk, panel of 64 tiles of its super-tile: all
// 8 x 8 tiles, or 4 rows of a 16 x 16 super-tile).  Entry i of the chunk
// covers a set of the panel's tiles (a 64-bit mask from its clipped
// rectangle); for each batch k of 64 entries the masks are transposed, so
// column word cw[k][t] has bit b set when entry 64 k + b covers tile t.
// Tile t's pairs from batch k then go to its start + the chunk's slot
// cc[c][t] + the pairs of t in batches before k + the rank of b among the
// set bits of cw[k][t]: one round per (k, t), whose active lanes write
// consecutive slots.
__global__ __launch_bounds__(256) void k_expand(const uint32_t* __restrict__ chunk_base,
                                                const uint32_t* __restrict__ st_start,
                                                const uint32_t* __restrict__ sttot, int ns,
                                                const uint32_t* __restrict__ e_g, const uint32_t* __restrict__ e_d,
                                                const uint32_t* __restrict__ e_r, const uint32_t* __restrict__ cc,
                                                const uint32_t* __restrict__ ranges, StGrid sg,
                                                const int64_t* __restrict__ m_eff, uint64_t* __restrict__ keys,
                                                uint32_t* __restrict__ vals) {
  constexpr int kK = kQ / 64;                                   // batches of 64 entries per chunk
  __shared__ uint64_t s_cw[kK][64];
  __shared__ uint32_t s_pre[kK][64];
  __shared__ uint32_t s_base[64];
  __shared__ uint32_t s_tile[64];
  __shared__ uint32_t s_eg[kQ];
  __shared__ uint32_t s_ed[kQ];
  if (*m_eff == 0) return;
  const uint32_t t = threadIdx.x, lane = t & 63u, w = t >> 6;
  const uint32_t S = 1u << sg.shift;
  const uint32_t qshift = 2u * uint32_t(sg.shift) - 6u;        // panels per super-tile: 1 or 4
  const uint32_t rows = 64u >> sg.shift;                        // tile rows per panel: 8 or 4
  const uint64_t rep = sg.shift == 3 ? 0x0101010101010101ull : 0x0001000100010001ull;
  const uint32_t tasks = chunk_base[ns] << qshift;
  for (uint32_t task = blockIdx.x; task < tasks; task += gridDim.x) {
    const uint32_t c = task >> qshift, q = task & ((1u << qshift) - 1u);
    int s;
    uint32_t e0, e1;
    chunk_span(chunk_base, st_start, sttot, ns, c, s, e0, e1);
    const uint32_t n = e1 - e0, r0 = q * rows;
    // entries -> panel masks, transposed per batch of 64 (wave w: batches w, w + 4)
#pragma unroll
    for (int h = 0; h < kK / 4; ++h) {
      const uint32_t k = w + 4u * uint32_t(h), i = 64u * k + lane;
      uint64_t m = 0;
      if (i < n) {
        const uint32_t r = e_r[e0 + i];
        s_eg[i] = e_g[e0 + i];
        s_ed[i] = e_d[e0 + i];
        const uint32_t x0 = r & 15u, wd = ((r >> 4) & 15u) + 1u, y0 = (r >> 8) & 15u, y1 = y0 + (r >> 12) + 1u;
        const uint32_t ya = y0 > r0 ? y0 : r0, yb = y1 < r0 + rows ? y1 : r0 + rows;
        if (ya < yb) {
          const uint64_t cm = ((1ull << wd) - 1ull) << x0;
          const uint64_t rm = (~0ull >> (64u - S * (yb - ya))) << (S * (ya - r0));
          m = (cm * rep) & rm;
        }
      }
      const uint64_t cw = wave_transpose64(m, lane);
      s_cw[k][lane] = cw;
      s_pre[k][lane] = uint32_t(__popcll(cw));
    }
    if (t < 64) {
      const uint32_t ly = r0 + (lane >> sg.shift), lx = lane & (S - 1u);
      const uint32_t tx = uint32_t(s % sg.sx) * S + lx, ty = uint32_t(s / sg.sx) * S + ly;
      const bool inside = tx < uint32_t(sg.tx) && ty < uint32_t(sg.ty);
      const uint32_t tile = inside ? ty * uint32_t(sg.tx) + tx : 0u;
      s_tile[lane] = tile;
      s_base[lane] = inside ? ranges[2 * size_t(tile)] + cc[size_t(c) * 256 + (ly << sg.shift) + lx] : 0u;
    }
    __syncthreads();
    if (t < 64) {
      uint32_t run = s_base[lane];
#pragma unroll
      for (int k = 0; k < kK; ++k) {
        const uint32_t v = s_pre[k][lane];
        s_pre[k][lane] = run;
        run += v;
      }
    }
    __syncthreads();
    // rounds (k, tile): lane b writes entry 64 k + b's pair when it covers the tile
#pragma unroll
    for (int h = 0; h < kK / 4; ++h) {
      const uint32_t k = w + 4u * uint32_t(h);
      if (64u * k >= n) break;
      const uint32_t i = 64u * k + lane;
      const uint32_t g = i < n ? s_eg[i] : 0u, d = i < n ? s_ed[i] : 0u;
      for (uint32_t tt = 0; tt < 64; ++tt) {
        const uint64_t cw = s_cw[k][tt];
        if (cw == 0) continue;
        if ((cw >> lane) & 1ull) {
          const uint32_t pos = s_pre[k][tt] + uint32_t(count_below(cw));
          if (keys != nullptr) keys[pos] = (uint64_t(s_tile[tt]) << 32) | d;
          vals[pos] = g;
        }
      }
    }
    __syncthreads();
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
__device__ __forceinline__ void tile_order_block(const uint32_t* __restrict__ ranges, int nT,
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

__global__ __launch_bounds__(1024) void k_tile_order(const uint32_t* __restrict__ ranges, int nT,
                                                     uint32_t* __restrict__ order) {
  tile_order_block(ranges, nT, order);
}

// The exact path's last step: tile counts to ranges [start, end) in tile-id
// order (empty tiles [0, 0)) and, with `order`, the rasterisers' launch
// order (as tile_order_block: a stable counting sort by descending bit
// length of the counts).  Workgroup b takes tiles [b kSlice, (b + 1)
// kSlice).  It first reads the counts of the tiles before its slice (their
// pair sum: the slice's first start) and, for the order, every tile's
// bucket (per bucket, the tiles in all and those before the slice), so no
// workgroup waits on another; the slice is then scanned and ranked with
// wave ballots, per (bucket, r, wave) in tile-id order.
constexpr int kTR = 256;                     // threads
constexpr int kTRR = 2;                      // tiles per thread
constexpr int kSlice = kTR * kTRR;           // tiles per workgroup
constexpr int kBk = 33;                      // order buckets: bit length 0..32

__device__ __forceinline__ uint32_t order_bucket(uint32_t len) {  // 0 = longest lists
  return 32u - (len != 0 ? 32u - uint32_t(__builtin_clz(len)) : 0u);
}

__global__ __launch_bounds__(kTR) void k_tile_ranges_order(int nT, const uint32_t* __restrict__ tcount,
                                                           uint32_t* __restrict__ ranges,
                                                           uint32_t* __restrict__ order) {
  __builtin_amdgcn_s_setprio(kFewPrio);
  constexpr int kW = kTR / 64;
  __shared__ uint32_t s_all[kBk], s_before[kBk];
  __shared__ uint32_t s_cnt[kBk][kTRR][kW];  // lanes per (bucket, r, wave), then their first slots
  __shared__ uint32_t sh[kW];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int s0 = int(blockIdx.x) * kSlice;
  const bool want_order = order != nullptr;
  if (t < kBk) {
    s_all[t] = 0;
    s_before[t] = 0;
  }
  for (int k = t; k < kBk * kTRR * kW; k += kTR) (&s_cnt[0][0][0])[k] = 0;
  __syncthreads();
  uint32_t before = 0;
  const int scan_end = want_order ? nT : s0;
  // (eight chunks' counts loaded together, so their latencies overlap)
  constexpr int kU = 8;
  for (int base0 = 0; base0 < scan_end; base0 += kU * kTR) {
    uint32_t cv[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int j = base0 + u * kTR + t;
      cv[u] = base0 + u * kTR < scan_end && j < nT ? tcount[j] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int base = base0 + u * kTR;
      if (base >= scan_end) break;
      const bool valid = base + t < nT;
      const uint32_t c = cv[u];
      const bool pre = base < s0;            // (kSlice is a multiple of kTR: chunks never straddle s0)
      before += pre ? c : 0u;
      if (want_order) {
        const uint32_t b = order_bucket(c);
        const uint64_t peers = match_bits<6>(b, ballot(valid));
        if (valid && count_below(peers) == 0) {
          const uint32_t k = uint32_t(__popcll(peers));
          atomicAdd(&s_all[b], k);
          if (pre) atomicAdd(&s_before[b], k);
        }
      }
    }
  }
  uint32_t carry;
  block_exclusive_scan<kTR, uint32_t>(before, sh, carry);
  uint32_t bk[kTRR], below[kTRR];
#pragma unroll
  for (int r = 0; r < kTRR; ++r) {
    const int i = s0 + r * kTR + t;
    const bool valid = i < nT;
    const uint32_t v = valid ? tcount[i] : 0u;
    uint32_t tot;
    const uint32_t start = carry + block_exclusive_scan<kTR, uint32_t>(v, sh, tot);
    carry += tot;
    if (valid) {
      ranges[2 * size_t(i)] = v != 0 ? start : 0u;
      ranges[2 * size_t(i) + 1] = v != 0 ? start + v : 0u;
    }
    bk[r] = order_bucket(v);
    below[r] = 0;
    if (want_order) {
      const uint64_t peers = match_bits<6>(bk[r], ballot(valid));
      below[r] = uint32_t(count_below(peers));
      if (valid && below[r] == 0) s_cnt[bk[r]][r][w] = uint32_t(__popcll(peers));
    }
  }
  if (!want_order) return;
  __syncthreads();
  if (t < kBk) {
    // tiles of longer buckets, then this bucket's tiles before the slice
    uint32_t run = s_before[t];
    for (int b = 0; b < t; ++b) run += s_all[b];
    for (int r = 0; r < kTRR; ++r)
      for (int k = 0; k < kW; ++k) {
        const uint32_t c = s_cnt[t][r][k];
        s_cnt[t][r][k] = run;
        run += c;
      }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kTRR; ++r) {
    const int i = s0 + r * kTR + t;
    if (i < nT) order[s_cnt[bk[r]][r][w] + below[r]] = uint32_t(i);
  }
}

// ---------------------------------------------------------------------------
// workspace layout
// ---------------------------------------------------------------------------
struct Ws {
  uint32_t *dkA, *dvA, *dkB, *dvB;   // depth sort ping-pong [n]
  uint4* crec;                       // compact records [n], visible-rank order
  uint4* srec;                       // the same, depth order
  uint32_t* H;                       // radix histograms [256][nb]
  uint32_t* rowtot;                  // [256]
  uint32_t* sttot;                   // [256], entries per super-tile
  uint32_t* st_start;                // [256], super-tile list starts
  uint32_t* chunk_base;              // [257], first chunk of each super-tile; number of chunks
  uint32_t* tcount;                  // [kMaxT * kMaxT], pairs per tile
  int64_t* bsums;                    // per-block tile sums [nbv + 1]
  int64_t* m_dev;                    // pair count
  int64_t* m_eff;                    // pair count if within capacity, else 0
  uint32_t* stcnt;                   // [256][nbv + 1], entries per (super-tile, block), then scanned
  uint32_t* cc;                      // [max_chunks(cap)][256], pairs per (chunk, local tile), then scanned
  uint64_t* pk;                      // pair keys scratch [cap]; super-tile entries (index, depth)
  uint32_t* pv;                      // pair values scratch [cap]; super-tile entry rectangles
};

// Chunks of the super-tile lists: at most one partial chunk per super-tile
// beyond the entries / kQ full ones (entries <= pairs <= capacity).
inline int64_t max_chunks(int64_t cap) { return cap / kQ + 257; }

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
  w.crec = reinterpret_cast<uint4*>(take(sizeof(uint4) * size_t(n)));
  w.srec = reinterpret_cast<uint4*>(take(sizeof(uint4) * size_t(n)));
  w.H = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * 256 * size_t(nbh)));
  w.rowtot = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * 256));
  w.sttot = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * 256));
  w.st_start = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * 256));
  w.chunk_base = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * 257));
  w.tcount = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * size_t(kMaxT) * kMaxT));
  w.bsums = reinterpret_cast<int64_t*>(take(sizeof(int64_t) * size_t(nbv + 1)));
  w.m_dev = reinterpret_cast<int64_t*>(take(sizeof(int64_t)));
  w.m_eff = reinterpret_cast<int64_t*>(take(sizeof(int64_t)));
  w.stcnt = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * 256 * size_t(nbv + 1)));
  w.cc = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * 256 * size_t(max_chunks(cap))));
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

// The super-tile path: images up to 256 x 256 tiles (at most 16 x 16
// super-tiles of 16 x 16 tiles).
inline bool exact_path(int32_t tiles_x, int32_t tiles_y) { return tiles_x <= kMaxT && tiles_y <= kMaxT; }

// Super-tiles of 8 x 8 tiles where at most 256 of them cover the image,
// else 16 x 16.
inline StGrid st_grid(int32_t tiles_x, int32_t tiles_y) {
  StGrid g;
  g.tx = tiles_x;
  g.ty = tiles_y;
  for (g.shift = 3; g.shift < 4; ++g.shift) {
    const int S = 1 << g.shift;
    if (((tiles_x + S - 1) / S) * ((tiles_y + S - 1) / S) <= 256 && (tiles_x + S - 1) / S < kMaxSide &&
        (tiles_y + S - 1) / S < kMaxSide)
      break;
  }
  const int S = 1 << g.shift;
  g.sx = (tiles_x + S - 1) / S;
  g.sy = (tiles_y + S - 1) / S;
  return g;
}

// Blocks of a sort of at most count_bound items at NI items per thread.
template <int NI>
int radix_blocks(int64_t count_bound) {
  return int(std::max<int64_t>(1, (count_bound + kRT * NI - 1) / (kRT * NI)));
}

template <class K, int NI>
void radix_pass_ni(const K* kin, const uint32_t* vin, K* kout, uint32_t* vout, const int64_t* count_dev,
                   int64_t count_host, int64_t count_bound, int shift, const Ws& w, hipStream_t st) {
  const int nb = radix_blocks<NI>(count_bound);
  k_upsweep<K, NI><<<nb, kRT, 0, st>>>(kin, count_dev, count_host, shift, w.H, nb);
  k_rowscan<<<256, kRT, 0, st>>>(w.H, nb, w.rowtot);
  k_scatter<K, NI><<<nb, kRT, 0, st>>>(kin, vin, kout, vout, count_dev, count_host, shift, w.H, w.rowtot, nb);
}

template <class K>
void radix_pass(const K* kin, const uint32_t* vin, K* kout, uint32_t* vout, const int64_t* count_dev,
                int64_t count_host, int64_t count_bound, int shift, const Ws& w, hipStream_t st) {
  if (count_bound >= kBigSort)
    radix_pass_ni<K, kRIBig>(kin, vin, kout, vout, count_dev, count_host, count_bound, shift, w, st);
  else
    radix_pass_ni<K, kRI>(kin, vin, kout, vout, count_dev, count_host, count_bound, shift, w, st);
}

// The depth sort's last pass (digit 24..31), records out.
template <int NI>
void rec_pass(const Ws& w, const int64_t* vis_count, int64_t n, hipStream_t st) {
  const int nb = radix_blocks<NI>(n);
  k_upsweep<uint32_t, NI><<<nb, kRT, 0, st>>>(w.dkB, vis_count, 0, 24, w.H, nb);
  k_rowscan<<<256, kRT, 0, st>>>(w.H, nb, w.rowtot);
  k_scatter_rec<NI><<<nb, kRT, 0, st>>>(w.dkB, w.dvB, w.crec, w.srec, vis_count, 24, w.H, w.rowtot, nb);
}

}  // namespace

size_t binsort_ws_bytes(int64_t n, int64_t pair_capacity) { return carve_bytes(n, pair_capacity); }

bool binsort_keys_optional(int32_t tiles_x, int32_t tiles_y) { return exact_path(tiles_x, tiles_y); }

int64_t* binsort_count_ptr(void* ws, int64_t n, int64_t pair_capacity) {
  return carve(ws, n, pair_capacity).m_dev;
}

hipError_t launch_binsort_stage1(const float* proj, const float* proj_bin, int64_t n, const int32_t* vis_idx,
                                 const int64_t* vis_count, int32_t tiles_x, int32_t tiles_y, int64_t* num_pairs_dev,
                                 void* ws, int64_t pair_capacity, hipStream_t st) {
  Ws w = carve(ws, n, pair_capacity);
  const float4* P = reinterpret_cast<const float4*>(proj);
  if (n > 0) {
    k_depth_gather<<<unsigned((n + 255) / 256), 256, 0, st>>>(P, reinterpret_cast<const float4*>(proj_bin), vis_idx,
                                                               vis_count, w.dkA, w.dvA, w.crec);
    // stable LSD radix on the 32 depth bits: A -> B -> A -> B, then the
    // records in depth order
    for (int pass = 0; pass < 3; ++pass) {
      const bool even = (pass & 1) == 0;
      radix_pass<uint32_t>(even ? w.dkA : w.dkB, even ? w.dvA : w.dvB, even ? w.dkB : w.dkA,
                           even ? w.dvB : w.dvA, vis_count, 0, n, 8 * pass, w, st);
    }
    if (n >= kBigSort)
      rec_pass<kRIBig>(w, vis_count, n, st);
    else
      rec_pass<kRI>(w, vis_count, n, st);
  }
  const int nbv = int(dup_blocks(n));
  int ns = 0;
  if (nbv > 0 && exact_path(tiles_x, tiles_y)) {
    // pair totals, entries per (super-tile, block)
    const StGrid sg = st_grid(tiles_x, tiles_y);
    ns = sg.sx * sg.sy;
    k_count_st<<<nbv, kDT, 0, st>>>(w.srec, vis_count, nbv, sg, w.bsums, w.stcnt);
    k_rowscan<<<unsigned(ns), kRT, 0, st>>>(w.stcnt, nbv + 1, w.sttot);
  } else if (nbv > 0) {
    k_tilesum<<<nbv, kDT, 0, st>>>(w.srec, vis_count, w.bsums);
  }
  // block offsets, M, the effective count; super-tile list starts and chunks
  k_stage1_tail<<<1, 1024, 0, st>>>(w.bsums, nbv, pair_capacity, w.m_dev, w.m_eff, num_pairs_dev,
                                    ns > 0 ? w.sttot : nullptr, ns, w.st_start, w.chunk_base);
  return hipGetLastError();
}

// Second half.  M_host >= 0: the pair count read by the caller (<= the
// capacity).  M_host < 0: the count stays on the device (nothing blocks);
// grids are sized for the capacity and every kernel reads the effective
// count (0 when M exceeds the capacity: then only empty ranges are written).
hipError_t launch_binsort_stage2(const float* proj, int64_t n, const int32_t* vis_idx,
                                 const int64_t* vis_count, int64_t M_host, int32_t tiles_x, int32_t tiles_y,
                                 uint64_t* keys, int32_t* vals, uint32_t* ranges, uint32_t* tile_order, void* ws,
                                 int64_t pair_capacity, hipStream_t st) {
  (void)vis_idx;
  (void)proj;
  Ws w = carve(ws, n, pair_capacity);
  const int64_t T = int64_t(tiles_x) * tiles_y;
  uint32_t* uvals = reinterpret_cast<uint32_t*>(vals);
  const int nbv = int(dup_blocks(n));
  const bool on_device = M_host < 0;
  const int64_t* m_dev = nullptr;
  int64_t bound = M_host;                       // upper bound of the count, for grid sizes
  if (on_device) {
    m_dev = w.m_eff;                            // from stage 1
    bound = pair_capacity;
  }
  if (exact_path(tiles_x, tiles_y) && nbv > 0) {
    // super-tile entries, per-chunk tile counts, ranges, then the pairs;
    // every kernel reads the effective count (0: no pairs or overflow)
    const StGrid sg = st_grid(tiles_x, tiles_y);
    const int ns = sg.sx * sg.sy;
    // the chunk counts' grid: up to 32 workgroups per CU, as the expansion's
    // below (a large capped grid lets the CUs freed first take more chunks)
    const unsigned grid = unsigned(std::min<int64_t>(max_chunks(pair_capacity), 8192));
    // the pair expansion's (chunk, panel) tasks: up to 64 workgroups per CU,
    // most of them queued, so the CUs that the rasterisers on the other
    // stream free first take more of the tasks
    const unsigned egrid = unsigned(std::min<int64_t>(max_chunks(pair_capacity) * 4, 16384));
    uint32_t* e_g = reinterpret_cast<uint32_t*>(w.pk);
    uint32_t* e_d = e_g + pair_capacity;
    uint32_t* e_r = w.pv;
    k_dup_st<<<nbv, kDT, 0, st>>>(w.srec, vis_count, w.stcnt, w.st_start, nbv, sg, w.m_eff, e_g, e_d, e_r);
    k_count_chunk<<<grid, 256, 0, st>>>(w.chunk_base, w.st_start, w.sttot, ns, e_r, sg, w.m_eff, w.cc);
    k_scan_chunks<<<unsigned(ns), 256, 0, st>>>(w.chunk_base, sg, w.m_eff, w.cc, w.tcount);
    k_tile_ranges_order<<<unsigned((T + kSlice - 1) / kSlice), kTR, 0, st>>>(int(T), w.tcount, ranges, tile_order);
    k_expand<<<egrid, 256, 0, st>>>(w.chunk_base, w.st_start, w.sttot, ns, e_g, e_d, e_r, w.cc, ranges, sg, w.m_eff,
                                   keys, uvals);
    return hipGetLastError();
  } else if (!on_device && M_host == 0) {
    k_fill_u32<<<unsigned((2 * T + 255) / 256), 256, 0, st>>>(ranges, 2 * T, 0u);
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
      k_duplicate<<<nbv, kDT, 0, st>>>(w.srec, vis_count, w.bsums, tiles_x, m_dev, bufk[cur], bufv[cur]);
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
