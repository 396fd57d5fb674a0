// View coupling (Odin summary page, "Relative locality graph": the edge
// weight of two views is the Jaccard similarity of their point sets, 0 for
// an empty union; the scheduling priority of a view given a previous set
// U_prev is the sum of its weights to the views in U_prev), with the views'
// visible-index lists (what the preprocess emits per view) as the point
// sets.
//
// Each list becomes a bitmap of n bits (one u32 word per 32 Gaussians; an
// ascending list fills each word from one thread, without atomics).  The
// intersection counts are then the Gram matrix of the bitmaps: entry (i, j)
// is the sum over words of popcount(word_i & word_j).  A workgroup owns a
// 64 x 64 tile of view pairs (tiles on or above the diagonal only) and a
// range of words; it stages 64 words of its 128 rows in LDS per step and
// each thread forms a 4 x 4 block of pairs.  Tile sums are added to the
// int64 matrix with atomics: integer addition is exact in any order, so
// the counts, and the fp64 weights computed from them, do not depend on
// the schedule.
#include <algorithm>

#include "gs_internal.h"

namespace gs {
namespace {

constexpr int kVT = 64;            // views per tile side
constexpr int kCW = 64;            // bitmap words per LDS step
constexpr int kRow = kCW + 4;      // LDS row stride in words (rows 16 apart land 64 banks apart)
constexpr int kTargetBlocks = 2048;

__global__ __launch_bounds__(256) void k_zero64(uint64_t* __restrict__ p, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) p[i] = 0u;
}

__global__ __launch_bounds__(256) void k_zero32(uint4* __restrict__ p, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Bitmap rows from the lists.  A wave takes a chunk of kChunkE consecutive
// entries of one list (loaded coalesced into LDS, with the entry before it
// and kSlice after it); lane i folds entries [32 i, 32 i + 32) of the chunk
// into words.  A word belongs to the lane whose slice holds its first
// entry: a lane skips the entries of the word open before its slice, and
// reads on past its slice until its own last word closes (at most 31
// entries: a word has 32 indices).  So every word is stored once, whole,
// with no atomics.  Entries outside [0, n) are skipped.
constexpr int kSlice = 32;
constexpr int kChunkE = 64 * kSlice;
constexpr int kStage = kChunkE + kSlice + 1;              // entries staged per chunk
constexpr int kStagePad = kStage + (kStage + 31) / 32;   // one pad word every 32 entries
constexpr int kStageIters = (kStage + 63) / 64;

__device__ __forceinline__ int stage_at(int k) { return k + (k >> 5); }

__device__ __forceinline__ bool wave_any_c(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

__global__ __launch_bounds__(256) void k_bitmap(const int32_t* __restrict__ lists, int64_t ld,
                                                const int64_t* __restrict__ counts, int64_t n, int per_view,
                                                int64_t words_pad, uint32_t* __restrict__ bm) {
  __shared__ int32_t s_e[4][kStagePad];
  const int wave = int(threadIdx.x) >> 6, lane = int(threadIdx.x) & 63;
  const int v = int(blockIdx.x) / per_view;
  const int part = int(blockIdx.x) % per_view;
  const int32_t* __restrict__ list = lists + size_t(v) * size_t(ld);
  int64_t count = counts[v];
  count = count < 0 ? 0 : count;
  count = count > ld ? ld : count;
  uint32_t* __restrict__ row = bm + size_t(v) * size_t(words_pad);
  int32_t* const buf = s_e[wave];
  const int64_t stride = int64_t(per_view) * 4 * kChunkE;
  for (int64_t base = (int64_t(part) * 4 + wave) * kChunkE; base < count; base += stride) {
    // staged position k holds entry base - 1 + k (-1 outside the list);
    // all loads issued before the first is waited for (the index is
    // clamped into the list, count > base >= 0, and the value dropped after)
    int32_t e[kStageIters];
    {
      // one wave-uniform base and 32-bit unsigned lane offsets, clamped
      // into the list
      const int64_t bu = int64_t((uint64_t(__builtin_amdgcn_readfirstlane(uint32_t(uint64_t(base) >> 32))) << 32) |
                                 uint64_t(__builtin_amdgcn_readfirstlane(uint32_t(base))));
      const int64_t pb = bu > 0 ? bu - 1 : 0;
      const int32_t* __restrict__ p = list + pb;
      const int shift = int(bu - 1 - pb);   // -1 for the list's first chunk, else 0
      const uint32_t hi = uint32_t(std::min<int64_t>(count - 1 - pb, int64_t(kStageIters) * 64));
#pragma unroll
      for (int m = 0; m < kStageIters; ++m) {
        const int o = lane + 64 * m + shift;
        const uint32_t u = o < 0 ? 0u : (uint32_t(o) > hi ? hi : uint32_t(o));
        e[m] = p[u];
      }
    }
#pragma unroll
    for (int m = 0; m < kStageIters; ++m) {
      const int k = lane + 64 * m;
      const int64_t r = base - 1 + k;
      if (k < kStage) buf[stage_at(k)] = r >= 0 && r < count ? e[m] : -1;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int64_t r0 = base + int64_t(kSlice) * lane;
    // staged position of entry r0 - 1 + k is 33 lane + k + (k >> 5) for k < 64
    const int32_t* const mine = buf + 33 * lane;
    const int jend = int(std::max<int64_t>(0, std::min<int64_t>(2 * kSlice, count - r0)));
    // 0 <= g < n as one unsigned compare (n < 2^31)
    const uint32_t un = uint32_t(n);
    const int32_t gp = mine[0];
    const int32_t wprev = uint32_t(gp) < un ? gp >> 5 : -1;
    int32_t wcur = -1;
    uint32_t bits = 0;
    bool cont = true;   // the open word may go on past the entries read so far
    // entries in batches of 8 (reads issued together); past the slice a
    // batch is read only while some lane's open word goes on
#pragma unroll
    for (int j0 = 0; j0 < 2 * kSlice; j0 += 8) {
      if (j0 >= kSlice && !wave_any_c(cont && j0 < jend)) break;
      int32_t g[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) g[q] = mine[1 + j0 + q + ((1 + j0 + q) >> 5)];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = j0 + q;
        // (bitwise &: every operand is already computed, a branch per
        // condition would cost more than the operation)
        const bool valid = (j < jend) & (uint32_t(g[q]) < un);
        const int32_t w = valid ? g[q] >> 5 : -2;
        // past the slice only the open word's entries count
        const bool take = valid & (w != wprev) & ((j < kSlice) | (w == wcur));
        const bool fresh = take & (w != wcur);
        if (fresh && wcur >= 0) row[wcur] = bits;
        bits = fresh ? 0u : bits;
        wcur = fresh ? w : wcur;
        bits |= take ? 1u << (g[q] & 31) : 0u;
        if (q == 7) cont = j < kSlice - 1 || take;
      }
    }
    if (wcur >= 0) row[wcur] = bits;
    __builtin_amdgcn_wave_barrier();
  }
}

// acc + popcount(m) as one v_bcnt_u32_b32 (left to itself the compiler
// counts into 0 and adds the counts in pairs: a third more instructions)
__device__ __forceinline__ uint32_t bcnt_add(uint32_t m, uint32_t acc) {
  uint32_t r;
  asm("v_bcnt_u32_b32 %0, %1, %2" : "=v"(r) : "v"(m), "v"(acc));
  return r;
}

// Tile t of the upper triangle (ti <= tj), row by row.
__device__ __forceinline__ void tile_of(int t, int nt, int& ti, int& tj) {
  ti = 0;
  int rem = t;
  while (rem >= nt - ti) {
    rem -= nt - ti;
    ++ti;
  }
  tj = ti + rem;
}

// Workgroup b: tile b % T over word steps [s0, s1) of split b / T.  Thread
// (ty, tx) = (t / 16, t % 16) owns rows 4 ty + r (a wave: 16 consecutive
// rows) and columns tx + 16 c.
__global__ __launch_bounds__(256) void k_overlap(const uint32_t* __restrict__ bm, int B, int64_t words_pad, int nt,
                                                 int T, int steps_per_split, unsigned long long* __restrict__ inter) {
  __shared__ uint4 s_a[kVT * kRow / 4];
  __shared__ uint4 s_b[kVT * kRow / 4];
  const int t = threadIdx.x;
  const int tile = int(blockIdx.x) % T;
  const int split = int(blockIdx.x) / T;
  int ti, tj;
  tile_of(tile, nt, ti, tj);
  const int r0 = ti * kVT, c0 = tj * kVT;
  const int64_t nsteps = words_pad / kCW;
  const int64_t s0 = int64_t(split) * steps_per_split;
  const int64_t s1 = std::min<int64_t>(nsteps, s0 + steps_per_split);
  const int ty = t >> 4, tx = t & 15;
  // a wave whose 16 rows all lie past the last view has nothing to add
  const bool rows_live = r0 + 16 * (t >> 6) < B;

  // staging: uint4 e = t + 256 k of a panel is row e / 16, words 4 (e % 16)
  uint4 ra[4], rb[4];
  auto fetch = [&](int64_t s) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = t + 256 * k;
      const int row = e >> 4, q = e & 15;
      const size_t off = size_t(s) * kCW + size_t(4 * q);
      ra[k] = r0 + row < B ? *reinterpret_cast<const uint4*>(bm + size_t(r0 + row) * size_t(words_pad) + off)
                           : make_uint4(0u, 0u, 0u, 0u);
      rb[k] = c0 + row < B ? *reinterpret_cast<const uint4*>(bm + size_t(c0 + row) * size_t(words_pad) + off)
                           : make_uint4(0u, 0u, 0u, 0u);
    }
  };

  uint32_t acc[4][4] = {};
  if (s0 < s1) fetch(s0);
  for (int64_t s = s0; s < s1; ++s) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = t + 256 * k;
      const int row = e >> 4, q = e & 15;
      s_a[(row * kRow) / 4 + q] = ra[k];
      s_b[(row * kRow) / 4 + q] = rb[k];
    }
    __syncthreads();
    if (s + 1 < s1) fetch(s + 1);
    if (rows_live) {
#pragma unroll 4
      for (int q = 0; q < kCW / 4; ++q) {
        uint4 a[4], b[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) a[r] = s_a[((4 * ty + r) * kRow) / 4 + q];
#pragma unroll
        for (int c = 0; c < 4; ++c) b[c] = s_b[((tx + 16 * c) * kRow) / 4 + q];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            uint32_t x = acc[r][c];
            x = bcnt_add(a[r].x & b[c].x, x);
            x = bcnt_add(a[r].y & b[c].y, x);
            x = bcnt_add(a[r].z & b[c].z, x);
            x = bcnt_add(a[r].w & b[c].w, x);
            acc[r][c] = x;
          }
      }
    }
    __syncthreads();
  }
  if (!rows_live || s0 >= s1) return;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int i = r0 + 4 * ty + r, j = c0 + tx + 16 * c;
      if (i >= B || j >= B || acc[r][c] == 0u) continue;
      atomicAdd(inter + size_t(i) * B + j, (unsigned long long)acc[r][c]);
      if (ti != tj) atomicAdd(inter + size_t(j) * B + i, (unsigned long long)acc[r][c]);
    }
}

// w_ij = |V_i n V_j| / (|V_i| + |V_j| - |V_i n V_j|), 0 for an empty union.
__global__ __launch_bounds__(256) void k_jaccard(const int64_t* __restrict__ inter, int B, double* __restrict__ w) {
  const int64_t nn = int64_t(B) * B;
  for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < nn; e += int64_t(gridDim.x) * 256) {
    const int64_t i = e / B, j = e % B;
    const int64_t x = inter[e];
    const int64_t u = inter[i * B + i] + inter[j * B + j] - x;
    w[e] = u > 0 ? double(x) / double(u) : 0.0;
  }
}

// s(v | U_prev): the weights w_uv added in the order of `prev` (entries
// outside [0, B) are skipped).
__global__ __launch_bounds__(256) void k_priority(const double* __restrict__ w, int B,
                                                  const int32_t* __restrict__ prev, int nprev,
                                                  double* __restrict__ s) {
  const int v = int(blockIdx.x) * 256 + threadIdx.x;
  if (v >= B) return;
  double acc = 0.0;
  for (int k = 0; k < nprev; ++k) {
    const int32_t u = prev[k];
    if (u >= 0 && u < B) acc = acc + w[size_t(u) * B + v];
  }
  s[v] = acc;
}

int64_t words_padded(int64_t n) { return ((n + 31) / 32 + kCW - 1) / kCW * kCW; }

}  // namespace

size_t coupling_ws_bytes(int64_t n, int32_t num_views) {
  return sizeof(uint32_t) * size_t(words_padded(n)) * size_t(num_views > 0 ? num_views : 0);
}

hipError_t launch_view_overlap(const int32_t* lists, int64_t ld, const int64_t* counts, int B, int64_t n,
                               int64_t* inter, double* weights, void* ws, hipStream_t st) {
  const int64_t words_pad = words_padded(n);
  uint32_t* bm = static_cast<uint32_t*>(ws);
  unsigned long long* acc = reinterpret_cast<unsigned long long*>(inter);
  const int64_t nn = int64_t(B) * B;
  k_zero64<<<unsigned(std::min<int64_t>((nn + 255) / 256, 4096)), 256, 0, st>>>(
      reinterpret_cast<uint64_t*>(inter), nn);
  if (words_pad > 0) {
    const int64_t q = int64_t(B) * words_pad / 4;   // rows are whole uint4s
    k_zero32<<<unsigned(std::min<int64_t>((q + 255) / 256, 8192)), 256, 0, st>>>(reinterpret_cast<uint4*>(bm), q);
    // about 8192 workgroups over all the lists, each list at least one
    const int per_view =
        int(std::max<int64_t>(1, std::min<int64_t>((n + 4 * kChunkE - 1) / (4 * kChunkE), 8192 / B)));
    k_bitmap<<<unsigned(B * per_view), 256, 0, st>>>(lists, ld, counts, n, per_view, words_pad, bm);
    const int nt = (B + kVT - 1) / kVT;
    const int T = nt * (nt + 1) / 2;
    const int64_t nsteps = words_pad / kCW;
    const int64_t splits = std::max<int64_t>(1, std::min<int64_t>(nsteps, (kTargetBlocks + T - 1) / T));
    const int steps_per_split = int((nsteps + splits - 1) / splits);
    const int64_t used = (nsteps + steps_per_split - 1) / steps_per_split;
    k_overlap<<<unsigned(T * used), 256, 0, st>>>(bm, B, words_pad, nt, T, steps_per_split, acc);
  }
  if (weights != nullptr)
    k_jaccard<<<unsigned(std::min<int64_t>((nn + 255) / 256, 65536)), 256, 0, st>>>(inter, B, weights);
  return hipGetLastError();
}

hipError_t launch_view_priority(const double* weights, int B, const int32_t* prev, int nprev, double* score,
                                hipStream_t st) {
  k_priority<<<unsigned((B + 255) / 256), 256, 0, st>>>(weights, B, prev, nprev, score);
  return hipGetLastError();
}

}  // namespace gs
