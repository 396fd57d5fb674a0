// Pieces shared by the forward and backward rasterisers.
//
// Work layout: four waves (64 lanes each) per 16x16 tile, wave q owning the
// tile's 8x8 quarter q (x + 8 (q & 1), y + 8 (q >> 1)); lane l owns the
// pixel at offset (l & 7, l >> 3) of it.  The tile's depth-sorted list is
// consumed in chunks of 64 entries: lane l stages entry l's record in LDS
// and tests the Gaussian's alpha >= 1/255 footprint against the wave's
// quarter; one ballot gives the 64-bit set of chunk entries that can
// reach it.  The loop then visits only set bits (scalar
// bit scans), so Gaussians that cannot reach a quarter cost it no vector
// work.
#pragma once

#include "gs_device.hpp"

namespace gs {

constexpr int kChunk = 64;

// Wave issue priority of the rasterisers (s_setprio, 0..3; other kernels
// run at 0).
constexpr int kRasterPrio = 2;

// Waves (one per quarter) per tile.
constexpr int kWPT = 4;

// Split backward of long lists.  While compositing, a quarter's forward
// records its per-pixel state at each list position that is a multiple of
// the segment length (up to kCkSeg of them, in slots taken from a counter):
// T before that entry and the colour the segment ending there added.  At
// its end it turns those into the colour behind each recorded position (the
// sum of the later segments over T: positive terms, no cancellation) and
// lists every whole segment below its last composited entry as a work
// item.  The backward's helper waves run those segments from the recorded
// state while one wave per quarter runs the rest of its list, so a long
// list is walked by several waves at once instead of by one wave long after
// the rest of the grid has finished.
constexpr int kCkSeg = 31;               // recorded positions per quarter (5 bits)
// Recorded states come from kPools pools of equal size; a quarter takes
// them from pool (its wave index mod kPools), so each slot counter is
// contended by few waves at a time.  A quarter whose pool is exhausted
// stops recording (the rest of its list stays one piece, walked by one
// wave: the heavy quarters, which reach their later boundaries last, are
// the ones refused).  Pools hold one state per quarter of the image (at
// least 64 each): lists of 1080p views split at 512 entries ask for about
// 0.45 per quarter, the busiest pool for 0.56.
constexpr int kPools = 64;
constexpr int kCounterWords = kPools * 32;   // two counters per pool, 128 bytes apart

// Sizes of the split state of one image.
struct SplitLayout {
  int64_t quarters;   // kWPT per tile
  int pool_slots;     // states per pool
  size_t bytes;       // the whole workspace
};

__host__ __device__ inline SplitLayout split_layout(int32_t width, int32_t height) {
  SplitLayout l;
  l.quarters = int64_t((width + kTile - 1) / kTile) * ((height + kTile - 1) / kTile) * kWPT;
  const int64_t per_pool = (l.quarters + kPools - 1) / kPools;
  l.pool_slots = int(per_pool < 64 ? 64 : per_pool);
  const size_t slots = size_t(kPools) * l.pool_slots;
  l.bytes = slots * 64 * 16 + 2 * slots * 4 + size_t(l.quarters) * 4 + kCounterWords * 4;
  return l;
}

// The workspace: states, their owners, the pools' work lists, per-quarter
// segment counts, and per pool the counters (slots taken, items listed).
struct SplitState {
  float4* ck;          // [slots][64]: (T, colour) per pixel
  uint32_t* owner;     // [slots]: quarter << 5 | position index
  uint32_t* items;     // [kPools][pool_slots]: slots whose segment the helpers run
  uint32_t* qsegs;     // [quarters]: segments of the quarter run by helpers
  uint32_t* counters;  // [kPools][32]
};

__host__ __device__ inline SplitState split_state(void* base, const SplitLayout& l) {
  const uintptr_t p = reinterpret_cast<uintptr_t>(base);   // base may be NULL (no split)
  const size_t slots = size_t(kPools) * l.pool_slots;
  SplitState s;
  s.ck = reinterpret_cast<float4*>(p);
  s.owner = reinterpret_cast<uint32_t*>(p + slots * 64 * 16);
  s.items = reinterpret_cast<uint32_t*>(p + slots * 64 * 16 + 4 * slots);
  s.qsegs = reinterpret_cast<uint32_t*>(p + slots * 64 * 16 + 8 * slots);
  s.counters = reinterpret_cast<uint32_t*>(p + slots * 64 * 16 + 8 * slots + 4 * size_t(l.quarters));
  return s;
}

// Workgroup -> (tile rank, quarter).  Workgroups go to the 8 XCDs round
// robin (workgroup b on XCD b mod 8), each XCD with its own L2; the four
// quarters of a rank are workgroups 32 g + x + 8 q (q = 0..3) of group g,
// all on XCD x, so one L2 serves the tile's list and records to its four
// waves, which start within a few workgroups of each other.
constexpr int kXcds = 8;
__host__ __device__ inline void quarter_of(int b, int& rank, int& q0) {
  const int g = b / (kWPT * kXcds), r = b % (kWPT * kXcds);
  rank = g * kXcds + r % kXcds;
  q0 = r / kXcds;
}

// Tiles are taken in `order` (longest lists first) when given, so the
// heavy ones start early and light ones fill the gaps.  Returns -1 for
// workgroups past the end.
__device__ __forceinline__ int order_tile(const uint32_t* __restrict__ order, int nT, int& q0) {
  int rank;
  quarter_of(int(blockIdx.x), rank, q0);
  if (rank >= nT) return -1;
  return order != nullptr ? int(order[rank]) : rank;
}

// Workgroups for nT tiles: whole groups of kXcds tiles.
inline unsigned raster_grid(int nT) { return unsigned((nT + kXcds - 1) / kXcds * kXcds * kWPT); }

// e^x for x in [-5.6, 0], the compositing weight's exponential: 2^t with
// t = x log2 e, t = k + f (k = rint(t), f = t - k exact), 2^f by a degree-5
// polynomial (near-minimax on [-1/2, 1/2] in relative error) with fmaf,
// then 2^k; within 6e-7 relative of e^x.  Ten instructions.
__device__ __forceinline__ float aexp(float x) {
  const float t = x * 1.44269504088896341f;
  const float kf = rintf(t);
  const float f = t - kf;
  float p = 0x1.5bb9e4p-10f;
  p = fmaf(p, f, 0x1.3cea7ap-7f);
  p = fmaf(p, f, 0x1.c6b752p-5f);
  p = fmaf(p, f, 0x1.ebf9bcp-3f);
  p = fmaf(p, f, 0x1.62e42ap-1f);
  p = fmaf(p, f, 1.0f);
  return ldexpf(p, static_cast<int>(kf));
}

// A chunk's Gaussians as the rasterisers read them from LDS, one 48-byte
// record per entry: a = (u, v, -A/2, -B), c = (opacity, r, g, b),
// d = (-C/2, Gaussian index bits).  A visit reads a and d.x for the
// exponent, then c: uniform LDS broadcasts from one address register (one
// base, immediate offsets).
struct LdsRec {
  float4 a, c;
  float2 d, pad;
};
struct LdsRecs {
  LdsRec r[kChunk];
};

// LDS addresses as 32-bit byte offsets.  Record reads and sum stores go
// through them so that an entry's address is one 32-bit add of a scalar
// offset (through a generic pointer the compiler formed it with a 64-bit
// multiply-add on every visit).
using LdsFloatL = __attribute__((address_space(3))) float;
typedef float F4v __attribute__((ext_vector_type(4)));
typedef float F2v __attribute__((ext_vector_type(2)));
using LdsF4L = __attribute__((address_space(3))) F4v;
using LdsF2L = __attribute__((address_space(3))) F2v;
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return uint32_t(uintptr_t((__attribute__((address_space(3))) const char*)p));
}
// base + off for a wave-uniform offset: the offset is kept in a scalar
// register, opaque to the compiler (which would otherwise fold a multiply
// into the add as that 64-bit multiply-add), so the sum is one vector add.
__device__ __forceinline__ uint32_t lds_add_uniform(uint32_t base, uint32_t off) {
  asm("" : "+s"(off));
  return base + off;
}
__device__ __forceinline__ float4 lds_load4(uint32_t a) {
  const auto v = *(LdsF4L*)uintptr_t(a);
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float2 lds_load2(uint32_t a) {
  const auto v = *(LdsF2L*)uintptr_t(a);
  return make_float2(v.x, v.y);
}
__device__ __forceinline__ float lds_load1(uint32_t a) { return *(LdsFloatL*)uintptr_t(a); }
__device__ __forceinline__ void lds_store1(uint32_t a, float x) { *(LdsFloatL*)uintptr_t(a) = x; }

// Any lane of the wave true (the predicate's ballot, tested in scalar
// registers).
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// One list entry's record as loaded from HBM: the first 11 words of the
// projected record (u, v, A, B | C, opacity, r, g | b, cull extent x, y)
// and the Gaussian's index (-1: no entry).
struct EntryRec {
  float4 q0, q1;
  float b, ex, ey;
  int32_t g;
};

__device__ __forceinline__ int32_t load_index(const int32_t* __restrict__ vals, uint32_t j, bool valid) {
  return valid ? vals[j] : -1;
}

__device__ __forceinline__ EntryRec load_entry(const float4* __restrict__ proj, int32_t g) {
  EntryRec r;
  r.g = g;
  if (g >= 0) {
    const float4* q = proj + 4 * int64_t(g);
    r.q0 = q[0];
    r.q1 = q[1];
    const float4 q2 = q[2];
    r.b = q2.x;
    r.ex = q2.y;
    r.ey = q2.z;
  } else {
    r.q0 = r.q1 = make_float4(0.f, 0.f, 0.f, 0.f);
    r.b = r.ex = r.ey = 0.f;
  }
  return r;
}

// The chunk is consumed while the next one is in flight: the records of
// chunk c + 1 and the list indices of chunk c + 2 are loaded before chunk c
// is staged, so the two dependent HBM round trips (index, then record) of
// a chunk overlap the compositing of the one before it.
//
// True when the Gaussian's alpha is provably below 1/255 at every point of
// the rectangle [x0, x1] x [y0, y1] of pixel centres, so no pixel there can
// composite it.  alpha = opacity * exp(-Q / 2) with Q(d) = d^T [A B; B C] d
// (d: pixel centre minus mean) falls below 1/255 exactly where
// Q > 2 ln(255 opacity).  Q is convex, so its minimum over the rectangle is
// 0 when the mean lies inside and otherwise lies on an edge, where the 1-D
// minimiser is the unconstrained one clamped to the edge.  The margin
// covers the rounding of this evaluation and of the rasteriser's own
// evaluation of Q at any pixel of the rectangle (both a few fp32 ulps of
// the term magnitudes, bounded by S below), and the hardware log2.
__device__ __forceinline__ bool ellipse_misses(float u, float v, float A, float B, float C, float opac, float x0,
                                               float x1, float y0, float y1) {
  if (!(A > 0.0f && C > 0.0f)) return false;
  const float dx0 = x0 - u, dx1 = x1 - u, dy0 = y0 - v, dy1 = y1 - v;
  if (dx0 <= 0.0f && dx1 >= 0.0f && dy0 <= 0.0f && dy1 >= 0.0f) return false;
  // (hardware reciprocals: a perturbed minimiser is still a point of the
  // edge, and Q grows only quadratically away from the true one)
  const float rc = B * __builtin_amdgcn_rcpf(C), ra = B * __builtin_amdgcn_rcpf(A);
  const auto quad = [&](float dx, float dy) { return fmaf(A * dx, dx, fmaf(2.0f * B * dx, dy, C * dy * dy)); };
  const float ey0 = fminf(fmaxf(-rc * dx0, dy0), dy1), ey1 = fminf(fmaxf(-rc * dx1, dy0), dy1);
  const float ex0 = fminf(fmaxf(-ra * dy0, dx0), dx1), ex1 = fminf(fmaxf(-ra * dy1, dx0), dx1);
  const float qmin = fminf(fminf(quad(dx0, ey0), quad(dx1, ey1)), fminf(quad(ex0, dy0), quad(ex1, dy1)));
  const float X = fmaxf(fabsf(dx0), fabsf(dx1)), Y = fmaxf(fabsf(dy0), fabsf(dy1));
  const float S = fmaf(A * X, X, fmaf(2.0f * fabsf(B) * X, Y, C * Y * Y));
  const float tau2 = 1.38629436f * __log2f(255.0f * opac);   // 2 ln(255 opacity)
  return qmin > tau2 + 1.0e-3f * fabsf(tau2) + 2.0e-3f + 1.0e-5f * S;
}

// A box of pixel centres [x0, x1] x [y0, y1].
struct PixBox {
  float x0, x1, y0, y1;
};
__device__ __forceinline__ PixBox quarter_box(float qx, float qy) { return {qx, qx + 7.0f, qy, qy + 7.0f}; }

// The box spanned by the rows and columns of a quarter's lanes in `live`
// (lane = 8 row + column; non-zero): an entry whose footprint misses it
// reaches none of those pixels.  `live` is wave-uniform, so the masks are
// scalar work.
__device__ __forceinline__ PixBox live_box(uint64_t live, float qx, float qy) {
  uint64_t c = live | (live >> 32);
  c |= c >> 16;
  c |= c >> 8;
  const uint32_t cols = uint32_t(c) & 0xFFu;
  uint32_t rows = 0;
#pragma unroll
  for (int r = 0; r < 8; ++r) rows |= ((live >> (8 * r)) & 0xFFu) != 0 ? (1u << r) : 0u;
  return {qx + float(__builtin_ctz(cols)), qx + float(31 - __builtin_clz(cols)), qy + float(__builtin_ctz(rows)),
          qy + float(31 - __builtin_clz(rows))};
}

// Stage a loaded entry (if any) into LDS record `lane` and return whether
// it can reach a pixel centre of the box (the wave's quarter, or the part
// of it whose pixels still composite): first the Gaussian's alpha >= 1/255
// box [u - ex, u + ex] x [v - ey, v + ey] against it, then (for finite
// boxes) the exact test of the footprint ellipse against it.
__device__ __forceinline__ bool stage_entry(const EntryRec& r, const PixBox& bx, LdsRecs& s_rec, int lane) {
  bool hit = false;
  if (r.g >= 0) {
    s_rec.r[lane].a = make_float4(r.q0.x, r.q0.y, -0.5f * r.q0.z, -r.q0.w);
    s_rec.r[lane].c = make_float4(r.q1.y, r.q1.z, r.q1.w, r.b);
    s_rec.r[lane].d = make_float2(-0.5f * r.q1.x, __builtin_bit_cast(float, r.g));
    const float u = r.q0.x, v = r.q0.y;
    hit = u + r.ex >= bx.x0 && u - r.ex <= bx.x1 && v + r.ey >= bx.y0 && v - r.ey <= bx.y1;
    if (hit && r.ex < 1.0e30f)
      hit = !ellipse_misses(u, v, r.q0.z, r.q0.w, r.q1.x, r.q1.y, bx.x0, bx.x1, bx.y0, bx.y1);
  }
  return hit;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) {
    const uint32_t o = uint32_t(__shfl_xor(int(v), d, 64));
    v = o > v ? o : v;
  }
  return v;
}

}  // namespace gs
