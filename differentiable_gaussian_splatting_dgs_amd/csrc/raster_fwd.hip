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
#include <algorithm>

#include "raster_common.hpp"

namespace gs {
namespace {

// Zeroes the per-tile maxima and the split state's counters.
__global__ __launch_bounds__(256) void k_clear(uint32_t* __restrict__ p, int n, uint32_t* __restrict__ counters) {
  const int i = int(blockIdx.x) * 256 + int(threadIdx.x);
  if (p != nullptr && i < n) p[i] = 0u;
  if (counters != nullptr && i < kCounterWords) counters[i] = 0u;
}

// Compositing state of a quarter's 64 pixels (one per lane).
struct FwdState {
  float T, C0, C1, C2;
  uint32_t lastp, read;
  uint64_t livem;           // lanes still compositing, as a wave mask (scalar registers)
  int nck;                  // states recorded
  uint32_t slotv;           // lane k: the slot of record k
  float U0, U1, U2;         // colour composited in the current segment
};

// The quarter's list [start, end) front to back until every pixel has
// stopped.  kRec: the list is longer than a segment and records its state
// at the segment boundaries it reaches (only then are the segment colours
// U summed: a list that records nothing leaves them unused).  kTiles: the
// list position where each pixel stopped is kept (per-tile processed
// counts).
template <bool kTiles, bool kRec>
__device__ __forceinline__ void fwd_list(const float4* __restrict__ proj, const int32_t* __restrict__ vals,
                                         uint32_t start, uint32_t end, float qx, float qy, float pxc, float pyc,
                                         const SplitLayout& sl, const SplitState& sp, uint32_t seg_mask,
                                         uint32_t qid, uint32_t pool, LdsRecs& s_rec, FwdState& st) {
  const int lane = threadIdx.x & 63;
  uint32_t* const pool_count = sp.counters + 32 * pool;   // slots taken, items listed
  bool ck_open = kRec;
  const uint32_t ul = uint32_t(lane);
  EntryRec cur = load_entry(proj, load_index(vals, start + ul, start + ul < end));
  int32_t gnext = load_index(vals, start + kChunk + ul, start + kChunk + ul < end);
  for (uint32_t cs = start; cs < end && st.livem != 0; cs += kChunk) {
    if (kRec && ck_open && cs != start && ((cs - start) & seg_mask) == 0) {
      uint32_t slot = 0;
      if (lane == 0) slot = atomicAdd(pool_count, 1u);
      slot = __builtin_amdgcn_readfirstlane(slot);
      if (slot < uint32_t(sl.pool_slots)) {
        slot += pool * uint32_t(sl.pool_slots);
        // T before entry cs - start, and the colour the segment now ending added
        sp.ck[size_t(slot) * 64 + lane] = make_float4(st.T, st.U0, st.U1, st.U2);
        if (lane == 0) sp.owner[slot] = (qid << 5) | uint32_t(st.nck);
        st.slotv = lane == st.nck ? slot : st.slotv;
        st.U0 = st.U1 = st.U2 = 0.0f;
        ++st.nck;
        ck_open = st.nck < kCkSeg;
      } else {
        ck_open = false;   // pool exhausted: the segments from here on stay one
      }
    }
    const EntryRec nxt = load_entry(proj, gnext);
    const uint32_t j2 = cs + 2 * kChunk + ul;
    gnext = load_index(vals, j2, j2 < end);
    // (against the box of the pixels still compositing: an entry outside
    // it would be skipped by every one of them)
    const bool hit = stage_entry(cur, live_box(st.livem, qx, qy), s_rec, lane);
    cur = nxt;
    uint64_t active = __ballot(hit);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint32_t pos0 = cs - start + 1;   // list position + 1 of the chunk's entry 0
    // Visits in order of the set bits.  The next visit's record is read from
    // LDS while the current one is composited, so the read's latency is off
    // the serial chain of the long quarters, which run with few waves
    // beside them at the kernel's end (unrolled by two: the two records
    // alternate between two register sets without copies).
    const auto visit = [&](int k, const float4& a, float hc, const float4& c) {
      const float dx = pxc - a.x, dy = pyc - a.y;
      const float power = fmaf(dx, fmaf(a.z, dx, a.w * dy), (hc * dy) * dy);
      // power < -5.6 gives alpha < e^-5.6 < 1/255 for any opacity <= 1.
      // (Decisions are kept as wave masks of direct comparisons, so none is
      // turned into a per-lane value and back.)
      const uint64_t okm = __builtin_amdgcn_ballot_w64(!(power > 0.0f)) &
                           __builtin_amdgcn_ballot_w64(!(power < -5.6f)) & st.livem;
      if (okm == 0) return;
      // c: opacity, r, g, b
      const float alpha = fminf(0.99f, c.x * aexp(power));
      const uint64_t okm2 = okm & __builtin_amdgcn_ballot_w64(!(alpha < 1.0f / 255.0f));
      const float nt = st.T * (1.0f - alpha);
      const uint64_t stopm = okm2 & __builtin_amdgcn_ballot_w64(nt < 0.0001f);
      const bool comp = __builtin_amdgcn_inverse_ballot_w64(okm2 & ~stopm);
      const uint32_t pos1 = pos0 + uint32_t(k);
      // a zero weight leaves the colour sums exactly as they are
      // (non-negative colours, sums from +0)
      const float wgt = comp ? alpha * st.T : 0.0f;
      st.C0 = fmaf(c.y, wgt, st.C0);
      st.C1 = fmaf(c.z, wgt, st.C1);
      st.C2 = fmaf(c.w, wgt, st.C2);
      if constexpr (kRec) {
        st.U0 = fmaf(c.y, wgt, st.U0);
        st.U1 = fmaf(c.z, wgt, st.U1);
        st.U2 = fmaf(c.w, wgt, st.U2);
      }
      st.T = comp ? nt : st.T;
      st.lastp = comp ? pos1 : st.lastp;
      if constexpr (kTiles) st.read = __builtin_amdgcn_inverse_ballot_w64(stopm) ? pos1 : st.read;
      st.livem &= ~stopm;
    };
    if (active != 0) {
      // record k at rb + 48 k: a (u, v, -A/2, -B) at +0, c at +16, -C/2 at +32
      const uint32_t rb = lds_addr(s_rec.r);
      int k = __builtin_ctzll(active);
      uint32_t ra = lds_add_uniform(rb, uint32_t(k) * uint32_t(sizeof(LdsRec)));
      float4 aa = lds_load4(ra), ca = lds_load4(ra + 16);
      float ha = lds_load1(ra + 32);
      for (;;) {
        active &= active - 1;
        const int kb = active != 0 ? __builtin_ctzll(active) : k;
        const uint32_t rbb = lds_add_uniform(rb, uint32_t(kb) * uint32_t(sizeof(LdsRec)));
        const float4 ab = lds_load4(rbb), cb = lds_load4(rbb + 16);
        const float hb = lds_load1(rbb + 32);
        visit(k, aa, ha, ca);
        if (active == 0) break;
        k = kb;
        active &= active - 1;
        const int ka = active != 0 ? __builtin_ctzll(active) : k;
        ra = lds_add_uniform(rb, uint32_t(ka) * uint32_t(sizeof(LdsRec)));
        aa = lds_load4(ra);
        ca = lds_load4(ra + 16);
        ha = lds_load1(ra + 32);
        visit(k, ab, hb, cb);
        if (active == 0) break;
        k = ka;
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// kTiles: the per-tile count of processed list entries is recorded (it
// needs the list position where each pixel stopped).
template <bool kTiles>
__global__ __launch_bounds__(64 * kWPT) void k_render_fwd(const float4* __restrict__ proj, const int32_t* __restrict__ vals,
                                                   const uint32_t* __restrict__ ranges,
                                                   const uint32_t* __restrict__ order, int64_t num_pairs, int W,
                                                   int H, int TX, int nT, float* __restrict__ image,
                                                   float* __restrict__ T_final, uint32_t* __restrict__ last,
                                                   uint32_t* __restrict__ tile_processed, void* split,
                                                   int seg_shift) {
  __shared__ LdsRecs s_recs[kWPT];
  // issue priority over waves of other kernels sharing the CU (the next
  // view's binning on the side stream): this kernel is issue-bound and on
  // the step's critical path
  __builtin_amdgcn_s_setprio(kRasterPrio);
  const int rank = int(blockIdx.x);
  if (rank >= nT) return;
  const int tile = order != nullptr ? int(order[rank]) : rank;
  const int q0 = int(threadIdx.x) >> 6;
  const int lane = int(threadIdx.x) & 63;
  LdsRecs& s_rec = s_recs[q0];
  const int tx = tile % TX, ty = tile / TX;
  const int x0 = tx * kTile, y0 = ty * kTile;
  const float qx = float(x0 + (q0 & 1) * 8) + 0.5f, qy = float(y0 + (q0 >> 1) * 8) + 0.5f;
  uint32_t start = ranges[2 * tile], end = ranges[2 * tile + 1];
  if (end > uint64_t(num_pairs)) end = uint32_t(num_pairs);
  if (start > end) start = end;

  const int px = x0 + (q0 & 1) * 8 + (lane & 7), py = y0 + (q0 >> 1) * 8 + (lane >> 3);
  const float pxc = float(px) + 0.5f, pyc = float(py) + 0.5f;
  const bool inside = px < W && py < H;
  FwdState st;
  st.T = 1.0f;
  st.C0 = st.C1 = st.C2 = 0.0f;
  st.lastp = 0;
  st.read = end - start;
  st.livem = __builtin_amdgcn_ballot_w64(inside);
  st.nck = 0;
  st.slotv = 0;
  st.U0 = st.U1 = st.U2 = 0.0f;

  // split backward: lists longer than a segment record their state at the
  // segment boundaries they reach; lane k keeps the slot of record k
  const SplitLayout sl = split_layout(W, H);
  const SplitState sp = split_state(split, sl);
  const uint32_t seg_mask = (1u << seg_shift) - 1u;
  const bool rec = split != nullptr && end - start > seg_mask + 1u;
  const uint32_t qid = uint32_t(tile) * kWPT + uint32_t(q0);
  const uint32_t pool = (blockIdx.x * kWPT + uint32_t(q0)) % kPools;
  if (rec)
    fwd_list<kTiles, true>(proj, vals, start, end, qx, qy, pxc, pyc, sl, sp, seg_mask, qid, pool, s_rec, st);
  else
    fwd_list<kTiles, false>(proj, vals, start, end, qx, qy, pxc, pyc, sl, sp, seg_mask, qid, pool, s_rec, st);

  if (inside) {
    const size_t P = size_t(W) * H;
    const size_t pix = size_t(py) * W + px;
    image[pix] = st.C0;
    image[P + pix] = st.C1;
    image[2 * P + pix] = st.C2;
    T_final[pix] = st.T;
    last[pix] = st.lastp;
  }
  if (kTiles) {
    const uint32_t rmax = wave_max_u32(inside ? st.read : 0u);
    if (lane == 0 && rmax != 0) atomicMax(tile_processed + tile, rmax);
  }
  if (split != nullptr) {
    const uint32_t slotv = st.slotv;
    const int nck = st.nck;
    float U0 = st.U0, U1 = st.U1, U2 = st.U2;
    // recorded segment colours -> the colour behind each boundary b: the
    // sum of the segments after it (positive terms, no cancellation) / T_b
    // (T_b >= 1e-4: a pixel stops before its transmittance drops below)
    // (loads issued four at a time, so the heaviest quarters, which record
    // the most, do not wait for one round trip per record at their end)
    for (int k0 = nck - 1; k0 >= 0; k0 -= 4) {
      float4 v[4];
      float4* p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = k0 - j >= 0 ? k0 - j : 0;
        p[j] = sp.ck + size_t(__builtin_amdgcn_readlane(slotv, k)) * 64 + lane;
        v[j] = *p[j];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (k0 - j >= 0) {
          *p[j] = make_float4(v[j].x, U0 / v[j].x, U1 / v[j].x, U2 / v[j].x);
          U0 += v[j].y;
          U1 += v[j].z;
          U2 += v[j].w;
        }
      }
    }
    // the whole segments below the last entry any pixel composited go to
    // the helpers; the quarter's own wave keeps the rest
    const uint32_t lmax = wave_max_u32(st.lastp);
    uint32_t nseg = lmax == 0 ? 0u : (lmax - 1) >> seg_shift;
    if (nseg > uint32_t(nck)) nseg = uint32_t(nck);
    if (lane == 0) sp.qsegs[qid] = nseg;
    if (nseg != 0) {
      uint32_t b = 0;
      if (lane == 0) b = atomicAdd(sp.counters + 32 * pool + 1, nseg);
      b = __builtin_amdgcn_readfirstlane(b);
      if (uint32_t(lane) < nseg) sp.items[pool * uint32_t(sl.pool_slots) + b + uint32_t(lane)] = slotv;
    }
  }
}

}  // namespace

size_t raster_split_bytes(int32_t width, int32_t height) { return split_layout(width, height).bytes; }

bool raster_split_fits(int32_t width, int32_t height) {
  return split_layout(width, height).quarters < (int64_t(1) << 27);   // quarter << 5 in 32 bits
}

hipError_t launch_render_fwd(const float* proj, const int32_t* vals, const uint32_t* ranges,
                             const uint32_t* tile_order, int64_t num_pairs, int32_t width, int32_t height,
                             float* image, float* T_final, uint32_t* last, uint32_t* tile_processed, void* split,
                             int seg_shift, hipStream_t st) {
  const int TX = (width + kTile - 1) / kTile, TY = (height + kTile - 1) / kTile;
  const int nT = TX * TY;
  if (split != nullptr && !raster_split_fits(width, height)) split = nullptr;
  uint32_t* const counters = split != nullptr ? split_state(split, split_layout(width, height)).counters : nullptr;
  if (tile_processed != nullptr || counters != nullptr)
    k_clear<<<unsigned(std::max(tile_processed != nullptr ? (nT + 255) / 256 : 0, kCounterWords / 256)), 256, 0, st>>>(
        tile_processed, nT, counters);
  if (tile_processed != nullptr)
    k_render_fwd<true><<<unsigned(nT), 64 * kWPT, 0, st>>>(reinterpret_cast<const float4*>(proj), vals, ranges, tile_order,
                                                      num_pairs, width, height, TX, nT, image, T_final, last,
                                                      tile_processed, split, seg_shift);
  else
    k_render_fwd<false><<<unsigned(nT), 64 * kWPT, 0, st>>>(reinterpret_cast<const float4*>(proj), vals, ranges,
                                                       tile_order, num_pairs, width, height, TX, nT, image, T_final,
                                                       last, nullptr, split, seg_shift);
  return hipGetLastError();
}

}  // namespace gs
