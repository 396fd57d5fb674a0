// Backward pass of one view (the "back-propagation" step of the Grendel-GS
// notes' training pipeline), in two kernels, one per entry point:
//
//  k_render_bwd  -- the forward's layout (waves owning 8x8 quarters of a
//    tile), reverse traversal of the tile's list from the last Gaussian
//    any pixel composited.  Each pixel rebuilds its
//    transmittance by division, T_i = T_{i+1} / (1 - alpha_i), carries the
//    suffix colour S (S_{i-1} = alpha_i c_i + (1 - alpha_i) S_i, S = 0 behind
//    the last one: black background), and forms
//      dL/dc_i = alpha_i T_i G,   dL/dalpha_i = T_i (c_i - S_i) . G,
//    then chains alpha = o e^power (unless clamped at 0.99) into the opacity,
//    the conic and the 2D mean.  Skip decisions are recomputed with the same
//    fp32 arithmetic as the forward, so exactly the composited set is
//    visited.  The nine partials of a Gaussian are summed over a lane's
//    pixels in registers, then over the wave by two lane-half swaps that fold
//    several values at once (permlane32/16 swap) and four DPP row steps
//    (to row totals), and parked in LDS; at the end of each chunk 16-lane
//    rows turn them into gradients and add them with nine global float
//    atomics per (Gaussian, wave), one coalesced request per Gaussian.
//
//  k_project_bwd -- one thread per visible Gaussian: the chain rule of the
//    projection from the screen-space gradients to all 59 parameters
//    (SH coefficients and view direction, EWA covariance, scale via exp,
//    rotation via the normalised quaternion, mean via the pinhole map),
//    accumulated (+=) into the [59][ld] gradient planes; the consumed
//    screen-space rows are zeroed so the buffer is clean for the next view.
#include "project_grad.hpp"
#include "raster_common.hpp"

namespace gs {
namespace {

constexpr int kG2 = 12;   // floats per Gaussian in the screen-gradient buffer
constexpr int kAcc = 9;   // LDS stride of a chunk entry's nine sums (odd: no bank conflicts)

__device__ __forceinline__ float f_of(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t u_of(float f) { return __builtin_bit_cast(uint32_t, f); }

// Lanes l and l ^ 32 summed: lanes 0-31 carry x's sums, lanes 32-63 y's.
__device__ __forceinline__ float fold32(float x, float y) {
  const auto s = __builtin_amdgcn_permlane32_swap(u_of(x), u_of(y), false, false);
  return f_of(s[0]) + f_of(s[1]);
}

// Within each half, rows (16 lanes) 0 and 1 summed: of x = [a | b] and
// y = [c | d] (halves), rows 0..3 of the result carry a, c, b, d.
__device__ __forceinline__ float fold16(float x, float y) {
  const auto s = __builtin_amdgcn_permlane16_swap(u_of(x), u_of(y), false, false);
  return f_of(s[0]) + f_of(s[1]);
}

// Sum over each 8-lane half of a row; every lane ends with its half's
// total (the two halves are added when the sums leave LDS).
__device__ __forceinline__ float half_row_sum(float v) {
  v += f_of(__builtin_amdgcn_update_dpp(0, u_of(v), 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v += f_of(__builtin_amdgcn_update_dpp(0, u_of(v), 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v += f_of(__builtin_amdgcn_update_dpp(0, u_of(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
  return v;
}

// The wave's total of v in lane 63 (other lanes: partial sums): half-row
// sums, row sums (mirror), then each row adds the last lane of the row
// before it (row_bcast:15: row 3 holds rows 2 + 3, lane 31 rows 0 + 1),
// and rows 2 and 3 add lane 31 (row_bcast:31).  (Every row takes part in
// the two broadcasts, so each is one fused add; what rows 0 and 1 end with
// is not used.)
__device__ __forceinline__ float wave_total_lane63(float v) {
  v = half_row_sum(v);
  v += f_of(__builtin_amdgcn_update_dpp(0, u_of(v), 0x140, 0xF, 0xF, false));   // row_mirror
  v += f_of(__builtin_amdgcn_update_dpp(0, u_of(v), 0x142, 0xF, 0xF, false));   // row_bcast:15
  v += f_of(__builtin_amdgcn_update_dpp(0, u_of(v), 0x143, 0xF, 0xF, false));   // row_bcast:31
  return v;
}

// Sum over each 16-lane row; every lane ends with its row's total.
__device__ __forceinline__ float row_sum(float v) {
  v = half_row_sum(v);
  return v + f_of(__builtin_amdgcn_update_dpp(0, u_of(v), 0x140, 0xF, 0xF, false));   // row_mirror
}

// Sums of nine per-lane values over the wave.  The first eight are folded
// so each fold serves several values: rows 0..3 of q0 end with the totals
// of v0, v2, v1, v3, of q1 with those of v4, v6, v5, v7.  The ninth has no
// partner and takes the plain DPP reduction (six steps, against two folds
// with a zero register plus four steps).
__device__ __forceinline__ void wave_sum9(const float v[9], float& q0, float& q1, float& q2) {
  const float r0 = fold32(v[0], v[1]), r1 = fold32(v[2], v[3]), r2 = fold32(v[4], v[5]);
  const float r3 = fold32(v[6], v[7]);
  q0 = row_sum(fold16(r0, r1));
  q1 = row_sum(fold16(r2, r3));
  q2 = wave_total_lane63(v[8]);
}

// One pass of a quarter's list positions [lo, hi), back to front, from the
// per-pixel state (T, S) at position hi.  With kCount, nvis counts the
// lane's pixel-entry pairs that composited (the steps back-propagated).
template <bool kCount>
__device__ __forceinline__ void bwd_range(const float4* __restrict__ proj, const int32_t* __restrict__ vals,
                                          uint32_t start, uint32_t lo, uint32_t hi, float qx, float qy, float pxc,
                                          float pyc, uint32_t lastp, float T, float S0, float S1, float S2,
                                          float G0, float G1, float G2, float* __restrict__ grad2d,
                                          uint8_t* __restrict__ touched, LdsRecs& s_rec, float* s_acc,
                                          uint32_t& nvis) {
  const int lane = threadIdx.x;
  // lanes 0, 16, 32, 48 (row r = lane / 16) store the row totals: row r of
  // the folded sums q0 / q1 carries sum (0, 2, 1, 3)[r] / (4, 6, 5, 7)[r],
  // sum j sits at j of the entry's slot; lane 63 stores sum 8.  (Nine words
  // per entry, not two half sums each: the smaller LDS footprint admits
  // more waves per CU.)
  const int row = lane >> 4;
  const int comp0 = ((row & 1) << 1) | (row >> 1);
  const uint32_t acc_lane = lds_addr(s_acc) + 4u * uint32_t(comp0);   // word comp0 of entry 0
  // flush: lane (lane & 15) = c of its row writes gradient c; fk is its
  // factor for c >= 2 (conic A, B, C: -1/2, -1, -1/2; the rest 1)
  const int fc = lane & 15;
  const float fk = (fc == 2 || fc == 4) ? -0.5f : (fc == 3 ? -1.0f : 1.0f);
  const int64_t base = int64_t(start) + lo;    // first position of the range

  // chunks from the range's last entry down to its first (every chunk
  // below the first one processed lies wholly inside the composited
  // prefix; entries are loaded one chunk ahead, indices two)
  const uint32_t ul = uint32_t(lane);
  const int64_t top = int64_t(start) + int64_t((hi - 1) / kChunk) * kChunk;
  EntryRec cur = load_entry(proj, load_index(vals, uint32_t(top) + ul, uint32_t(top) + ul - start < hi));
  int32_t gnext = load_index(vals, uint32_t(top - kChunk) + ul, top - kChunk >= base);
  for (int64_t cs = top; cs >= base; cs -= kChunk) {
    uint64_t written = 0;   // chunk entries with sums in s_acc
    const EntryRec nxt = load_entry(proj, gnext);
    gnext = load_index(vals, uint32_t(cs - 2 * kChunk) + ul, cs - 2 * kChunk >= base);
    const uint32_t pos = uint32_t(cs) + ul - start;
    const uint32_t pos0 = uint32_t(cs) - start;
    // chunk entry k lies before the lane's last composited one when k < klim
    // (list positions < 2^31); entries are staged against the box of the
    // pixels with klim > 0, the only ones that take any entry of the chunk
    const int32_t klim = int32_t(lastp) - int32_t(pos0);
    const uint64_t live = __builtin_amdgcn_ballot_w64(klim > 0);
    const bool hit = stage_entry(cur, live != 0 ? live_box(live, qx, qy) : quarter_box(qx, qy), s_rec, lane);
    cur = nxt;
    uint64_t active = uint64_t(__ballot(hit && pos < hi));
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    while (active != 0) {
      const int k = 63 - __builtin_clzll(active);      // back to front
      active &= ~(1ull << k);
      const float4 a = s_rec.r[k].a;
      const float hc = s_rec.r[k].d.x;
      const float dx = pxc - a.x, dy = pyc - a.y;
      const float power = fmaf(dx, fmaf(a.z, dx, a.w * dy), (hc * dy) * dy);
      bool ok = k < klim && !(power > 0.0f) && !(power < -5.6f);
      if (!wave_any(ok)) continue;
      const float4 c = s_rec.r[k].c;   // opacity, r, g, b
      const float e = aexp(power);
      const float araw = c.x * e;
      const float alpha = fminf(0.99f, araw);
      ok = ok && !(alpha < 1.0f / 255.0f);
      if constexpr (kCount) nvis += ok ? 1u : 0u;
      // same decisions as the forward: `ok` = this pixel composited it.  A
      // lane that did not takes alpha 0: 1 - 0 = 1 has an exact hardware
      // reciprocal, T * 1 = T and fma(0, c, 1 * S) = S (colours and S are
      // finite and >= 0), so its T and S pass through bit for bit, as a
      // select would keep them, and its weight is 0
      const float a_ok = ok ? alpha : 0.0f;
      const float om = 1.0f - a_ok;
      const float Ti = T * __builtin_amdgcn_rcpf(om);
      const float wgt = a_ok * Ti;
      const float dal = Ti * fmaf(c.w - S2, G2, fmaf(c.z - S1, G1, (c.y - S0) * G0));
      S0 = fmaf(a_ok, c.y, om * S0);
      S1 = fmaf(a_ok, c.z, om * S1);
      S2 = fmaf(a_ok, c.w, om * S2);
      T = Ti;
      // the 0.99 clamp passes no gradient
      const float dl = (ok && !(araw > 0.99f)) ? dal : 0.0f;
      const float dp = dl * alpha;
      // per-lane terms of the nine sums: the 2D mean and conic gradients
      // are carried as sums of dp (dx, dy) and dp (dx^2, dx dy, dy^2) and
      // turned into gradients once per entry
      const float sx = dp * dx, sy = dp * dy;
      const float v9[9] = {sx, sy, sx * dx, sx * dy, sy * dy, dl * e, wgt * G0, wgt * G1, wgt * G2};
      float q0s, q1s, q2s;
      wave_sum9(v9, q0s, q1s, q2s);
      // keeps the last DPP step's adds out of the store branch below, where
      // they could not fuse with their DPP moves
      asm volatile("" : "+v"(q0s), "+v"(q1s), "+v"(q2s));
      if ((lane & 15) == 0) {
        const uint32_t acc = lds_add_uniform(acc_lane, uint32_t(k) * uint32_t(kAcc * 4));
        lds_store1(acc, q0s);
        lds_store1(acc + 16, q1s);
      }
      if (lane == 63) s_acc[k * kAcc + 8] = q2s;
      written |= 1ull << k;
    }
    // the chunk's entries leave four at a time, one 16-lane row each (lane
    // c < 9 of the row: gradient c), so a Gaussian's nine atomics go out as
    // one request: u = A sx + B sy, v = C sy + B sx, conic -sxx / 2, -sxy,
    // -syy / 2; opacity and colour as summed
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    while (written != 0) {
      int ks[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ks[r] = written != 0 ? __builtin_ctzll(written) : -1;
        written &= written - 1;
      }
      const int kk = row == 0 ? ks[0] : (row == 1 ? ks[1] : (row == 2 ? ks[2] : ks[3]));
      if (kk >= 0 && fc < 9) {
        // (the offsets as 24-bit multiplies: kk < 64)
        const uint32_t acc = lds_addr(s_acc) + __umul24(uint32_t(kk), uint32_t(kAcc * 4));
        const uint32_t rk = lds_addr(s_rec.r) + __umul24(uint32_t(kk), uint32_t(sizeof(LdsRec)));
        const float x = lds_load1(acc + 4 * fc);
        const float4 a = lds_load4(rk);
        const float2 d = lds_load2(rk + 32);   // -C/2, index bits
        const float m1 = fc == 0 ? -2.0f * a.z : (fc == 1 ? -2.0f * d.x : fk);
        // the mean gradients also take the other mean sum (lanes 0 and 1)
        const float gval = fc < 2 ? fmaf(m1, x, -a.w * lds_load1(acc + 4 * (fc ^ 1))) : m1 * x;
        const int32_t gi = __builtin_bit_cast(int32_t, d.y);
        if (gval != 0.0f) unsafeAtomicAdd(grad2d + size_t(gi) * kG2 + fc, gval);
        // the row's byte in the touched map: every row with a non-zero word
        // has it set (any flushed entry marks its row)
        if (touched != nullptr && fc == 0) touched[size_t(gi) * kTouchedStride] = 1;
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Workgroups [0, nhelp) are helpers: helper h takes the forward's listed
// segments h / kPools, h / kPools + nhelp / kPools, ... of pool h % kPools
// (nhelp = kPools x half the pool size: a pool's items rarely exceed
// that), each from its recorded state; the rest own one quarter each (in
// `order`) and run its list from the last composited entry down to the
// first position no helper covers.
template <bool kCount>
__global__ __launch_bounds__(64) void k_render_bwd(const float4* __restrict__ proj, const int32_t* __restrict__ vals,
                                                   const uint32_t* __restrict__ ranges,
                                                   const uint32_t* __restrict__ order, int64_t num_pairs, int W,
                                                   int H, int TX, int nT, const float* __restrict__ T_final,
                                                   const uint32_t* __restrict__ last,
                                                   const float* __restrict__ dL_dimage, float* __restrict__ grad2d,
                                                   uint8_t* __restrict__ touched, const void* split, int seg_shift,
                                                   int nhelp, unsigned long long* __restrict__ visits) {
  __shared__ LdsRecs s_rec;
  __shared__ float s_acc[kChunk * kAcc];   // a chunk's nine wave sums per entry
  __builtin_amdgcn_s_setprio(kRasterPrio);   // (as the forward)
  const SplitLayout sl = split_layout(W, H);
  const SplitState sp = split_state(const_cast<void*>(split), sl);
  const int lane = threadIdx.x;
  const size_t P = size_t(W) * H;
  const bool helper = int(blockIdx.x) < nhelp;
  const uint32_t pool = blockIdx.x % kPools;
  uint32_t nitems = 0;
  if (helper) {
    nitems = sp.counters[32 * pool + 1];
    if (nitems > uint32_t(sl.pool_slots)) nitems = uint32_t(sl.pool_slots);
  }
  uint32_t nvis = 0;
  for (uint32_t item = blockIdx.x / kPools;; item += uint32_t(nhelp / kPools)) {
    int tile, q0;
    uint32_t lo, seg_hi = 0, slot = 0;
    if (helper) {
      if (item >= nitems) break;
      slot = sp.items[pool * uint32_t(sl.pool_slots) + item];
      if (slot >= uint32_t(kPools * sl.pool_slots)) break;
      const uint32_t own = sp.owner[slot];
      tile = int(own >> 7);
      q0 = int(own >> 5) & 3;
      lo = (own & 31u) << seg_shift;
      seg_hi = lo + (1u << seg_shift);
    } else {
      int rank;
      quarter_of(int(blockIdx.x) - nhelp, rank, q0);   // nhelp: a multiple of kXcds
      if (rank >= nT) break;
      tile = order != nullptr ? int(order[rank]) : rank;
      lo = split != nullptr ? sp.qsegs[tile * kWPT + q0] << seg_shift : 0u;
    }
    if (tile >= nT) break;
    const int tx = tile % TX, ty = tile / TX;
    const int x0 = tx * kTile, y0 = ty * kTile;
    const float qx = float(x0 + (q0 & 1) * 8) + 0.5f, qy = float(y0 + (q0 >> 1) * 8) + 0.5f;
    uint32_t start = ranges[2 * tile], end = ranges[2 * tile + 1];
    if (end > uint64_t(num_pairs)) end = uint32_t(num_pairs);
    if (start > end) start = end;
    const int px = x0 + (q0 & 1) * 8 + (lane & 7), py = y0 + (q0 >> 1) * 8 + (lane >> 3);
    const bool inside = px < W && py < H;
    const size_t pix = size_t(py) * W + px;
    const uint32_t lastp = inside ? last[pix] : 0u;
    uint32_t lmax = wave_max_u32(lastp);     // entries a pixel of the quarter composited
    if (lmax > end - start) lmax = end - start;
    // a helper's segment ends where the next one's recorded state starts;
    // the quarter's own pass starts from T_final and black behind
    const uint32_t hi = helper ? (seg_hi < lmax ? seg_hi : lmax) : lmax;
    if (lo < hi) {
      float T, S0, S1, S2;
      if (helper) {
        const float4 v = sp.ck[size_t(slot) * 64 + lane];
        T = v.x;
        S0 = v.y;
        S1 = v.z;
        S2 = v.w;
      } else {
        T = inside ? T_final[pix] : 1.0f;
        S0 = S1 = S2 = 0.0f;
      }
      const float G0 = inside ? dL_dimage[pix] : 0.0f;
      const float G1 = inside ? dL_dimage[P + pix] : 0.0f;
      const float G2 = inside ? dL_dimage[2 * P + pix] : 0.0f;
      bwd_range<kCount>(proj, vals, start, lo, hi, qx, qy, float(px) + 0.5f, float(py) + 0.5f, lastp, T, S0, S1, S2,
                        G0, G1, G2, grad2d, touched, s_rec, s_acc, nvis);
    }
    if (!helper) break;
  }
  if constexpr (kCount) {
    // (every exit above is taken by the whole wave)
    uint32_t c = nvis;
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) c += uint32_t(__shfl_xor(int(c), d, 64));
    if (lane == 0 && c != 0) atomicAdd(visits, static_cast<unsigned long long>(c));
  }
}

__global__ __launch_bounds__(256) void k_project_bwd(const float* __restrict__ params, int64_t n, int64_t ld,
                                                     CamArgs cam, const int32_t* __restrict__ vis,
                                                     const int64_t* __restrict__ vis_count,
                                                     float4* __restrict__ grad2d, float* __restrict__ grads) {
  const int64_t r = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (r >= *vis_count) return;
  const int64_t i = vis[r];
  const float4 ga4 = grad2d[3 * i], gb4 = grad2d[3 * i + 1], gc4 = grad2d[3 * i + 2];
  const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
  grad2d[3 * i] = z4;            // consumed: the buffer is zero again for the next view
  grad2d[3 * i + 1] = z4;
  grad2d[3 * i + 2] = z4;
  const uint32_t off4 = uint32_t(i) << 2;
  float p[59];
#pragma unroll
  for (int k = 0; k < 59; ++k) p[k] = *plane_elem(params, ld, k, off4);
  const float grgb[3] = {gb4.z, gb4.w, gc4.x};
  float g[59];
  project_grads(p, cam, ga4.x, ga4.y, ga4.z, ga4.w, gb4.x, gb4.y, grgb, g);
#pragma unroll
  for (int k = 0; k < 59; ++k) *plane_elem(grads, ld, k, off4) += g[k];
}

}  // namespace

hipError_t launch_render_bwd(const float* proj, const int32_t* vals, const uint32_t* ranges,
                             const uint32_t* tile_order, int64_t num_pairs, int32_t width, int32_t height,
                             const float* T_final, const uint32_t* last, const float* dL_dimage, float* grad2d,
                             uint8_t* touched, const void* split, int seg_shift, uint64_t* visits, hipStream_t st) {
  const int TX = (width + kTile - 1) / kTile, TY = (height + kTile - 1) / kTile;
  const int nT = TX * TY;
  if (split != nullptr && !raster_split_fits(width, height)) split = nullptr;
  // a helper per two recorded states the pools can hold (a multiple of
  // kXcds, so the quarters' workgroups keep their XCD mapping)
  const int nhelp = split != nullptr ? kPools * ((split_layout(width, height).pool_slots + 1) / 2) : 0;
  const unsigned grid = unsigned(nhelp) + raster_grid(nT);
  unsigned long long* const vc = reinterpret_cast<unsigned long long*>(visits);
  if (visits != nullptr)
    k_render_bwd<true><<<grid, 64, 0, st>>>(reinterpret_cast<const float4*>(proj), vals, ranges, tile_order, num_pairs,
                                            width, height, TX, nT, T_final, last, dL_dimage, grad2d, touched, split,
                                            seg_shift, nhelp, vc);
  else
    k_render_bwd<false><<<grid, 64, 0, st>>>(reinterpret_cast<const float4*>(proj), vals, ranges, tile_order,
                                             num_pairs, width, height, TX, nT, T_final, last, dL_dimage, grad2d,
                                             touched, split, seg_shift, nhelp, nullptr);
  return hipGetLastError();
}

hipError_t launch_project_bwd(const float* params, int64_t n, int64_t ld, const CamArgs& cam,
                              const int32_t* vis_idx, const int64_t* vis_count, float* grad2d, float* grads,
                              hipStream_t st) {
  if (n == 0) return hipSuccess;
  k_project_bwd<<<unsigned((n + 255) / 256), 256, 0, st>>>(params, n, ld, cam, vis_idx, vis_count,
                                                           reinterpret_cast<float4*>(grad2d), grads);
  return hipGetLastError();
}

}  // namespace gs
