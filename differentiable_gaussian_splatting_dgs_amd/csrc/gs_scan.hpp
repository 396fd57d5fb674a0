// Block-level scan helpers for wave64 workgroups.
#pragma once

#include "gs_device.hpp"

namespace gs {

// Inclusive prefix sum over the 64 lanes of a wave.
template <class T>
__device__ __forceinline__ T wave_inclusive_scan(T v) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const T o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// Exclusive prefix sum over a block of NT threads (NT a multiple of 64,
// at most 1024); `total` receives the block sum.  `sh` must hold NT/64
// elements.  Contains __syncthreads.
template <int NT, class T>
__device__ __forceinline__ T block_exclusive_scan(T v, T* sh, T& total) {
  constexpr int NW = NT / 64;
  const int lane = lane_id();
  const int w = threadIdx.x >> 6;
  const T inc = wave_inclusive_scan(v);
  if (lane == 63) sh[w] = inc;
  __syncthreads();
  T base = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    const T s = sh[k];
    base += (k < w) ? s : T(0);
    tot += s;
  }
  __syncthreads();
  total = tot;
  return base + inc - v;
}

}  // namespace gs
