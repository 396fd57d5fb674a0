// Stream compaction of a byte-flag array into the ascending list of set
// indices: the per-view visible-index list and the batch union list (the
// Odin summary page, "Background and motivation": a view reads and writes
// only a sparse, view-dependent set of primitive indices).
//
// Reduce-then-scan in two launches: per-block counts, then a per-block
// write whose offset is the sum of the counts before the block (each block
// adds them itself; the last one also writes the total).  No
// inter-workgroup waiting.
#include "gs_scan.hpp"

namespace gs {
namespace {

constexpr int kCT = 256;          // threads per block
constexpr int kCI = 16;           // flags per thread (one uint4 load)
constexpr int kCB = kCT * kCI;    // flags per block

__device__ __forceinline__ int load_flags(const uint8_t* flags, int64_t n, int64_t start, uint8_t f[kCI]) {
  int c = 0;
  if (start + kCI <= n) {
    const uint4 q = *reinterpret_cast<const uint4*>(flags + start);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int k = 0; k < kCI; ++k) {
      f[k] = (w[k >> 2] >> (8 * (k & 3))) & 0xFFu;
      c += f[k] != 0;
    }
  } else {
#pragma unroll
    for (int k = 0; k < kCI; ++k) {
      f[k] = (start + k < n) ? flags[start + k] : 0;
      c += f[k] != 0;
    }
  }
  return c;
}

__global__ __launch_bounds__(kCT) void k_count(const uint8_t* __restrict__ flags, int64_t n,
                                               int32_t* __restrict__ block_counts) {
  __shared__ int sh[kCT / 64];
  const int64_t start = int64_t(blockIdx.x) * kCB + int64_t(threadIdx.x) * kCI;
  uint8_t f[kCI];
  const int c = load_flags(flags, n, start, f);
  int total;
  block_exclusive_scan<kCT>(c, sh, total);
  if (threadIdx.x == 0) block_counts[blockIdx.x] = total;
}

// Grid: max(1, blocks) workgroups; the last writes the total count.
__global__ __launch_bounds__(kCT) void k_write(uint8_t* __restrict__ flags, int64_t n,
                                               const int32_t* __restrict__ block_counts,
                                               int32_t* __restrict__ idx, int64_t* __restrict__ total_out,
                                               int clear) {
  __shared__ int sh[kCT / 64];
  __shared__ int64_t sh64[kCT / 64];
  const int64_t start = int64_t(blockIdx.x) * kCB + int64_t(threadIdx.x) * kCI;
  // the counts of the blocks before this one
  int64_t before = 0;
  for (int j = int(threadIdx.x); j < int(blockIdx.x); j += kCT) before += block_counts[j];
  uint8_t f[kCI];
  const int c = load_flags(flags, n, start, f);
  int64_t base;
  block_exclusive_scan<kCT, int64_t>(before, sh64, base);
  int total;
  int off = block_exclusive_scan<kCT>(c, sh, total) + int(base);
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) *total_out = base + total;
#pragma unroll
  for (int k = 0; k < kCI; ++k)
    if (f[k]) idx[off++] = int32_t(start + k);
  if (clear) {
    if (start + kCI <= n) {
      *reinterpret_cast<uint4*>(flags + start) = make_uint4(0, 0, 0, 0);
    } else {
      for (int k = 0; k < kCI; ++k)
        if (start + k < n) flags[start + k] = 0;
    }
  }
}

}  // namespace

size_t compact_ws_bytes(int64_t n) {
  const int64_t nb = (n + kCB - 1) / kCB;
  return align_up(size_t(nb + 1) * sizeof(int32_t), 256);
}

hipError_t launch_compact(uint8_t* flags, int64_t n, int32_t* idx, int64_t* count, bool clear_flags,
                          void* ws, hipStream_t st) {
  const int64_t nb = (n + kCB - 1) / kCB;
  int32_t* counts = static_cast<int32_t*>(ws);
  if (nb > 0) k_count<<<dim3(unsigned(nb)), kCT, 0, st>>>(flags, n, counts);
  k_write<<<dim3(unsigned(nb > 0 ? nb : 1)), kCT, 0, st>>>(flags, n, counts, idx, count, clear_flags ? 1 : 0);
  return hipGetLastError();
}

}  // namespace gs
