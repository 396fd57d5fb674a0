// Stream compaction of a byte-flag array into the ascending list of set
// indices: the per-view visible-index list and the batch union list (the
// Odin summary page, "Background and motivation": a view reads and writes
// only a sparse, view-dependent set of primitive indices).
//
// Reduce-then-scan, three launches: per-block counts, one-block scan of the
// counts, per-block write.  No inter-workgroup waiting.
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

// One block of 1024 threads scans nb counts in place (exclusive) and writes
// the total.
__global__ __launch_bounds__(1024) void k_scan_counts(int32_t* __restrict__ counts, int nb,
                                                       int64_t* __restrict__ total_out) {
  __shared__ int64_t sh[16];
  __shared__ int64_t carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < nb; base += 1024) {
    const int i = base + int(threadIdx.x);
    const int64_t v = i < nb ? counts[i] : 0;
    int64_t tot;
    const int64_t ex = block_exclusive_scan<1024, int64_t>(v, sh, tot);
    if (i < nb) counts[i] = int32_t(carry + ex);
    __syncthreads();
    if (threadIdx.x == 0) carry += tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) *total_out = carry;
}

__global__ __launch_bounds__(kCT) void k_write(uint8_t* __restrict__ flags, int64_t n,
                                               const int32_t* __restrict__ block_offsets,
                                               int32_t* __restrict__ idx, int clear) {
  __shared__ int sh[kCT / 64];
  const int64_t start = int64_t(blockIdx.x) * kCB + int64_t(threadIdx.x) * kCI;
  uint8_t f[kCI];
  const int c = load_flags(flags, n, start, f);
  int total;
  int off = block_exclusive_scan<kCT>(c, sh, total) + block_offsets[blockIdx.x];
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
  if (nb == 0) {
    k_scan_counts<<<1, 1024, 0, st>>>(counts, 0, count);
    return hipGetLastError();
  }
  k_count<<<dim3(unsigned(nb)), kCT, 0, st>>>(flags, n, counts);
  k_scan_counts<<<1, 1024, 0, st>>>(counts, int(nb), count);
  k_write<<<dim3(unsigned(nb)), kCT, 0, st>>>(flags, n, counts, idx, clear_flags ? 1 : 0);
  return hipGetLastError();
}

}  // namespace gs
