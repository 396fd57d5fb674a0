// Sparse Adam over the union of the batch's visible sets (Odin summary page,
// "Background and motivation": a view updates only the primitives it
// touched; Grendel-GS notes, "Hyper-parameter scaling rule": lr * sqrt(b),
// beta^b for a batch of b views -- the caller passes the scaled values and
// the bias corrections 1 - beta^t).
//
// One thread per listed row; it walks the 59 parameter planes, so every
// plane access is coalesced across the wave (the list is ascending).  The
// consumed gradient is zeroed for the next step.  Rows not in the list are
// never touched.
#include "project_grad.hpp"

namespace gs {
namespace {

__global__ __launch_bounds__(256) void k_adam(float* __restrict__ params, float* __restrict__ grads,
                                              float* __restrict__ m, float* __restrict__ v, int64_t ld,
                                              const int32_t* __restrict__ rows, const int64_t* __restrict__ row_count,
                                              float lr, float b1, float b2, float eps, float bc1, float bc2) {
  const int64_t s = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (s >= *row_count) return;
  const int64_t i = rows[s];
  const float ob1 = 1.0f - b1, ob2 = 1.0f - b2;
  const float ibc1 = 1.0f / bc1, ibc2 = 1.0f / bc2;
#pragma unroll 4
  for (int k = 0; k < 59; ++k) {
    const int64_t q = int64_t(k) * ld + i;
    const float g = grads[q];
    const float mn = fmaf(b1, m[q], ob1 * g);
    const float vn = fmaf(b2, v[q], ob2 * g * g);
    m[q] = mn;
    v[q] = vn;
    params[q] -= lr * (mn * ibc1) / (sqrtf(vn * ibc2) + eps);
    grads[q] = 0.0f;
  }
}

// The batch's last view's projection backward fused with the Adam step,
// one thread per listed row: a row the last view saw (its projected record
// has tiles) adds that view's parameter gradients, chained from its
// screen-space gradients (which it re-zeroes), to the accumulated ones;
// then Adam as k_adam.  The same arithmetic as the two steps one after
// the other, without writing and re-reading the gradient planes.
__global__ __launch_bounds__(256) void k_project_adam(float* __restrict__ params, float* __restrict__ grads,
                                                      float* __restrict__ m, float* __restrict__ v, int64_t ld,
                                                      CamArgs cam, const float4* __restrict__ proj,
                                                      float4* __restrict__ grad2d, const int32_t* __restrict__ rows,
                                                      const int64_t* __restrict__ row_count, float lr, float b1,
                                                      float b2, float eps, float bc1, float bc2) {
  const int64_t s = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (s >= *row_count) return;
  const int64_t i = rows[s];
  float p[59], g[59];
#pragma unroll
  for (int k = 0; k < 59; ++k) p[k] = params[int64_t(k) * ld + i];
  if (__builtin_bit_cast(uint32_t, proj[4 * i + 3].w) != 0u) {
    const float4 ga4 = grad2d[3 * i], gb4 = grad2d[3 * i + 1], gc4 = grad2d[3 * i + 2];
    const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
    grad2d[3 * i] = z4;
    grad2d[3 * i + 1] = z4;
    grad2d[3 * i + 2] = z4;
    const float grgb[3] = {gb4.z, gb4.w, gc4.x};
    project_grads(p, cam, ga4.x, ga4.y, ga4.z, ga4.w, gb4.x, gb4.y, grgb, g);
#pragma unroll
    for (int k = 0; k < 59; ++k) g[k] += grads[int64_t(k) * ld + i];
  } else {
#pragma unroll
    for (int k = 0; k < 59; ++k) g[k] = grads[int64_t(k) * ld + i];
  }
  const float ob1 = 1.0f - b1, ob2 = 1.0f - b2;
  const float ibc1 = 1.0f / bc1, ibc2 = 1.0f / bc2;
#pragma unroll 4
  for (int k = 0; k < 59; ++k) {
    const int64_t q = int64_t(k) * ld + i;
    const float mn = fmaf(b1, m[q], ob1 * g[k]);
    const float vn = fmaf(b2, v[q], ob2 * g[k] * g[k]);
    m[q] = mn;
    v[q] = vn;
    params[q] = p[k] - lr * (mn * ibc1) / (sqrtf(vn * ibc2) + eps);
    grads[q] = 0.0f;
  }
}

}  // namespace

hipError_t launch_project_adam(float* params, float* grads, float* m, float* v, int64_t n, int64_t ld,
                               const CamArgs& cam, const float* proj, float* grad2d, const int32_t* rows,
                               const int64_t* row_count, float lr, float beta1, float beta2, float eps, float bc1,
                               float bc2, hipStream_t st) {
  if (n == 0) return hipSuccess;
  k_project_adam<<<unsigned((n + 255) / 256), 256, 0, st>>>(params, grads, m, v, ld, cam,
                                                            reinterpret_cast<const float4*>(proj),
                                                            reinterpret_cast<float4*>(grad2d), rows, row_count, lr,
                                                            beta1, beta2, eps, bc1, bc2);
  return hipGetLastError();
}

hipError_t launch_sparse_adam(float* params, float* grads, float* m, float* v, int64_t n, int64_t ld,
                              const int32_t* rows, const int64_t* row_count, float lr, float beta1,
                              float beta2, float eps, float bc1, float bc2, hipStream_t st) {
  if (n == 0) return hipSuccess;
  k_adam<<<unsigned((n + 255) / 256), 256, 0, st>>>(params, grads, m, v, ld, rows, row_count, lr, beta1, beta2, eps,
                                                    bc1, bc2);
  return hipGetLastError();
}

}  // namespace gs
