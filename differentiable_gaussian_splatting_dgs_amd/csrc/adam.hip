// Sparse Adam over the union of the batch's visible sets (Odin summary page,
// "Background and motivation": a view updates only the primitives it
// touched; Grendel-GS notes, "Hyper-parameter scaling rule": lr * sqrt(b),
// beta^b for a batch of b views -- the caller passes the scaled values and
// the bias corrections 1 - beta^t).
//
// One thread per listed row; it walks the 59 parameter planes, so every
// plane access is coalesced across the wave (the list is ascending).  The
// consumed gradient is zeroed for the next step.  Rows not in the list are
// never touched.  The update's square root and reciprocal are the hardware
// ones (about 1 ulp each): it feeds no discrete decision, and its relative
// error stays below 1e-6 of the step.
#include "project_grad.hpp"
#include "project_record.hpp"

namespace gs {
namespace {

__global__ __launch_bounds__(256) void k_adam(float* __restrict__ params, float* __restrict__ grads,
                                              float* __restrict__ m, float* __restrict__ v, int64_t ld,
                                              const int32_t* __restrict__ rows, const int64_t* __restrict__ row_count,
                                              float lr, float b1, float b2, float eps, float bc1, float bc2) {
  const int64_t s = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (s >= *row_count) return;
  const uint32_t off4 = uint32_t(rows[s]) << 2;
  const float ob1 = 1.0f - b1, ob2 = 1.0f - b2;
  const float ibc1 = 1.0f / bc1, ibc2 = 1.0f / bc2;
#pragma unroll 4
  for (int k = 0; k < 59; ++k) {
    auto* const gq = plane_elem(grads, ld, k, off4);
    auto* const mq = plane_elem(m, ld, k, off4);
    auto* const vq = plane_elem(v, ld, k, off4);
    auto* const pq = plane_elem(params, ld, k, off4);
    const float g = *gq;
    const float mn = fmaf(b1, *mq, ob1 * g);
    const float vn = fmaf(b2, *vq, ob2 * g * g);
    *mq = mn;
    *vq = vn;
    *pq -= lr * (mn * ibc1) * __builtin_amdgcn_rcpf(__builtin_amdgcn_sqrtf(vn * ibc2) + eps);
    *gq = 0.0f;
  }
}

using ArgCam = const __attribute__((address_space(4))) CamArgs;

// A camera read field by field from the kernel-argument segment (scalar
// loads: every lane reads the same words).
__device__ __forceinline__ CamArgs arg_camera(ArgCam* c) {
  CamArgs r;
#pragma unroll
  for (int j = 0; j < 9; ++j) r.R[j] = c->R[j];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    r.t[j] = c->t[j];
    r.campos[j] = c->campos[j];
  }
  r.fx = c->fx;
  r.fy = c->fy;
  r.cx = c->cx;
  r.cy = c->cy;
  r.near_z = c->near_z;
  r.width = c->width;
  r.height = c->height;
  r.tiles_x = c->tiles_x;
  r.tiles_y = c->tiles_y;
  return r;
}

// The projection backward of the batch's last views fused with the Adam
// step, one thread per listed row: for each fused view whose screen-space
// row is non-zero (a row the view's raster backward reached; a zero row
// chains to a zero gradient), that view's parameter gradients, chained
// from the row (then re-zeroed), are added in view order to the gradients
// accumulated so far (the gradient planes, or zero without them); then
// Adam as k_adam.  The same arithmetic as the projection backward of each
// view followed by k_adam, without writing and re-reading the gradient
// planes; the parameters are read once for all the views.
// (Three waves per SIMD, what its 48 KB of LDS per workgroup allows: the
// register allocation is held to that, 168 VGPRs; one more register would
// drop it to two waves.)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void k_project_adam(
    FusedViews views, float* __restrict__ params, float* __restrict__ grads, float* __restrict__ m,
    float* __restrict__ v, int64_t ld, const int32_t* __restrict__ rows, const int64_t* __restrict__ row_count,
    float lr, float b1, float b2, float eps, float bc1, float bc2) {
  const int64_t s = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (s >= *row_count) return;
  const int64_t i = rows[s];
  const uint32_t off4 = uint32_t(i) << 2;
  // the 48 SH coefficient gradients accumulate in LDS (plane j + 11 of
  // this thread at s_sh[j][tid]), the other 11 in registers
  __shared__ float s_sh[48 * 256];
  float* sh = s_sh + threadIdx.x;
  float p[59], g[59];
#pragma unroll
  for (int k = 0; k < 59; ++k) p[k] = params[int64_t(k) * ld + i];
#pragma unroll
  for (int k = 0; k < 11; ++k) g[k] = grads != nullptr ? grads[int64_t(k) * ld + i] : 0.0f;
#pragma unroll
  for (int j = 0; j < 48; ++j) sh[j * 256] = grads != nullptr ? grads[int64_t(11 + j) * ld + i] : 0.0f;
  // the views are read in place from the argument segment (the first
  // argument sits at its start), so a view's camera is a few scalar loads
  (void)views;
  using ArgViews = const __attribute__((address_space(4))) FusedViews;
  ArgViews* fv = (ArgViews*)__builtin_amdgcn_kernarg_segment_ptr();
  const int nv = fv->count;
  // the views that may have touched the row (all without a touched map)
  uint32_t tbits = 0xFFFFu;
  uint8_t* const tmap = fv->touched;
  if (tmap != nullptr) {
    const uint4 tb = reinterpret_cast<const uint4*>(tmap)[i];
    const uint32_t tw[4] = {tb.x, tb.y, tb.z, tb.w};
    tbits = 0;
#pragma unroll
    for (int b = 0; b < 16; ++b) tbits |= ((tw[b >> 2] >> (8 * (b & 3))) & 0xFFu) != 0u ? (1u << b) : 0u;
    if (tbits != 0) reinterpret_cast<uint4*>(tmap)[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  for (int w = 0; w < nv; ++w) {
    if (((tbits >> w) & 1u) == 0) continue;   // (a row the view's backward never reached is zero)
    float4* g2 = reinterpret_cast<float4*>(fv->grad2d[w]) + 3 * i;
    const float4 ga4 = g2[0], gb4 = g2[1], gc4 = g2[2];
    const bool nz = ga4.x != 0.f || ga4.y != 0.f || ga4.z != 0.f || ga4.w != 0.f || gb4.x != 0.f ||
                    gb4.y != 0.f || gb4.z != 0.f || gb4.w != 0.f || gc4.x != 0.f || gc4.y != 0.f ||
                    gc4.z != 0.f || gc4.w != 0.f;
    if (nz) {
      const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
      g2[0] = z4;
      g2[1] = z4;
      g2[2] = z4;
      const float grgb[3] = {gb4.z, gb4.w, gc4.x};
      const CamArgs cam = arg_camera(&fv->cam[w]);
      project_grads<true, 256>(p, cam, ga4.x, ga4.y, ga4.z, ga4.w, gb4.x, gb4.y, grgb, g, sh);
    }
  }
  const float ob1 = 1.0f - b1, ob2 = 1.0f - b2;
  const float ibc1 = 1.0f / bc1, ibc2 = 1.0f / bc2;
  // the row offset passed through an empty asm: the plane addresses below
  // are formed here rather than hoisted and kept alive across the
  // projection.  Fully unrolled (p and g stay in registers: constant
  // indices), in groups of eight planes the scheduler may not merge, so the
  // Adam state of only one group is in flight at a time
  uint32_t offa = off4;
  asm volatile("" : "+v"(offa));
#pragma unroll
  for (int k = 0; k < 59; ++k) {
    auto* const mq = plane_elem(m, ld, k, offa);
    auto* const vq = plane_elem(v, ld, k, offa);
    const float gk = k < 11 ? g[k] : sh[(k - 11) * 256];
    const float mn = fmaf(b1, *mq, ob1 * gk);
    const float vn = fmaf(b2, *vq, ob2 * gk * gk);
    *mq = mn;
    *vq = vn;
    p[k] = p[k] - lr * (mn * ibc1) * __builtin_amdgcn_rcpf(__builtin_amdgcn_sqrtf(vn * ibc2) + eps);
    *plane_elem(params, ld, k, offa) = p[k];
    if (grads != nullptr) *plane_elem(grads, ld, k, offa) = 0.0f;
    if ((k & 7) == 7) __builtin_amdgcn_sched_barrier(0);
  }
  // the next view's record of the updated row (as the preprocess computes it)
  if (fv->next_proj != nullptr) {
    const CamArgs nc = arg_camera(&fv->next);
    float4 rec[4];
    const bool visible = project_record(p, nc, rec);
    float4* r = reinterpret_cast<float4*>(fv->next_proj) + 4 * i;
    r[0] = rec[0];
    r[1] = rec[1];
    r[2] = rec[2];
    r[3] = rec[3];
    if (fv->next_bin != nullptr) reinterpret_cast<float4*>(fv->next_bin)[i] = rec[3];
    if (visible) {
      fv->next_flags[i] = 1;
      fv->union_flags[i] = 1;
    }
  }
}

}  // namespace

hipError_t launch_project_adam(float* params, float* grads, float* m, float* v, int64_t n, int64_t ld,
                               const FusedViews& views, const int32_t* rows, const int64_t* row_count, float lr,
                               float beta1, float beta2, float eps, float bc1, float bc2, hipStream_t st) {
  if (n == 0) return hipSuccess;
  k_project_adam<<<unsigned((n + 255) / 256), 256, 0, st>>>(views, params, grads, m, v, ld, rows, row_count, lr,
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
