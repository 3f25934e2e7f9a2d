// fp32 expert FFN kernels: one thread per output element, fp32 FMA.
// Used for fp32 layers (small shapes); the bf16 path runs on MFMA.
// SwiGLU expert: W_down (SiLU(W_gate x) ⊙ W_up x) [page "MOE 专家选择与路由机制"
// (wuhy-notes), §一 expert formula].
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

__device__ __forceinline__ int group_of(const int32_t* offsets, int G, int r) {
  if (!offsets) return 0;
  int lo = 0, hi = G;  // offsets[lo] <= r < offsets[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

__global__ void gateup_f32_kernel(GroupedProblem p) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)p.M * p.Ncols) return;
  const int r = (int)(idx / p.Ncols), n = (int)(idx % p.Ncols);
  if (p.offsets && r >= p.offsets[p.groups]) return;   // rows past the last group
  const int g = group_of(p.offsets, p.groups, r);
  const int src = p.perm ? p.perm[r] / p.kdiv : r;
  const float* a = static_cast<const float*>(p.A) + (int64_t)src * p.lda;
  const float* wg = static_cast<const float*>(p.B0) + g * p.b_gstride + (int64_t)n * p.ldb;
  const float* wu = static_cast<const float*>(p.B1) + g * p.b_gstride + (int64_t)n * p.ldb;
  float sg = 0.0f, su = 0.0f;
  for (int c = 0; c < p.K; ++c) {
    sg = fmaf(a[c], wg[c], sg);
    su = fmaf(a[c], wu[c], su);
  }
  static_cast<float*>(p.C)[(p.c_row0 + r) * p.ldc + n] = silu_precise(sg) * su;
  if (p.C2) {
    p.C2[(p.c_row0 + r) * p.ldc2 + n] = sg;
    p.C2[(p.c_row0 + r) * p.ldc2 + p.Ncols + n] = su;
  }
}

// Gate and up pre-activations side by side (ldc = 2 Ncols): the backward
// pass's recompute.
__global__ void gateup_preact_f32_kernel(GroupedProblem p) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)p.M * p.Ncols) return;
  const int r = (int)(idx / p.Ncols), n = (int)(idx % p.Ncols);
  if (p.offsets && r >= p.offsets[p.groups]) return;
  const int g = group_of(p.offsets, p.groups, r);
  const int src = p.perm ? p.perm[r] / p.kdiv : r;
  const float* a = static_cast<const float*>(p.A) + (int64_t)src * p.lda;
  const float* wg = static_cast<const float*>(p.B0) + g * p.b_gstride + (int64_t)n * p.ldb;
  const float* wu = static_cast<const float*>(p.B1) + g * p.b_gstride + (int64_t)n * p.ldb;
  float sg = 0.0f, su = 0.0f;
  for (int c = 0; c < p.K; ++c) {
    sg = fmaf(a[c], wg[c], sg);
    su = fmaf(a[c], wu[c], su);
  }
  float* out = static_cast<float*>(p.C) + (p.c_row0 + r) * p.ldc;
  out[n] = sg;
  out[p.Ncols + n] = su;
}

__global__ void down_f32_kernel(GroupedProblem p) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)p.M * p.Ncols) return;
  const int r = (int)(idx / p.Ncols), n = (int)(idx % p.Ncols);
  if (p.offsets && r >= p.offsets[p.groups]) return;   // rows past the last group
  const int g = group_of(p.offsets, p.groups, r);
  const int src = p.perm ? p.perm[r] / p.kdiv : r;
  const float* a = static_cast<const float*>(p.A) + (int64_t)src * p.lda;
  const float* w = static_cast<const float*>(p.B0) + g * p.b_gstride + (int64_t)n * p.ldb;
  float s = 0.0f;
  for (int c = 0; c < p.K; ++c) s = fmaf(a[c], w[c], s);
  static_cast<float*>(p.C)[(p.c_row0 + r) * p.ldc + n] = s;
}

}  // namespace

hipError_t launch_gateup_f32(const GroupedProblem& p, hipStream_t st) {
  const int64_t n = (int64_t)p.M * p.Ncols;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(gateup_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_gateup_preact_f32(const GroupedProblem& p, hipStream_t st) {
  const int64_t n = (int64_t)p.M * p.Ncols;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(gateup_preact_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     st, p);
  return hipGetLastError();
}

hipError_t launch_down_f32(const GroupedProblem& p, hipStream_t st) {
  const int64_t n = (int64_t)p.M * p.Ncols;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(down_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace moe
