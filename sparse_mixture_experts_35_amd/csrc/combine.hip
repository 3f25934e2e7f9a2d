// Combine: weighted gather-sum of each token's expert outputs back to token
// order, y_t = (shared row) + Σ_j g_tj · out_rows[row_of[t·k + j]].
// The contributions are added, never written over one another [page
// "MoE：router 怎样选 expert" (cooking-agi), section on how outputs come
// back; page "【大模型】MoE（专家混合模型）简介" (horizon.auto), §3 ④ Gather].
//
// A slot dropped by the expert capacity (row_of = -1) adds nothing [page
// "MOE 专家选择与路由机制" (wuhy-notes), §六 Expert Capacity].
//
// One block per token; each thread owns 16-byte column chunks and reads the
// k rows (and the shared row) at those columns, so every load is coalesced,
// four slots' loads in flight at once; fp32 accumulation in slot order; no
// atomics.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void combine_bf16_kernel(
    const bf16_t* __restrict__ rows, const int32_t* __restrict__ row_of,
    const float* __restrict__ gates, bf16_t* __restrict__ y, int T, int k, int d,
    int has_shared) {
  const int t = blockIdx.x;
  const int64_t R = (int64_t)T * k;
  for (int c = threadIdx.x * 8; c < d; c += kThreads * 8) {
    float acc[8];
    if (has_shared) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(rows + (R + t) * d + c);
      unpack_bf16x8(v, acc);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    }
    // slots in groups of four: the group's row loads are all issued before
    // the first of them is used, then added in slot order
    for (int j0 = 0; j0 < k; j0 += 4) {
      int64_t r[4];
      float g[4];
      u32x4 raw[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = j0 + q;
        r[q] = j < k ? row_of[(int64_t)t * k + j] : -1;
        g[q] = j < k ? gates[(int64_t)t * k + j] : 0.0f;
        raw[q] = r[q] >= 0 ? *reinterpret_cast<const u32x4*>(rows + r[q] * d + c)
                           : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (r[q] < 0) continue;
        float v[8];
        unpack_bf16x8(raw[q], v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(g[q], v[i], acc[i]);
      }
    }
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
    *reinterpret_cast<u32x4*>(y + (int64_t)t * d + c) = o;
  }
}

__global__ __launch_bounds__(kThreads) void combine_f32_kernel(
    const float* __restrict__ rows, const int32_t* __restrict__ row_of,
    const float* __restrict__ gates, float* __restrict__ y, int T, int k, int d,
    int has_shared) {
  const int t = blockIdx.x;
  const int64_t R = (int64_t)T * k;
  for (int c = threadIdx.x; c < d; c += kThreads) {
    float acc = has_shared ? rows[(R + t) * d + c] : 0.0f;
    for (int j = 0; j < k; ++j) {
      const int64_t r = row_of[(int64_t)t * k + j];
      if (r < 0) continue;
      acc = fmaf(gates[(int64_t)t * k + j], rows[r * d + c], acc);
    }
    y[(int64_t)t * d + c] = acc;
  }
}

}  // namespace

hipError_t launch_combine(const void* out_rows, const int32_t* row_of, const float* gates,
                          void* y, int T, int k, int d, int has_shared, int bf16,
                          hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (bf16) {
    hipLaunchKernelGGL(combine_bf16_kernel, dim3(T), dim3(kThreads), 0, st,
                       static_cast<const bf16_t*>(out_rows), row_of, gates,
                       static_cast<bf16_t*>(y), T, k, d, has_shared);
  } else {
    hipLaunchKernelGGL(combine_f32_kernel, dim3(T), dim3(kThreads), 0, st,
                       static_cast<const float*>(out_rows), row_of, gates,
                       static_cast<float*>(y), T, k, d, has_shared);
  }
  return hipGetLastError();
}

}  // namespace moe
