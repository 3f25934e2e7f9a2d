// Router: scores, top-k selection and gates.
//
//   z_t = W_r h_t (+ b_r)            [page "MOE 专家选择与路由机制" (wuhy-notes),
//                                     §二 第一步; the fp32 logits kernel is
//                                     here, the bf16 one is an MFMA GEMM]
//   softmax / sigmoid scores         [wuhy-notes §二 第二步; page
//                                     "MoE：router 怎样选 expert" (cooking-agi),
//                                     first section]
//   S_t = TopK(score_t, k) + gates   [wuhy-notes §二 第三步; cooking-agi first
//                                     section; pwwt.cn §2.1 route()]
//
// One wavefront per token. Lane l holds experts l, l+64, ... (N <= 512, so
// at most eight per lane, in registers). Top-k is k rounds of a wave-wide
// argmax (butterfly over __shfl_xor) on (score, index) with the lower index
// winning ties. In the softmax modes the selection runs on z, which orders
// the experts exactly as the softmax does. Per-block sums of the routing
// probabilities go to p_part in a fixed order, never through float atomics.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kTokensPerBlock = 64;   // 16 per wave
constexpr int kMaxPerLane = 8;        // 512 experts / 64 lanes
constexpr int kMaxK = 16;

__global__ void router_logits_f32_kernel(const float* __restrict__ h,
                                         const float* __restrict__ w, float* __restrict__ z,
                                         int T, int d, int N) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T * N) return;
  const int t = (int)(idx / N), e = (int)(idx % N);
  const float* a = h + (int64_t)t * d;
  const float* b = w + (int64_t)e * d;
  float s = 0.0f;
  for (int c = 0; c < d; ++c) s = fmaf(a[c], b[c], s);
  z[idx] = s;
}

__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void route_select_kernel(
    const float* __restrict__ z_part, int splits, const float* __restrict__ b_router,
    const float* __restrict__ b_select, int32_t* __restrict__ ids,
    float* __restrict__ gates, float* __restrict__ p_part, int T, int N, int k) {
  __shared__ float s_p[4][512];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t TN = (int64_t)T * N;

  float pacc[kMaxPerLane];
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) pacc[i] = 0.0f;

  const int tw0 = blockIdx.x * kTokensPerBlock + w * (kTokensPerBlock / 4);
  for (int tt = 0; tt < kTokensPerBlock / 4; ++tt) {
    const int t = tw0 + tt;
    if (t >= T) break;
    // ---- logits (sum of split-K slices in order, then the router bias)
    float zv[kMaxPerLane], sel[kMaxPerLane], aux[kMaxPerLane];
    bool cand[kMaxPerLane];
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + 64 * i;
      cand[i] = e < N;
      float v = 0.0f;
      if (cand[i]) {
        const float* zp = z_part + (int64_t)t * N + e;
        for (int s = 0; s < splits; ++s) v += zp[s * TN];
        if (b_router) v += b_router[e];
      }
      zv[i] = v;
      if (MODE == 2) {
        const float s = 1.0f / (1.0f + expf(-v));   // sigmoid score
        aux[i] = s;
        sel[i] = cand[i] ? s + b_select[e] : 0.0f;
      } else {
        aux[i] = v;
        sel[i] = v;
      }
    }
    // ---- top-k: k rounds of a wave argmax
    int win_id[kMaxK];
    float win_aux[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      win_id[j] = 0;
      win_aux[j] = 0.0f;
    }
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY, ba = 0.0f;
      int bi = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i) {
        const int e = lane + 64 * i;
        if (cand[i] && better(sel[i], e, bv, bi)) {
          bv = sel[i];
          bi = e;
          ba = aux[i];
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        const float oa = __shfl_xor(ba, o, 64);
        if (better(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
          ba = oa;
        }
      }
      // every lane now holds the same winner; its owner drops it
      if ((bi & 63) == lane) {
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i)
          if (i == (bi >> 6)) cand[i] = false;
      }
#pragma unroll
      for (int jj = 0; jj < kMaxK; ++jj)
        if (jj == j) {
          win_id[jj] = bi;
          win_aux[jj] = ba;
        }
    }
    // ---- gates
    float zmax = -INFINITY, denom_all = 0.0f;
    const bool need_full = (MODE == 1) || (p_part != nullptr);
    if (MODE != 2 && need_full) {
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i)
        if (lane + 64 * i < N) m = fmaxf(m, zv[i]);
      zmax = wave_max(m);
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i)
        if (lane + 64 * i < N) s += expf(zv[i] - zmax);
      denom_all = wave_sum(s);
    }
    float gsel[kMaxK];
    if (MODE == 0) {
      // softmax over the selected logits; win_aux[0] is the largest
      float sum = 0.0f;
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) {
        gsel[j] = (j < k) ? expf(win_aux[j] - win_aux[0]) : 0.0f;
        sum += gsel[j];
      }
      const float inv = 1.0f / sum;
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) gsel[j] *= inv;
    } else if (MODE == 1) {
      const float inv = 1.0f / denom_all;
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) gsel[j] = (j < k) ? expf(win_aux[j] - zmax) * inv : 0.0f;
    } else {
      float sum = 0.0f;
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) sum += (j < k) ? win_aux[j] : 0.0f;
      const float inv = 1.0f / sum;
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) gsel[j] = (j < k) ? win_aux[j] * inv : 0.0f;
    }
    int my_id = 0;
    float my_g = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j == lane) {
        my_id = win_id[j];
        my_g = gsel[j];
      }
    if (lane < k) {
      ids[(int64_t)t * k + lane] = my_id;
      gates[(int64_t)t * k + lane] = my_g;
    }
    // ---- routing probabilities for p_i
    if (p_part) {
      if (MODE == 2) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i)
          if (lane + 64 * i < N) s += aux[i];
        const float inv = 1.0f / wave_sum(s);
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i)
          if (lane + 64 * i < N) pacc[i] += aux[i] * inv;
      } else {
        const float inv = 1.0f / denom_all;
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i)
          if (lane + 64 * i < N) pacc[i] += expf(zv[i] - zmax) * inv;
      }
    }
  }
  if (p_part) {
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i)
      if (lane + 64 * i < N) s_p[w][lane + 64 * i] = pacc[i];
    __syncthreads();
    for (int e = tid; e < N; e += kThreads)
      p_part[(int64_t)blockIdx.x * N + e] = ((s_p[0][e] + s_p[1][e]) + s_p[2][e]) + s_p[3][e];
  }
}

// p_mean[e] = (sum over blocks, in block order, of p_part[b][e]) / T
__global__ void p_reduce_kernel(const float* __restrict__ p_part, float* __restrict__ p_mean,
                                int blocks, int T, int N) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= N) return;
  float s = 0.0f;
  for (int b = 0; b < blocks; ++b) s += p_part[(int64_t)b * N + e];
  p_mean[e] = s / (float)T;
}

}  // namespace

hipError_t launch_router_logits_f32(const float* h, const float* w, float* z, int T, int d,
                                    int N, hipStream_t st) {
  const int64_t n = (int64_t)T * N;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(router_logits_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     st, h, w, z, T, d, N);
  return hipGetLastError();
}

int route_select_blocks(int T) { return (T + kTokensPerBlock - 1) / kTokensPerBlock; }

hipError_t launch_route_select(const float* z_part, int splits, const float* b_router,
                               const float* b_select, int32_t* ids, float* gates,
                               float* p_part, int T, int N, int k, int mode, hipStream_t st) {
  const int blocks = route_select_blocks(T);
  if (blocks == 0) return hipSuccess;
  switch (mode) {
    case 0:
      hipLaunchKernelGGL(route_select_kernel<0>, dim3(blocks), dim3(kThreads), 0, st, z_part,
                         splits, b_router, b_select, ids, gates, p_part, T, N, k);
      break;
    case 1:
      hipLaunchKernelGGL(route_select_kernel<1>, dim3(blocks), dim3(kThreads), 0, st, z_part,
                         splits, b_router, b_select, ids, gates, p_part, T, N, k);
      break;
    default:
      hipLaunchKernelGGL(route_select_kernel<2>, dim3(blocks), dim3(kThreads), 0, st, z_part,
                         splits, b_router, b_select, ids, gates, p_part, T, N, k);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_p_reduce(const float* p_part, float* p_mean, int blocks, int T, int N,
                           hipStream_t st) {
  if (T == 0 || N == 0) return hipSuccess;
  hipLaunchKernelGGL(p_reduce_kernel, dim3((N + 255) / 256), dim3(256), 0, st, p_part, p_mean,
                     blocks, T, N);
  return hipGetLastError();
}

}  // namespace moe
