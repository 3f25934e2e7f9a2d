// fp32 expert FFN kernels: LDS-tiled fp32 FMA GEMMs over the experts' row
// groups (fp32 layers; the bf16 path runs on MFMA).
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

// Tiled fp32 grouped GEMM: a 256-thread block computes 64 rows x 64 columns
// of one expert (of gate and up together for the gate/up GEMM), each thread
// a 4 x 4 patch. K advances in chunks of 16 staged in LDS (A and B
// transposed to [k][row]), read back four rows or columns at a time. Every
// output is one fmaf chain over k = 0, 1, ..., K - 1 from zero, the same
// sequence of operations as a plain dot-product loop.
constexpr int kFM = 64, kFN = 64, kFK = 16;
constexpr int kFMaxGroups = 512;
enum F32Mode { F32_SWIGLU = 0, F32_PREACT = 1, F32_DOWN = 2 };

// acc[b] += A[rows] · B_b[columns]^T over k in [kbeg, kend): row i of the
// staging map (tid / 16 + 16 i) reads arow[i][k] when aval[i] (else 0), and
// the same for the columns from brow[b][i]; every output's sum runs over k
// in order.
template <int NB>
__device__ __forceinline__ void f32_tile_loop(const float* const (&arow)[4],
                                              const bool (&aval)[4],
                                              const float* const (&brow)[NB][4],
                                              const bool (&bval)[4], int kbeg, int kend,
                                              float (*sA)[kFM + 4], float (*sB)[kFK][kFN + 4],
                                              float (&acc)[NB][4][4]) {
  const int tid = threadIdx.x;
  const int kk = tid % kFK;
  const int tx = tid % 16, ty = tid / 16;   // columns 4 tx .. 4 tx + 3, rows 4 ty .. 4 ty + 3
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[b][i][j] = 0.0f;
  for (int k0 = kbeg; k0 < kend; k0 += kFK) {
    const int k = k0 + kk;
    const bool kv = k < kend;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = tid / kFK + 16 * i;
      sA[kk][row] = (aval[i] && kv) ? arow[i][k] : 0.0f;
#pragma unroll
      for (int b = 0; b < NB; ++b) sB[b][kk][row] = (bval[i] && kv) ? brow[b][i][k] : 0.0f;
    }
    __syncthreads();
    const int kn = min(kFK, kend - k0);
    for (int c = 0; c < kn; ++c) {
      const float4 a4 = *reinterpret_cast<const float4*>(&sA[c][4 * ty]);
      const float a[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float4 b4 = *reinterpret_cast<const float4*>(&sB[b][c][4 * tx]);
        const float w[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[b][i][j] = fmaf(a[i], w[j], acc[b][i][j]);
      }
    }
    __syncthreads();
  }
}

template <int MODE>
__global__ __launch_bounds__(256) void grouped_f32_kernel(GroupedProblem p, int nt_n) {
  constexpr bool DUAL = MODE != F32_DOWN;
  constexpr int NB = DUAL ? 2 : 1;
  __shared__ __attribute__((aligned(16))) float sA[kFK][kFM + 4];
  __shared__ __attribute__((aligned(16))) float sB[NB][kFK][kFN + 4];
  __shared__ int s_pref[kFMaxGroups + 1];
  const int tid = threadIdx.x;
  const int G = p.offsets ? p.groups : 1;
  // m-tiles per group, exclusive prefix (one wave; at most 512 groups)
  if (tid < 64) {
    int loc[kFMaxGroups / 64];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kFMaxGroups / 64; ++i) {
      const int g = tid * (kFMaxGroups / 64) + i;
      int c = 0;
      if (g < G) c = ((p.offsets ? p.offsets[g + 1] - p.offsets[g] : p.M) + kFM - 1) / kFM;
      loc[i] = c;
      sum += c;
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o, 64);
      if (tid >= o) incl += t;
    }
    int run = incl - sum;
#pragma unroll
    for (int i = 0; i < kFMaxGroups / 64; ++i) {
      const int g = tid * (kFMaxGroups / 64) + i;
      if (g < G) s_pref[g] = run;
      run += loc[i];
    }
    if (tid == 63) s_pref[G] = incl;
  }
  __syncthreads();
  const int mt = (int)(blockIdx.x / nt_n), nt = (int)(blockIdx.x % nt_n);
  if (mt >= s_pref[G]) return;
  int lo = 0, hi = G;   // s_pref[lo] <= mt < s_pref[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_pref[mid] <= mt) lo = mid; else hi = mid;
  }
  const int g = lo;
  const int gend = p.offsets ? p.offsets[g + 1] : p.M;
  const int m0 = (p.offsets ? p.offsets[g] : 0) + (mt - s_pref[g]) * kFM;
  const int n0 = nt * kFN;

  // staging: element tid + 256 i of a chunk is row (or column) tid / 16 +
  // 16 i, k = tid % 16 (16 threads read 64 contiguous bytes of a row)
  const float* A = static_cast<const float*>(p.A);
  const float* arow[4];
  const float* brow[NB][4];
  bool aval[4], bval[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = tid / kFK + 16 * i;
    const int r = m0 + row;
    aval[i] = r < gend;
    const int src = aval[i] ? (p.perm ? p.perm[r] / p.kdiv : r) : 0;
    arow[i] = A + (int64_t)src * p.lda;
    const int col = n0 + row;
    bval[i] = col < p.Ncols;
    const int64_t boff = (int64_t)g * p.b_gstride + (int64_t)(bval[i] ? col : 0) * p.ldb;
    brow[0][i] = static_cast<const float*>(p.B0) + boff;
    if (DUAL) brow[NB - 1][i] = static_cast<const float*>(p.B1) + boff;
  }

  float acc[NB][4][4];
  f32_tile_loop<NB>(arow, aval, brow, bval, 0, p.K, sA, sB, acc);
  const int tx = tid % 16, ty = tid / 16;

  float* C = static_cast<float*>(p.C);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = m0 + 4 * ty + i;
    if (r >= gend) break;
    const int64_t orow = (p.c_row0 + r) * (int64_t)p.ldc;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + 4 * tx + j;
      if (n >= p.Ncols) break;
      if constexpr (MODE == F32_SWIGLU) {
        C[orow + n] = silu_precise(acc[0][i][j]) * acc[1][i][j];
        if (p.C2) {
          const int64_t o2 = (p.c_row0 + r) * p.ldc2;
          p.C2[o2 + n] = acc[0][i][j];
          p.C2[o2 + p.Ncols + n] = acc[1][i][j];
        }
      } else if constexpr (MODE == F32_PREACT) {
        C[orow + n] = acc[0][i][j];
        C[orow + p.Ncols + n] = acc[1][i][j];
      } else {
        C[orow + n] = acc[0][i][j];
      }
    }
  }
}

// Weight gradients: C_g[m][n] = sum over k in [kofs[g], kofs[g+1]) of
// A[m][k] B[n][k], a 64 x 64 tile of one group per block.
__global__ __launch_bounds__(256) void kgroup_f32_kernel(const float* __restrict__ A, int lda,
                                                         const float* __restrict__ B, int ldb,
                                                         const int32_t* __restrict__ kofs, int M,
                                                         int Ncols, float* __restrict__ C,
                                                         int64_t c_gstride, int ldc, int nt_n) {
  __shared__ __attribute__((aligned(16))) float sA[kFK][kFM + 4];
  __shared__ __attribute__((aligned(16))) float sB[1][kFK][kFN + 4];
  const int tid = threadIdx.x;
  const int g = blockIdx.y;
  const int m0 = (int)(blockIdx.x / nt_n) * kFM, n0 = (int)(blockIdx.x % nt_n) * kFN;
  const float* arow[4];
  const float* brow[1][4];
  bool aval[4], bval[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = tid / kFK + 16 * i;
    aval[i] = m0 + row < M;
    bval[i] = n0 + row < Ncols;
    arow[i] = A + (int64_t)(aval[i] ? m0 + row : 0) * lda;
    brow[0][i] = B + (int64_t)(bval[i] ? n0 + row : 0) * ldb;
  }
  float acc[1][4][4];
  f32_tile_loop<1>(arow, aval, brow, bval, kofs[g], kofs[g + 1], sA, sB, acc);
  const int tx = tid % 16, ty = tid / 16;
  float* Cg = C + (int64_t)g * c_gstride;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + 4 * ty + i;
    if (m >= M) break;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + 4 * tx + j;
      if (n >= Ncols) break;
      Cg[(int64_t)m * ldc + n] = acc[0][i][j];
    }
  }
}

template <int MODE>
hipError_t launch_grouped_f32(const GroupedProblem& p, hipStream_t st) {
  const int G = p.offsets ? p.groups : 1;
  if (p.M == 0 || p.Ncols == 0 || G == 0) return hipSuccess;
  if (G > kFMaxGroups) return hipErrorInvalidValue;
  const int nt_n = (p.Ncols + kFN - 1) / kFN;
  // m-tiles: at most M / 64 + one partial tile per group
  const int64_t mt_bound = (int64_t)(p.M + kFM - 1) / kFM + (p.offsets ? G : 0);
  const int64_t blocks = mt_bound * nt_n;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((grouped_f32_kernel<MODE>), dim3((unsigned)blocks), dim3(256), 0, st, p,
                     nt_n);
  return hipGetLastError();
}

}  // namespace

// SwiGLU expert: W_down (SiLU(W_gate x) ⊙ W_up x) [page "MOE 专家选择与路由机制"
// (wuhy-notes), §一 expert formula], in fp32.
hipError_t launch_gateup_f32(const GroupedProblem& p, hipStream_t st) {
  return launch_grouped_f32<F32_SWIGLU>(p, st);
}

// Gate and up pre-activations side by side (ldc = 2 Ncols): the backward
// pass's recompute.
hipError_t launch_gateup_preact_f32(const GroupedProblem& p, hipStream_t st) {
  return launch_grouped_f32<F32_PREACT>(p, st);
}

hipError_t launch_down_f32(const GroupedProblem& p, hipStream_t st) {
  return launch_grouped_f32<F32_DOWN>(p, st);
}

hipError_t launch_kgroup_f32(const float* A, int lda, const float* B, int ldb,
                             const int32_t* kofs, int groups, int M, int Ncols, float* C,
                             int64_t c_gstride, int ldc, hipStream_t st) {
  if ((int64_t)M * Ncols == 0 || groups == 0) return hipSuccess;
  const int nt_n = (Ncols + kFN - 1) / kFN;
  const int64_t blocks = (int64_t)((M + kFM - 1) / kFM) * nt_n;
  if (blocks > 0x7fffffff || groups > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kgroup_f32_kernel, dim3((unsigned)blocks, groups), dim3(256), 0, st, A, lda,
                     B, ldb, kofs, M, Ncols, C, c_gstride, ldc, nt_n);
  return hipGetLastError();
}

}  // namespace moe
