// Dispatch: stable regroup of the (token, slot) pairs by expert, and the
// load statistics.
//
// After top-k every token sends a copy of itself to each selected expert;
// the copies going to one expert are gathered into one contiguous batch
// [page "MOE 专家选择与路由机制" (wuhy-notes), §三 "Token Dispatch" table and
// grouping; page "【大模型】MoE（专家混合模型）简介" (horizon.auto), §3 ②].
// Within an expert the copies keep token order, which makes the permutation
// unique (the pages' grouped listing is in token order).
//
// One block per expert e. Each block builds the full expert histogram of the
// T·k flat slots in LDS (integer atomics: the counts do not depend on their
// order), takes offsets[e] from it, then walks the slots in order with a
// block-wide exclusive scan of the "slot goes to e" predicate to place each
// of expert e's slots at its stable rank. No atomic decides any position and
// no float is summed by an atomic.
//
// Expert capacity [wuhy-notes §六 Expert Capacity]: with a capacity C, expert
// e keeps its first kept_e = min(counts_e, C) slots in that order; offsets
// are the prefix of the kept counts and a later slot gets row_of = -1.
//
// Statistics [page "拆解 MoE：单个 Token 如何经过专家层" (feinterview),
// load-balance section]: f_e = counts_e / (T·k) (the routing, before any
// drop); block 0 also forms L_aux = α·N·Σ_e f_e p_e with a fixed-order
// reduction, and the capacity usage and dropped fraction from the exact
// integer total of kept slots [wuhy-notes, monitoring list].
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 8;                      // consecutive slots per thread
constexpr int kChunk = kThreads * kPerThread;      // slots per scan step

__device__ __forceinline__ int block_excl_scan(int v, int* s_wave, int& total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) s_wave[w] = incl;
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) base += (i < w) ? s_wave[i] : 0;
  total = s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
  __syncthreads();
  return base + incl - v;
}

__global__ __launch_bounds__(kThreads) void dispatch_kernel(
    const int32_t* __restrict__ ids, int T, int k, int N, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm_src, int32_t* __restrict__ row_of,
    const float* __restrict__ p_mean, float* __restrict__ f_out, float* __restrict__ l_aux,
    float alpha, int cap_in, float* __restrict__ cap_stats) {
  __shared__ int s_hist[512];
  __shared__ int s_wave[4];
  __shared__ float s_red[kThreads];
  const int e = blockIdx.x, tid = threadIdx.x;
  const int R = T * k;
  const bool limited = cap_in > 0;
  const int cap = limited ? cap_in : 0x7fffffff;

  for (int i = tid; i < N; i += kThreads) s_hist[i] = 0;
  __syncthreads();
  for (int f = tid; f < R; f += kThreads) {
    const int id = ids[f];
    if ((unsigned)id < (unsigned)N) atomicAdd(&s_hist[id], 1);
  }
  __syncthreads();

  // offsets[e] = sum of the kept counts of experts below e
  int part = 0;
  for (int i = tid; i < e; i += kThreads) part += min(s_hist[i], cap);
  int total;
  block_excl_scan(part, s_wave, total);
  const int off_e = total;
  const int cnt_e = s_hist[e];
  const int kept_e = min(cnt_e, cap);
  if (tid == 0) {
    counts[e] = cnt_e;
    offsets[e] = off_e;
    if (e == N - 1) offsets[N] = off_e + kept_e;
    if (f_out) f_out[e] = (float)cnt_e / (float)R;
  }

  if (e == 0 && cap_stats) {
    // usage = sum kept / (N C), dropped = (T k - sum kept) / (T k); the
    // integer total is exact, each ratio one double division rounded once
    int kp = 0;
    for (int i = tid; i < N; i += kThreads) kp += min(s_hist[i], cap);
    int kept_all;
    block_excl_scan(kp, s_wave, kept_all);
    if (tid == 0) {
      cap_stats[0] = limited ? (float)((double)kept_all / ((double)N * (double)cap)) : 0.0f;
      cap_stats[1] = limited ? (float)((double)(R - kept_all) / (double)R) : 0.0f;
    }
  }

  if (e == 0 && l_aux) {
    // L_aux = alpha * N * sum_e f_e p_e, fixed reduction order
    float s = 0.0f;
    for (int i = tid; i < N; i += kThreads) s += ((float)s_hist[i] / (float)R) * p_mean[i];
    s_red[tid] = s;
    __syncthreads();
    for (int o = kThreads / 2; o > 0; o >>= 1) {
      if (tid < o) s_red[tid] += s_red[tid + o];
      __syncthreads();
    }
    if (tid == 0) l_aux[0] = alpha * (float)N * s_red[0];
  }

  // stable placement of expert e's slots; ranks from kept_e on are dropped
  int placed = 0;
  for (int base = 0; base < R && placed < cnt_e; base += kChunk) {
    const int f0 = base + tid * kPerThread;
    int match[kPerThread];
    int c = 0;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int f = f0 + i;
      match[i] = (f < R && ids[f] == e) ? 1 : 0;
      c += match[i];
    }
    int chunk_total;
    int pos = off_e + placed + block_excl_scan(c, s_wave, chunk_total);
#pragma unroll
    for (int i = 0; i < kPerThread; ++i)
      if (match[i]) {
        if (pos < off_e + kept_e) {
          perm_src[pos] = f0 + i;
          row_of[f0 + i] = pos;
        } else {
          row_of[f0 + i] = -1;
        }
        ++pos;
      }
    placed += chunk_total;
  }
}

}  // namespace

hipError_t launch_dispatch(const int32_t* ids, int T, int k, int N, int32_t* counts,
                           int32_t* offsets, int32_t* perm_src, int32_t* row_of,
                           const float* p_mean, float* f_out, float* l_aux, float alpha,
                           int cap, float* cap_stats, hipStream_t st) {
  hipLaunchKernelGGL(dispatch_kernel, dim3(N), dim3(kThreads), 0, st, ids, T, k, N, counts,
                     offsets, perm_src, row_of, p_mean, f_out, l_aux, alpha, cap, cap_stats);
  return hipGetLastError();
}

}  // namespace moe
