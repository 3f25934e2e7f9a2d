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
// Two kernels over chunks of consecutive flat slots f = t·k + j (one kernel,
// counting its own chunk, when all slots fit one chunk of 1024; else chunks
// of 256):
//  1. dispatch_hist_kernel: block c counts its chunk's slots per expert (LDS
//     integer atomics: counts do not depend on their order) into hist[e][c]
//     (expert-major, rows padded to a multiple of 4 chunks with zeros);
//  2. dispatch_place_kernel: block c sums the chunk counts into the expert
//     totals (and, over the chunks before c, the number of each expert's
//     slots that precede the chunk), scans the kept totals into offsets, then
//     places its chunk's slots stably (dispatch_place.hpp). No atomic decides
//     any position and no float is summed by an atomic.
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
#include "dispatch_place.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

using dsp::kChunk;
using dsp::kMaxN;
using dsp::kThreads;

__global__ __launch_bounds__(kThreads) void dispatch_hist_kernel(const int32_t* __restrict__ ids,
                                                                 int R, int N, int chunks,
                                                                 int32_t* __restrict__ hist) {
  __shared__ int s_h[kMaxN];
  const int tid = threadIdx.x;
  for (int i = tid; i < N; i += kThreads) s_h[i] = 0;
  __syncthreads();
  const int chunk = dsp::chunk_slots(R);
  const int f0 = blockIdx.x * chunk, f1 = min(f0 + chunk, R);
  for (int f = f0 + tid; f < f1; f += kThreads) {
    const int id = ids[f];
    if ((unsigned)id < (unsigned)N) atomicAdd(&s_h[id], 1);
  }
  __syncthreads();
  const int ld = dsp::hist_ld(chunks);
  for (int i = tid; i < N; i += kThreads) hist[(int64_t)i * ld + blockIdx.x] = s_h[i];
  if (blockIdx.x == 0) {
    const int pad = ld - chunks;
    for (int i = tid; i < N * pad; i += kThreads) hist[(int64_t)(i / pad) * ld + chunks + i % pad] = 0;
  }
}

__global__ __launch_bounds__(kThreads) void dispatch_place_kernel(
    const int32_t* __restrict__ ids, int T, int k, int N, const int32_t* __restrict__ hist,
    int chunks, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm_src, int32_t* __restrict__ row_of,
    const float* __restrict__ p_mean, float* __restrict__ f_out, float* __restrict__ l_aux,
    float alpha, int cap_in, float* __restrict__ cap_stats, int32_t* __restrict__ zero,
    int zero_n) {
  dsp::place_chunk(blockIdx.x, ids, T, k, N, hist, chunks, counts, offsets, perm_src, row_of,
                   p_mean, f_out, l_aux, alpha, cap_in, cap_stats, zero, zero_n);
}

}  // namespace

int dispatch_chunks(int T, int k) {
  const int64_t R = (int64_t)T * k;
  const int chunk = dsp::chunk_slots(R);
  return (int)((R + chunk - 1) / chunk);
}

int64_t dispatch_hist_ints(int T, int k, int N) {
  const int chunks = dispatch_chunks(T, k);
  return chunks > 1 ? (int64_t)N * dsp::hist_ld(chunks) : 0;
}

hipError_t launch_dispatch(const int32_t* ids, int T, int k, int N, int32_t* counts,
                           int32_t* offsets, int32_t* perm_src, int32_t* row_of,
                           const float* p_mean, float* f_out, float* l_aux, float alpha,
                           int cap, float* cap_stats, int32_t* hist, hipStream_t st,
                           int32_t* zero, int zero_n) {
  const int chunks = dispatch_chunks(T, k);
  if (chunks == 0) return hipSuccess;
  if (chunks > 1)
    hipLaunchKernelGGL(dispatch_hist_kernel, dim3(chunks), dim3(kThreads), 0, st, ids, T * k, N,
                       chunks, hist);
  hipLaunchKernelGGL(dispatch_place_kernel, dim3(chunks), dim3(kThreads), 0, st, ids, T, k, N,
                     chunks > 1 ? hist : nullptr, chunks, counts, offsets, perm_src, row_of,
                     p_mean, f_out, l_aux, alpha, cap, cap_stats, zero, zero_n);
  return hipGetLastError();
}

}  // namespace moe
