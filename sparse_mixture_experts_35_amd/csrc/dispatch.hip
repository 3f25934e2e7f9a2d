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
// Two kernels over chunks of kChunk consecutive flat slots f = t·k + j (one
// kernel, counting its own chunk, when there is a single chunk):
//  1. dispatch_hist_kernel: block c counts its chunk's slots per expert (LDS
//     integer atomics: counts do not depend on their order) into hist[c][e];
//  2. dispatch_place_kernel: block c sums the chunk counts into the expert
//     totals (and, over the chunks before c, the number of each expert's
//     slots that precede the chunk), scans the kept totals into offsets, then
//     walks its chunk in rounds of 256 slots. A slot's rank inside a round
//     comes from a wave-level match loop (ballot of the lanes holding the
//     same expert, rank = lanes below it) plus the counts of the earlier
//     waves of the round; running per-expert counts carry the rank across
//     rounds. No atomic decides any position and no float is summed by an
//     atomic.
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
constexpr int kChunk = 1024;                       // flat slots per block
constexpr int kRounds = kChunk / kThreads;         // slots per thread
constexpr int kMaxN = 512;

__global__ __launch_bounds__(kThreads) void dispatch_hist_kernel(const int32_t* __restrict__ ids,
                                                                 int R, int N,
                                                                 int32_t* __restrict__ hist) {
  __shared__ int s_h[kMaxN];
  const int tid = threadIdx.x;
  for (int i = tid; i < N; i += kThreads) s_h[i] = 0;
  __syncthreads();
  const int f0 = blockIdx.x * kChunk, f1 = min(f0 + kChunk, R);
  for (int f = f0 + tid; f < f1; f += kThreads) {
    const int id = ids[f];
    if ((unsigned)id < (unsigned)N) atomicAdd(&s_h[id], 1);
  }
  __syncthreads();
  for (int i = tid; i < N; i += kThreads) hist[(int64_t)blockIdx.x * N + i] = s_h[i];
}

// exclusive scan over the block of one value per thread; total in `total`
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

__global__ __launch_bounds__(kThreads) void dispatch_place_kernel(
    const int32_t* __restrict__ ids, int T, int k, int N, const int32_t* __restrict__ hist,
    int chunks, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm_src, int32_t* __restrict__ row_of,
    const float* __restrict__ p_mean, float* __restrict__ f_out, float* __restrict__ l_aux,
    float alpha, int cap_in, float* __restrict__ cap_stats) {
  __shared__ int s_cnt[kMaxN];     // routed slots per expert (all chunks)
  __shared__ int s_base[kMaxN];    // slots of e in the chunks before this one
  __shared__ int s_off[kMaxN];     // first bucket row of e
  __shared__ int s_kept[kMaxN];
  __shared__ int s_run[kMaxN];     // slots of e placed in the earlier rounds
  __shared__ int s_wc[4][kMaxN];   // per-wave counts of the current round
  __shared__ int s_wave[4];
  __shared__ float s_red[kThreads];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = blockIdx.x;
  const int R = T * k;
  const bool limited = cap_in > 0;
  const int cap = limited ? cap_in : 0x7fffffff;

  // this thread's slots of the chunk, loaded up front (slot r0 + tid of
  // round r0 / kThreads)
  const int f0 = c * kChunk, f1 = min(f0 + kChunk, R);
  int my_e[kRounds];
#pragma unroll
  for (int q = 0; q < kRounds; ++q) {
    const int f = f0 + q * kThreads + tid;
    const int id = f < f1 ? ids[f] : -1;
    my_e[q] = (unsigned)id < (unsigned)N ? id : -1;
  }
  if (hist) {
    for (int e = tid; e < N; e += kThreads) {
      int tot = 0, base = 0;
#pragma unroll 8
      for (int cc = 0; cc < chunks; ++cc) {
        const int v = hist[(int64_t)cc * N + e];
        base += cc < c ? v : 0;
        tot += v;
      }
      s_cnt[e] = tot;
      s_base[e] = base;
      s_run[e] = 0;
    }
  } else {
    // a single chunk: count it here
    for (int e = tid; e < N; e += kThreads) {
      s_cnt[e] = 0;
      s_base[e] = 0;
      s_run[e] = 0;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kRounds; ++q)
      if (my_e[q] >= 0) atomicAdd(&s_cnt[my_e[q]], 1);
  }
  __syncthreads();
  for (int e = tid; e < N; e += kThreads) s_kept[e] = min(s_cnt[e], cap);
  __syncthreads();
  // offsets: exclusive scan of the kept counts (two experts per thread)
  const int e0 = 2 * tid, e1 = 2 * tid + 1;
  const int k0 = e0 < N ? s_kept[e0] : 0, k1 = e1 < N ? s_kept[e1] : 0;
  int kept_all;
  const int ex = block_excl_scan(k0 + k1, s_wave, kept_all);
  if (e0 < N) s_off[e0] = ex;
  if (e1 < N) s_off[e1] = ex + k0;
  __syncthreads();

  if (c == 0) {
    for (int e = tid; e < N; e += kThreads) {
      counts[e] = s_cnt[e];
      offsets[e] = s_off[e];
      if (f_out) f_out[e] = (float)s_cnt[e] / (float)R;
    }
    if (tid == 0) offsets[N] = kept_all;
    if (cap_stats && tid == 0) {
      // usage = sum kept / (N C), dropped = (T k - sum kept) / (T k); the
      // integer total is exact, each ratio one double division rounded once
      cap_stats[0] = limited ? (float)((double)kept_all / ((double)N * (double)cap)) : 0.0f;
      cap_stats[1] = limited ? (float)((double)(R - kept_all) / (double)R) : 0.0f;
    }
    if (l_aux) {
      // L_aux = alpha * N * sum_e f_e p_e, fixed reduction order
      float s = 0.0f;
      for (int i = tid; i < N; i += kThreads) s += ((float)s_cnt[i] / (float)R) * p_mean[i];
      s_red[tid] = s;
      __syncthreads();
      for (int o = kThreads / 2; o > 0; o >>= 1) {
        if (tid < o) s_red[tid] += s_red[tid + o];
        __syncthreads();
      }
      if (tid == 0) l_aux[0] = alpha * (float)N * s_red[0];
    }
  }

  // stable placement of this chunk's slots, 256 per round
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int q = 0; q < kRounds; ++q) {
    if (f0 + q * kThreads >= f1) break;      // uniform: no slots left
    for (int i = tid; i < 4 * N; i += kThreads) s_wc[i / N][i % N] = 0;
    __syncthreads();
    const int f = f0 + q * kThreads + tid;
    const int e = my_e[q];
    // rank among the lanes of this wave with the same expert
    uint64_t rem = __ballot(e >= 0);
    int rank = 0;
    while (rem) {
      const int leader = __ffsll((unsigned long long)rem) - 1;
      const int le = __shfl(e, leader, 64);
      const uint64_t m = __ballot(e == le);
      if (e == le) rank = __popcll(m & below);
      if (lane == leader) s_wc[w][le] = __popcll(m);
      rem &= ~m;
    }
    __syncthreads();
    if (e >= 0) {
      int pos = s_run[e] + rank;
      for (int ww = 0; ww < w; ++ww) pos += s_wc[ww][e];
      const int g = s_base[e] + pos;          // rank among all of e's slots
      if (g < s_kept[e]) {
        perm_src[s_off[e] + g] = f;
        row_of[f] = s_off[e] + g;
      } else {
        row_of[f] = -1;
      }
    }
    __syncthreads();
    for (int i = tid; i < N; i += kThreads)
      s_run[i] += s_wc[0][i] + s_wc[1][i] + s_wc[2][i] + s_wc[3][i];
    __syncthreads();
  }
}

}  // namespace

int dispatch_chunks(int T, int k) { return (int)(((int64_t)T * k + kChunk - 1) / kChunk); }

hipError_t launch_dispatch(const int32_t* ids, int T, int k, int N, int32_t* counts,
                           int32_t* offsets, int32_t* perm_src, int32_t* row_of,
                           const float* p_mean, float* f_out, float* l_aux, float alpha,
                           int cap, float* cap_stats, int32_t* hist, hipStream_t st) {
  const int chunks = dispatch_chunks(T, k);
  if (chunks == 0) return hipSuccess;
  if (chunks > 1)
    hipLaunchKernelGGL(dispatch_hist_kernel, dim3(chunks), dim3(kThreads), 0, st, ids, T * k, N,
                       hist);
  hipLaunchKernelGGL(dispatch_place_kernel, dim3(chunks), dim3(kThreads), 0, st, ids, T, k, N,
                     chunks > 1 ? hist : nullptr, chunks, counts, offsets, perm_src, row_of,
                     p_mean, f_out, l_aux, alpha, cap, cap_stats);
  return hipGetLastError();
}

}  // namespace moe
