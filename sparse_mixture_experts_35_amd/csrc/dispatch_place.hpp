// Dispatch placement of one chunk of flat slots, as a block-level device
// function: the dispatch kernel runs it for every chunk, and the fused
// selection + dispatch kernel of small batches runs it for its single chunk
// after selecting in the same block.
//
// Block c sums the per-chunk expert counts (or counts its own chunk when
// hist is NULL and there is one chunk), scans the kept totals into offsets
// and places its slots in rounds of 256: a slot's rank inside a round comes
// from a wave-level match loop (ballot of the lanes holding the same expert,
// rank = lanes below it) plus the counts of the earlier waves of the round;
// running per-expert counts carry the rank across rounds. No atomic decides
// a position and no float is summed by an atomic, so the permutation is the
// stable one [page "MOE 专家选择与路由机制" (wuhy-notes), §三 "Token
// Dispatch"]. With a capacity C an expert keeps its first min(count, C)
// slots [wuhy-notes §六 Expert Capacity]. Block 0 writes counts, offsets,
// f_e = count / (T·k), L_aux = α·N·Σ f_e p_e [page "拆解 MoE：单个 Token
// 如何经过专家层" (feinterview), load-balance section], the capacity usage
// and dropped fraction, and clears zero_n int32 counters at `zero` for a
// later kernel of the same call.
#pragma once

#include "common.hpp"

namespace moe {
namespace dsp {

constexpr int kThreads = 256;
constexpr int kChunk = 1024;                       // slots of a single-chunk dispatch
constexpr int kChunkMulti = 256;                   // slots per block otherwise
constexpr int kRounds = kChunk / kThreads;         // slots per thread at most
constexpr int kMaxN = 512;

// Flat slots per dispatch block: one block for up to kChunk slots (decode
// batches: one kernel), else kChunkMulti (more, shorter blocks).
__host__ __device__ __forceinline__ int chunk_slots(int64_t R) {
  return R <= kChunk ? kChunk : kChunkMulti;
}

// Row stride of the per-chunk counts, stored expert-major as hist[e][c]:
// the chunk count rounded up to 4 (the pad columns hold zeros), so that a
// row reads as int4.
__host__ __device__ __forceinline__ int hist_ld(int chunks) { return (chunks + 3) & ~3; }

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

__device__ __forceinline__ void place_chunk(
    int c, const int32_t* __restrict__ ids, int T, int k, int N,
    const int32_t* __restrict__ hist, int chunks, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm_src, int32_t* __restrict__ row_of,
    const float* __restrict__ p_mean, float* __restrict__ f_out, float* __restrict__ l_aux,
    float alpha, int cap_in, float* __restrict__ cap_stats, int32_t* __restrict__ zero,
    int zero_n) {
  __shared__ int s_cnt[kMaxN];     // routed slots per expert (all chunks)
  __shared__ int s_base[kMaxN];    // slots of e in the chunks before this one
  __shared__ int s_off[kMaxN];     // first bucket row of e
  __shared__ int s_kept[kMaxN];
  __shared__ int s_run[kMaxN];     // slots of e placed in the earlier rounds
  __shared__ int s_wc[4][kMaxN];   // per-wave counts of the current round
  __shared__ int s_wave[4];
  __shared__ float s_red[kThreads];
  __shared__ int s_pt[kThreads], s_pb[kThreads];   // partial sums of the chunk counts
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int R = T * k;
  const bool limited = cap_in > 0;
  const int cap = limited ? cap_in : 0x7fffffff;
  const int chunk = chunk_slots(R);

  // this thread's slots of the chunk, loaded up front (slot r0 + tid of
  // round r0 / kThreads)
  const int f0 = c * chunk, f1 = min(f0 + chunk, R);
  int my_e[kRounds];
#pragma unroll
  for (int q = 0; q < kRounds; ++q) {
    const int f = f0 + q * kThreads + tid;
    const int id = f < f1 ? ids[f] : -1;
    my_e[q] = (unsigned)id < (unsigned)N ? id : -1;
  }
  if (hist) {
    // P threads share an expert's row of chunk counts, each summing a range
    // of whole int4 groups: the loads of a range are independent, so few
    // round trips to the memory the counts were written through
    const int ld = hist_ld(chunks);
    const int P = N >= kThreads ? 1 : kThreads / N;
    const int L = ((ld / 4 + P - 1) / P) * 4;       // chunks per thread
    for (int i = tid; i < N * P; i += kThreads) {
      const int e = i % N, p = i / N;
      const int c0 = p * L, c1 = min(c0 + L, ld);
      const int4* row = reinterpret_cast<const int4*>(hist + (int64_t)e * ld);
      int tot = 0, base = 0;
#pragma unroll 8
      for (int cc = c0; cc < c1; cc += 4) {
        const int4 v = row[cc >> 2];
        tot += v.x + v.y + v.z + v.w;
        base += (cc < c ? v.x : 0) + (cc + 1 < c ? v.y : 0) + (cc + 2 < c ? v.z : 0) +
                (cc + 3 < c ? v.w : 0);
      }
      if (P == 1) {
        s_cnt[e] = tot;
        s_base[e] = base;
        s_run[e] = 0;
      } else {
        s_pt[i] = tot;
        s_pb[i] = base;
      }
    }
    if (P > 1) {
      __syncthreads();
      for (int e = tid; e < N; e += kThreads) {
        int tot = 0, base = 0;
        for (int p = 0; p < P; ++p) {
          tot += s_pt[p * N + e];
          base += s_pb[p * N + e];
        }
        s_cnt[e] = tot;
        s_base[e] = base;
        s_run[e] = 0;
      }
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
    for (int i = tid; i < zero_n; i += kThreads) zero[i] = 0;
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
    } else if (f < f1) {
      row_of[f] = -1;                         // an id outside [0, N): no row
    }
    __syncthreads();
    for (int i = tid; i < N; i += kThreads)
      s_run[i] += s_wc[0][i] + s_wc[1][i] + s_wc[2][i] + s_wc[3][i];
    __syncthreads();
  }
}

}  // namespace dsp
}  // namespace moe
