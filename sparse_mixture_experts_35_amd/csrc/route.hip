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
// A group of lanes per token (8 lanes when N <= 8, up to a whole wavefront;
// a lane holds one expert, or eight when N > 64, in registers; N <= 512).
// Top-k is k rounds of a group-wide argmax (butterfly over __shfl_xor) on
// (score, index) with the lower index winning ties. In the softmax modes the
// selection runs on z, which orders the experts exactly as the softmax does.
// Per-block sums of the routing probabilities go to p_part in a fixed order,
// never through float atomics.
//
// With a group limit [cooking-agi, section on choosing groups first across
// devices] the token's group scores (sum of each expert group's top-m
// selection scores) are formed from a copy of its scores in LDS, the best
// groups are kept by a few more rounds of argmax, and the other groups'
// experts leave the candidate set before the top-k.
#include <math.h>

#include "common.hpp"
#include "dispatch_place.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;

// Router logits for a few tokens (bf16): one wave per (token, expert) dot
// product, 16-byte loads of both rows, fp32 products summed per lane in
// order and then across the wave by a fixed butterfly. For T·N small, where
// a tiled GEMM would compute mostly padding.
__global__ __launch_bounds__(256) void router_gemv_bf16_kernel(const bf16_t* __restrict__ h,
                                                               const bf16_t* __restrict__ w,
                                                               float* __restrict__ z, int T,
                                                               int d, int N) {
  const int64_t wv = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (wv >= (int64_t)T * N) return;
  const int t = (int)(wv / N), e = (int)(wv % N);
  const bf16_t* a = h + (int64_t)t * d;
  const bf16_t* b = w + (int64_t)e * d;
  float s = 0.0f;
  // four 512-element steps per pass, their loads issued before the first
  // fmaf; the products still add in order of c
  for (int c0 = lane * 8; c0 < d; c0 += 4 * 512) {
    u32x4 va[4], vb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = c0 + j * 512;
      va[j] = c < d ? *reinterpret_cast<const u32x4*>(a + c) : u32x4{0u, 0u, 0u, 0u};
      vb[j] = c < d ? *reinterpret_cast<const u32x4*>(b + c) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (c0 + j * 512 >= d) break;
      float x[8], y[8];
      unpack_bf16x8(va[j], x);
      unpack_bf16x8(vb[j], y);
#pragma unroll
      for (int i = 0; i < 8; ++i) s = fmaf(x[i], y[i], s);
    }
  }
  s = wave_sum(s);
  if (lane == 0) z[wv] = s;
}

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

// A group of LPT lanes routes one token (LPT = 8/16/32 for N up to that
// many experts, else 64); lane li of the group holds experts li, li+LPT, ...
// (VPL values). All reductions stay inside the group (xor offsets < LPT).
// Block blk of the selection (tokens [blk·TPB, (blk+1)·TPB)).
template <int LPT, int VPL, int MODE, int ITER>
__device__ __forceinline__ void route_select_block(
    int blk, const float* __restrict__ z_part, int splits, const float* __restrict__ b_router,
    const float* __restrict__ b_select, int32_t* __restrict__ ids,
    float* __restrict__ gates, float* __restrict__ p_part, float* __restrict__ zl_part, int T,
    int N, int k, GroupLimit gl, RouteFinal fin) {
  constexpr int TPW = 64 / LPT;               // tokens per wave per iteration
  constexpr int TPB = 4 * TPW * ITER;         // tokens per block
  constexpr int GPL = 64 / LPT;               // groups per lane at most (64 groups)
  __shared__ float s_p[4][64][VPL];
  __shared__ float s_g[4][64 * VPL];          // group scoring values of the wave's tokens
  __shared__ float s_zl[4][64][2];            // per-lane sums of lse^2 and entropy
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int grp = lane / LPT, li = lane % LPT;
  const int64_t TN = (int64_t)T * N;

  float pacc[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) pacc[i] = 0.0f;
  float zl_acc = 0.0f, ent_acc = 0.0f;        // this lane's tokens (lane li == 0)

  for (int it = 0; it < ITER; ++it) {
    const int t = blk * TPB + (it * 4 + w) * TPW + grp;
    const bool tok = t < T;
    // ---- logits: split-K slices summed in order, then the router bias
    float zv[VPL], sel[VPL], aux[VPL];
    bool cand[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = li + LPT * i;
      const bool in = tok && e < N;
      cand[i] = in;
      float v = 0.0f;
      if (in) {
        // every slice's load issued before the first add (splits <=
        // kRouterMaxSplits); the sum still runs in slice order
        const float* zp = z_part + (int64_t)t * N + e;
        float part[kRouterMaxSplits];
#pragma unroll
        for (int s = 0; s < kRouterMaxSplits; ++s) part[s] = s < splits ? zp[s * TN] : 0.0f;
#pragma unroll
        for (int s = 0; s < kRouterMaxSplits; ++s)
          if (s < splits) v += part[s];
        if (b_router) v += b_router[e];
      }
      zv[i] = v;
      if (MODE == 2) {
        const float sg = 1.0f / (1.0f + expf(-v));   // sigmoid score
        aux[i] = sg;
        sel[i] = in ? sg + b_select[e] : 0.0f;
      } else {
        aux[i] = v;
        sel[i] = v;
      }
      // a NaN score (a NaN in h, W_r or the biases) selects as -inf: the
      // token still gets k distinct experts, lowest indices first among
      // equals, and its gates come out NaN
      if (__builtin_isnan(sel[i])) sel[i] = -INFINITY;
    }
    // ---- group limit: keep the gl.keep best expert groups as candidates
    if (gl.n_groups > 0) {
      // scoring values: the selection score (mode C), or exp(z - zmax),
      // which is the softmax probability up to the token's common factor
      float zm = 0.0f;
      if (MODE != 2) {
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
          if (li + LPT * i < N) m = fmaxf(m, zv[i]);
#pragma unroll
        for (int o = LPT / 2; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
        zm = m;
      }
      float* gv = &s_g[w][grp * N];
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int e = li + LPT * i;
        if (e < N) gv[e] = MODE == 2 ? sel[i] : expf(zv[i] - zm);
      }
      __syncthreads();
      const int gsz = N / gl.n_groups;
      float gsc[GPL];
#pragma unroll
      for (int q = 0; q < GPL; ++q) {
        const int g = li + LPT * q;
        gsc[q] = -INFINITY;
        if (g < gl.n_groups) {
          float top[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) top[j] = -INFINITY;
          for (int x = 0; x < gsz; ++x) {          // insert into the sorted top-m
            float v = gv[g * gsz + x];
#pragma unroll
            for (int j = 0; j < 8; ++j)
              if (j < gl.topm && v > top[j]) {
                const float t0 = top[j];
                top[j] = v;
                v = t0;
              }
          }
          float sum = 0.0f;
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (j < gl.topm) sum += top[j];
          gsc[q] = __builtin_isnan(sum) ? -INFINITY : sum;
        }
      }
      uint64_t kept = 0;
      for (int r = 0; r < gl.keep; ++r) {
        float bv = -INFINITY;
        int bg = 0x7fffffff;
#pragma unroll
        for (int q = 0; q < GPL; ++q) {
          const int g = li + LPT * q;
          if (g < gl.n_groups && !((kept >> g) & 1) && better(gsc[q], g, bv, bg)) {
            bv = gsc[q];
            bg = g;
          }
        }
#pragma unroll
        for (int o = LPT / 2; o >= 1; o >>= 1) {
          const float ov = __shfl_xor(bv, o, 64);
          const int og = __shfl_xor(bg, o, 64);
          if (better(ov, og, bv, bg)) {
            bv = ov;
            bg = og;
          }
        }
        kept |= 1ull << bg;
      }
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int e = li + LPT * i;
        if (e < N && !((kept >> (e / gsz)) & 1)) cand[i] = false;
      }
      __syncthreads();                       // before the next tokens reuse s_g
    }
    // ---- top-k: k rounds of a group-wide argmax, lower index wins ties;
    //      lane j of the group keeps the j-th winner (k <= LPT)
    int my_id = 0;
    float my_aux = 0.0f, aux0 = 0.0f;
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY, ba = 0.0f;
      int bi = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int e = li + LPT * i;
        if (cand[i] && better(sel[i], e, bv, bi)) {
          bv = sel[i];
          bi = e;
          ba = aux[i];
        }
      }
#pragma unroll
      for (int o = LPT / 2; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        const float oa = __shfl_xor(ba, o, 64);
        if (better(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
          ba = oa;
        }
      }
      if (bi % LPT == li) {                  // the owner drops the winner
#pragma unroll
        for (int i = 0; i < VPL; ++i)
          if (i == bi / LPT) cand[i] = false;
      }
      if (li == j) {
        my_id = bi;
        my_aux = ba;
      }
      if (j == 0) aux0 = ba;                 // the largest selected
    }
    // ---- full-softmax max and denominator (mode B gates, p statistics,
    //      z-loss)
    float zmax = 0.0f, denom_all = 1.0f;
    const bool need_full = (MODE == 1) || (p_part != nullptr) || (zl_part != nullptr);
    if (need_full) {
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (li + LPT * i < N) m = fmaxf(m, zv[i]);
#pragma unroll
      for (int o = LPT / 2; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      zmax = m;
      float sum = 0.0f;
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (li + LPT * i < N) sum += expf(zv[i] - zmax);
#pragma unroll
      for (int o = LPT / 2; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 64);
      denom_all = sum;
    }
    // ---- router z-loss term (log-sum-exp of the logits)^2 and the entropy
    //      of the routing distribution [wuhy-notes §五 Router z-loss]
    if (zl_part) {
      const float lse = zmax + logf(denom_all);
      float ent;
      if (MODE != 2) {
        // H = lse - sum_i p_i z_i
        float pz = 0.0f;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
          if (li + LPT * i < N) pz += expf(zv[i] - zmax) * zv[i];
#pragma unroll
        for (int o = LPT / 2; o >= 1; o >>= 1) pz += __shfl_xor(pz, o, 64);
        ent = lse - pz / denom_all;
      } else {
        // q = s / S: H = log S - sum_i s_i log s_i / S
        float ss = 0.0f, sls = 0.0f;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
          if (li + LPT * i < N) {
            ss += aux[i];
            sls += aux[i] > 0.0f ? aux[i] * logf(aux[i]) : 0.0f;
          }
#pragma unroll
        for (int o = LPT / 2; o >= 1; o >>= 1) {
          ss += __shfl_xor(ss, o, 64);
          sls += __shfl_xor(sls, o, 64);
        }
        ent = logf(ss) - sls / ss;
      }
      if (tok && li == 0) {
        zl_acc += lse * lse;
        ent_acc += ent;
      }
    }
    // ---- gates of the selected (lane li < k holds slot li), the sums over
    //      the k slots by the group's butterfly; correctly rounded divisions,
    //      so that one selected expert gets a gate of exactly 1 (a product
    //      with a rounded reciprocal can miss it by an ulp, and the backward's
    //      renormalisation term, exactly 0 then, would carry that ulp times
    //      dL/dg into the router gradient)
    float my_g;
    if (MODE == 0) {
      // softmax over the selected logits (aux0 is the largest)
      const float ex = li < k ? expf(my_aux - aux0) : 0.0f;
      float sum = ex;
#pragma unroll
      for (int o = LPT / 2; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 64);
      my_g = ex / sum;
    } else if (MODE == 1) {
      my_g = expf(my_aux - zmax) / denom_all;
    } else {
      float sum = li < k ? my_aux : 0.0f;
#pragma unroll
      for (int o = LPT / 2; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 64);
      my_g = my_aux / sum;
    }
    if (tok && li < k) {
      ids[(int64_t)t * k + li] = my_id;
      gates[(int64_t)t * k + li] = my_g;
    }
    // ---- routing probabilities for p_i
    if (p_part) {
      if (MODE == 2) {
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
          if (li + LPT * i < N) sum += aux[i];
#pragma unroll
        for (int o = LPT / 2; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 64);
        const float inv = 1.0f / sum;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
          if (tok && li + LPT * i < N) pacc[i] += aux[i] * inv;
      } else {
        const float inv = 1.0f / denom_all;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
          if (tok && li + LPT * i < N) pacc[i] += expf(zv[i] - zmax) * inv;
      }
    }
  }
  if (zl_part) {
    // block sums in a fixed order: waves, then token groups
    s_zl[w][lane][0] = zl_acc;
    s_zl[w][lane][1] = ent_acc;
    __syncthreads();
    if (tid < 2) {
      float sum = 0.0f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww)
#pragma unroll
        for (int g = 0; g < TPW; ++g) sum += s_zl[ww][g * LPT][tid];
      zl_part[(int64_t)blk * 2 + tid] = sum;
      float* out = tid == 0 ? fin.z_loss : fin.entropy;
      if (fin.on && out) *out = sum / (float)T;
    }
  }
  if (p_part) {
#pragma unroll
    for (int i = 0; i < VPL; ++i) s_p[w][lane][i] = pacc[i];
    __syncthreads();
    // block sum per expert: waves in order, token groups in order
    for (int e = tid; e < N; e += kThreads) {
      float sum = 0.0f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww)
#pragma unroll
        for (int g = 0; g < TPW; ++g) sum += s_p[ww][g * LPT + e % LPT][e / LPT];
      p_part[(int64_t)blk * N + e] = sum;
      if (fin.on && fin.p_mean) fin.p_mean[e] = sum / (float)T;
    }
  }
}

template <int LPT, int VPL, int MODE, int ITER>
__global__ __launch_bounds__(kThreads) void route_select_kernel(
    const float* __restrict__ z_part, int splits, const float* __restrict__ b_router,
    const float* __restrict__ b_select, int32_t* __restrict__ ids,
    float* __restrict__ gates, float* __restrict__ p_part, float* __restrict__ zl_part, int T,
    int N, int k, GroupLimit gl, RouteFinal fin) {
  route_select_block<LPT, VPL, MODE, ITER>(blockIdx.x, z_part, splits, b_router, b_select, ids,
                                           gates, p_part, zl_part, T, N, k, gl, fin);
}

// Selection and dispatch of a batch that fits one selection block and one
// dispatch chunk, in one block: the selection writes ids, gates and the
// final statistics, then (after a block barrier, which makes those global
// writes visible to the whole block) the same block places the slots. The
// results are those of the two separate kernels, bit for bit.
template <int LPT, int VPL, int MODE, int ITER>
__global__ __launch_bounds__(kThreads) void route_dispatch_kernel(
    const float* __restrict__ z_part, int splits, const float* __restrict__ b_router,
    const float* __restrict__ b_select, int32_t* __restrict__ ids,
    float* __restrict__ gates, float* __restrict__ p_part, float* __restrict__ zl_part, int T,
    int N, int k, GroupLimit gl, RouteFinal fin, DispatchOut dq) {
  route_select_block<LPT, VPL, MODE, ITER>(0, z_part, splits, b_router, b_select, ids, gates,
                                           p_part, zl_part, T, N, k, gl, fin);
  __syncthreads();
  dsp::place_chunk(0, ids, T, k, N, nullptr, 1, dq.counts, dq.offsets, dq.perm_src, dq.row_of,
                   fin.p_mean, dq.f_out, dq.l_aux, dq.alpha, dq.cap, dq.cap_stats, dq.zero,
                   dq.zero_n);
}

// p_mean[e] = (sum over blocks of p_part[b][e]) / T: one block per expert,
// thread i sums blocks i, i+256, ... in order, then a fixed tree.
// Blocks past the first n_p (when zl_part is given): z_loss and entropy as
// the sums of the per-block partials over T, by the same fixed tree.
__global__ __launch_bounds__(kThreads) void p_reduce_kernel(const float* __restrict__ p_part,
                                                            float* __restrict__ p_mean,
                                                            const float* __restrict__ zl_part,
                                                            float* __restrict__ z_loss,
                                                            float* __restrict__ entropy, int n_p,
                                                            int blocks, int T, int N) {
  __shared__ float s[2][kThreads];
  const int tid = threadIdx.x;
  const bool scalars = (int)blockIdx.x >= n_p;
  const int e = blockIdx.x;
  float v0 = 0.0f, v1 = 0.0f;
  for (int b = tid; b < blocks; b += kThreads) {
    if (scalars) {
      v0 += zl_part[(int64_t)b * 2];
      v1 += zl_part[(int64_t)b * 2 + 1];
    } else {
      v0 += p_part[(int64_t)b * N + e];
    }
  }
  s[0][tid] = v0;
  s[1][tid] = v1;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (tid < o) {
      s[0][tid] += s[0][tid + o];
      s[1][tid] += s[1][tid + o];
    }
    __syncthreads();
  }
  if (tid == 0) {
    if (!scalars) {
      p_mean[e] = s[0][0] / (float)T;
    } else {
      if (z_loss) *z_loss = s[0][0] / (float)T;
      if (entropy) *entropy = s[1][0] / (float)T;
    }
  }
}

// Launch configuration of route_select for N experts.
struct SelectCfg {
  int lpt, vpl, iter, tpb;
};
// Up to 64 experts: one expert per lane (8, 16, 32 or 64 lanes per token).
// More: four per lane up to 256 experts (32 or 64 lanes), eight beyond (64
// lanes), so that a token's reductions take few shuffle steps. A block
// routes each of its groups' tokens once (ITER 1) for batches of more than
// 16 tokens, so that there are many short blocks; batches of up to 16
// tokens loop ITER times so that one block routes them all (the single-block
// selection + dispatch kernel).
SelectCfg select_cfg(int T, int N) {
  SelectCfg c;
  if (N <= 64) {
    c.lpt = N <= 8 ? 8 : N <= 16 ? 16 : N <= 32 ? 32 : 64;
    c.vpl = 1;
  } else {
    c.lpt = N <= 128 ? 32 : 64;
    c.vpl = N <= 256 ? 4 : 8;
  }
  const int tpw = 64 / c.lpt;
  c.iter = (T > 16 || 4 * tpw >= 16) ? 1 : 16 / (4 * tpw);
  c.tpb = 4 * tpw * c.iter;
  return c;
}

// dq == NULL: the selection kernel (blocks of it); else the single-block
// selection + dispatch kernel
template <int LPT, int VPL, int MODE, int ITER>
void launch_select_m(const float* z_part, int splits, const float* b_router,
                     const float* b_select, int32_t* ids, float* gates, float* p_part,
                     float* zl_part, int T, int N, int k, GroupLimit gl, int blocks,
                     RouteFinal fin, const DispatchOut* dq, hipStream_t st) {
  if (dq)
    hipLaunchKernelGGL((route_dispatch_kernel<LPT, VPL, MODE, ITER>), dim3(1), dim3(kThreads), 0,
                       st, z_part, splits, b_router, b_select, ids, gates, p_part, zl_part, T, N,
                       k, gl, fin, *dq);
  else
    hipLaunchKernelGGL((route_select_kernel<LPT, VPL, MODE, ITER>), dim3(blocks), dim3(kThreads),
                       0, st, z_part, splits, b_router, b_select, ids, gates, p_part, zl_part, T,
                       N, k, gl, fin);
}

template <int LPT, int VPL, int ITER>
hipError_t launch_select_t(const float* z_part, int splits, const float* b_router,
                           const float* b_select, int32_t* ids, float* gates, float* p_part,
                           float* zl_part, int T, int N, int k, int mode, GroupLimit gl,
                           int blocks, RouteFinal fin, const DispatchOut* dq, hipStream_t st) {
  switch (mode) {
    case 0:
      launch_select_m<LPT, VPL, 0, ITER>(z_part, splits, b_router, b_select, ids, gates, p_part,
                                         zl_part, T, N, k, gl, blocks, fin, dq, st);
      break;
    case 1:
      launch_select_m<LPT, VPL, 1, ITER>(z_part, splits, b_router, b_select, ids, gates, p_part,
                                         zl_part, T, N, k, gl, blocks, fin, dq, st);
      break;
    default:
      launch_select_m<LPT, VPL, 2, ITER>(z_part, splits, b_router, b_select, ids, gates, p_part,
                                         zl_part, T, N, k, gl, blocks, fin, dq, st);
      break;
  }
  return hipGetLastError();
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

bool router_use_gemv(int T, int N) { return T <= 64 && (int64_t)T * N <= 2048; }

hipError_t launch_router_gemv_bf16(const void* h, const void* w, float* z, int T, int d, int N,
                                   hipStream_t st) {
  const int64_t waves = (int64_t)T * N;
  if (waves == 0) return hipSuccess;
  hipLaunchKernelGGL(router_gemv_bf16_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                     st, static_cast<const bf16_t*>(h), static_cast<const bf16_t*>(w), z, T, d,
                     N);
  return hipGetLastError();
}

int route_select_blocks(int T, int N) {
  const SelectCfg c = select_cfg(T, N);
  return (T + c.tpb - 1) / c.tpb;
}

hipError_t launch_route_select(const float* z_part, int splits, const float* b_router,
                               const float* b_select, int32_t* ids, float* gates,
                               float* p_part, float* zl_part, int T, int N, int k, int mode,
                               GroupLimit gl, RouteFinal fin, hipStream_t st,
                               const DispatchOut* dq) {
  const SelectCfg c = select_cfg(T, N);
  const int blocks = (T + c.tpb - 1) / c.tpb;
  if (blocks == 0) return hipSuccess;
  if (splits < 1 || splits > kRouterMaxSplits) return hipErrorInvalidValue;
  if (k > c.lpt) return hipErrorInvalidValue;   // a lane per selected slot (k <= 16 <= LPT, or k <= N <= LPT)
  fin.on = fin.on && blocks == 1;
  if (dq) {
    // the fused kernel is one block; its dispatch reads the p_mean it wrote
    if (blocks != 1 || dispatch_chunks(T, k) != 1) return hipErrorInvalidValue;
    fin.on = 1;
  }
#define MOE_SEL(L, V, I)                                                                    \
  if (c.lpt == L && c.vpl == V && c.iter == I)                                             \
    return launch_select_t<L, V, I>(z_part, splits, b_router, b_select, ids, gates, p_part, \
                                    zl_part, T, N, k, mode, gl, blocks, fin, dq, st);
  MOE_SEL(8, 1, 1)
  MOE_SEL(16, 1, 1)
  MOE_SEL(32, 1, 1)
  MOE_SEL(32, 1, 2)
  MOE_SEL(64, 1, 1)
  MOE_SEL(64, 1, 4)
  MOE_SEL(32, 4, 1)
  MOE_SEL(32, 4, 2)
  MOE_SEL(64, 4, 1)
  MOE_SEL(64, 4, 4)
  MOE_SEL(64, 8, 1)
  MOE_SEL(64, 8, 4)
#undef MOE_SEL
  return hipErrorInvalidValue;
}

hipError_t launch_p_reduce(const float* p_part, float* p_mean, const float* zl_part,
                           float* z_loss, float* entropy, int blocks, int T, int N,
                           hipStream_t st) {
  if (T == 0 || N == 0) return hipSuccess;
  const int n_p = p_mean ? N : 0;
  const int grid = n_p + ((z_loss || entropy) ? 1 : 0);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(p_reduce_kernel, dim3(grid), dim3(kThreads), 0, st, p_part, p_mean,
                     zl_part, z_loss, entropy, n_p, blocks, T, N);
  return hipGetLastError();
}

}  // namespace moe
