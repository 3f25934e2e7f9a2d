// Backward pass of the layer: the kernels around the GEMMs.
//
// For the forward pass's selection and dispatch, the gradient of
// <dy, y> + d_laux L_aux + d_zloss L_z follows the chain rule of the forward
// steps. The router learns only through the gate values of the selected
// experts, and through every logit that a normalisation involves (the full
// softmax of mode B) [page "MoE：router 怎样选 expert" (cooking-agi), section
// "top-k 不可导，router 怎么学"; page "MOE 专家选择与路由机制" (wuhy-notes),
// "Top-k 不可导，为什么 Router 还能学" and the total-loss paragraph].
//
// Per kept bucket row r (token t, slot j, expert e, gate g):
//   v_r     = W_down^(e)^T dy_t                       (GEMM, elsewhere; fp32)
//   dg_tj   = <v_r, act_r> = <dy_t, E_e(h_t)>          (swiglu_bwd_kernel)
//   dact_r  = g v_r; du = dact SiLU(gp); dgp = dact up SiLU'(gp)
//   dh rows = W_gate^T dgp + W_up^T du                 (GEMM)
// and per token the router-logit gradient dz_t (route_bwd_kernel). Weight
// gradients are GEMMs over each expert's rows, taken as K ranges of
// transposed, zero-padded copies of the row-major activations (pack_t).
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

template <typename TE>
__device__ __forceinline__ float ld(const TE* p, int64_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<bf16_t>(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

template <typename TE>
__device__ __forceinline__ void st(TE* p, int64_t i, float v);
template <>
__device__ __forceinline__ void st<float>(float* p, int64_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void st<bf16_t>(bf16_t* p, int64_t i, float v) {
  p[i] = (bf16_t)f32_to_bf16(v);
}

template <typename TE>
__device__ __forceinline__ TE from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return (bf16_t)f32_to_bf16(v); }

constexpr int kT = 256;

// kofs[e] = sum over e' < e of the kept rows of e' rounded up to 64 (the
// padded K range of expert e in the transposed copies: whole 64-deep slabs
// of the weight-gradient GEMMs); with no offsets one range of n_single rows.
__global__ __launch_bounds__(kT) void kofs_kernel(const int32_t* __restrict__ offsets, int G,
                                                  int n_single, int32_t* __restrict__ kofs) {
  __shared__ int s_wave[kT / 64];
  if (!offsets) {
    if (threadIdx.x == 0) {
      kofs[0] = 0;
      kofs[1] = (n_single + 63) & ~63;
    }
    return;
  }
  // G <= 512: two entries per thread, in order
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int c[2], sum = 0;
  for (int i = 0; i < 2; ++i) {
    const int e = 2 * tid + i;
    c[i] = e < G ? ((offsets[e + 1] - offsets[e] + 63) & ~63) : 0;
    sum += c[i];
  }
  int incl = sum;
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) s_wave[w] = incl;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < w; ++i) base += s_wave[i];
  int run = base + incl - sum;
  for (int i = 0; i < 2; ++i) {
    const int e = 2 * tid + i;
    if (e < G) kofs[e] = run;
    run += c[i];
    if (e == G - 1) kofs[G] = run;
  }
}

// Transposed, padded copy: dst[c][kofs[e] + i] = scale * src[row][c] for the
// i-th kept row of expert e (bucket row r = offsets[e] + i; source row
// perm[r] / kdiv, or r without perm; scale = scale[perm[r]] (or [r]), or 1),
// zero in the padding of each range and up to p_limit. A block moves a tile
// of 64 padded rows p x 64 columns c: the 64 rows' sources are resolved once
// into LDS, each row segment is read with 16-byte loads, the tile is staged
// in LDS (row pitch padded against bank conflicts) and written out along p
// with 16-byte stores. Grid (p_limit / 64, ncols / 64, batch): batch b reads
// src + b * src_bstride and writes dst + b * dst_bstride (per-expert weight
// copies). VEC: rows and strides allow 16-byte accesses (the launcher
// checks); otherwise element by element.
template <typename TE, bool VEC>
__global__ __launch_bounds__(kT) void pack_t_kernel(
    const TE* __restrict__ src, int ld_src, int ncols, const int32_t* __restrict__ perm,
    int kdiv, const float* __restrict__ scale, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ kofs, int G, int n_single, int64_t p_limit, TE* __restrict__ dst,
    int64_t ld_dst, int64_t src_bstride, int64_t dst_bstride) {
  constexpr int V = VEC ? 16 / sizeof(TE) : 1;   // elements per access
  constexpr int PITCH = 66;                   // LDS row pitch (elements): no bank conflicts
  __shared__ TE tile[64][PITCH];
  __shared__ int64_t s_row[64];
  __shared__ float s_scale[64];
  const int tid = threadIdx.x;
  src += blockIdx.z * src_bstride;
  dst += blockIdx.z * dst_bstride;
  const int64_t p0 = (int64_t)blockIdx.x * 64;
  const int c0 = blockIdx.y * 64;
  if (tid < 64) {
    const int64_t p = p0 + tid;
    int64_t srow = -1;
    float sc = 1.0f;
    if (offsets) {
      if (p < kofs[G]) {
        int lo = 0, hi = G;              // kofs[lo] <= p < kofs[hi]
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (kofs[mid] <= p) lo = mid; else hi = mid;
        }
        const int64_t local = p - kofs[lo];
        if (local < offsets[lo + 1] - offsets[lo]) {
          const int64_t r = offsets[lo] + local;
          srow = perm ? perm[r] / kdiv : r;
          if (scale) sc = scale[perm ? perm[r] : r];
        }
      }
    } else if (p < n_single) {
      srow = p;
      if (scale) sc = scale[p];
    }
    s_row[tid] = srow;
    s_scale[tid] = sc;
  }
  __syncthreads();
  // load: 64 rows x 64 columns = 64 x (64 / V) vectors
  constexpr int VPR = 64 / V;                 // vectors per row
  for (int q = tid; q < 64 * VPR; q += kT) {
    const int row = q / VPR, cv = (q % VPR) * V;
    const int64_t srow = s_row[row];
    const int c = c0 + cv;
    TE vals[V];
    if (srow >= 0 && c < ncols) {
      const float sc = s_scale[row];
      if constexpr (VEC) {
        // may read past ncols, never past the row (ld_src is a multiple of V)
        const u32x4 raw = *reinterpret_cast<const u32x4*>(src + srow * ld_src + c);
        const TE* e = reinterpret_cast<const TE*>(&raw);
#pragma unroll
        for (int i = 0; i < V; ++i) vals[i] = sc == 1.0f ? e[i] : from_f32<TE>(sc * ld(e, i));
      } else {
        const TE e = src[srow * ld_src + c];
        vals[0] = sc == 1.0f ? e : from_f32<TE>(sc * ld(&e, 0));
      }
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) vals[i] = from_f32<TE>(0.0f);
    }
#pragma unroll
    for (int i = 0; i < V; ++i) tile[row][cv + i] = vals[i];
  }
  __syncthreads();
  // store: 64 columns x 64 rows = 64 x (64 / V) vectors along p
  for (int q = tid; q < 64 * VPR; q += kT) {
    const int col = q / VPR, pv = (q % VPR) * V;
    const int c = c0 + col;
    const int64_t p = p0 + pv;
    if (c >= ncols || p >= p_limit) continue;
    if constexpr (VEC) {
      TE vals[V];
#pragma unroll
      for (int i = 0; i < V; ++i) vals[i] = tile[pv + i][col];
      *reinterpret_cast<u32x4*>(dst + (int64_t)c * ld_dst + p) =
          *reinterpret_cast<const u32x4*>(vals);
    } else {
      dst[(int64_t)c * ld_dst + p] = tile[pv][col];
    }
  }
}

// One block per bucket row r < rows (rows = offsets[G], or the grid):
// gu[r] = [gp | up] and v[r] in fp32; act[r] = SiLU(gp) up and
// dgu[r] = [dgp | du] out in the layer dtype; dg_slot[perm[r]] = <v_r, act_r>
// in fp32 from the fp32 inputs (fixed-order block reduction). The
// pre-activations and v stay fp32 because dg is a dot product that can
// cancel.
template <typename TO>
__global__ __launch_bounds__(kT) void swiglu_bwd_kernel(
    const float* __restrict__ gu, const float* __restrict__ v, TO* __restrict__ act,
    TO* __restrict__ dgu, const int32_t* __restrict__ perm, const float* __restrict__ gates,
    float* __restrict__ dg_slot, const int32_t* __restrict__ offsets, int G, int d_ff) {
  __shared__ float s_red[kT];
  const int64_t r = blockIdx.x;
  if (offsets && r >= offsets[G]) return;
  const int tid = threadIdx.x;
  const float g = gates ? gates[perm[r]] : 1.0f;
  const float* gr = gu + r * 2 * d_ff;
  const float* vr = v + r * d_ff;
  TO* ar = act + r * d_ff;
  TO* dr = dgu + r * 2 * d_ff;
  float dot = 0.0f;
  for (int j = tid; j < d_ff; j += kT) {
    const float gp = gr[j], up = gr[d_ff + j], vv = vr[j];
    const float s = 1.0f / (1.0f + expf(-gp));
    const float si = gp * s;
    const float a = si * up;
    dot = fmaf(vv, a, dot);
    const float dact = g * vv;
    st(ar, j, a);
    st(dr, j, dact * up * s * (1.0f + gp * (1.0f - s)));
    st(dr, d_ff + j, dact * si);
  }
  if (!dg_slot) return;
  s_red[tid] = dot;
  __syncthreads();
  for (int o = kT / 2; o > 0; o >>= 1) {
    if (tid < o) s_red[tid] += s_red[tid + o];
    __syncthreads();
  }
  if (tid == 0) dg_slot[perm[r]] = s_red[0];
}

// The routed rows' SwiGLU backward written for both of its consumers: the
// row-major [dgp | du] (A of the h-row GEMM) and the transposed, padded
// copies act^T [d_ff rows][ld_t] and [dgp | du]^T [2 d_ff rows][ld_t] that
// the weight-gradient GEMMs read as K ranges (pack_t's layout: index p =
// kofs[e] + i for the i-th kept row of expert e, zeros in the padding, up to
// p_limit). The values are swiglu_bwd_kernel's. A block takes 64 indices p
// and kTC columns c: the rows behind its p are resolved once into LDS, gu
// and v are read along c (one row per wave and pass), the results staged in
// LDS and written along p with 16-byte stores (64-column tiles measured
// faster than 128-column ones: 0.64 against 0.79 ms at the Mixtral shape).
// dg_part[ct * ld_dg + r] is the fp32 dot <v_r, act_r> over column tile ct,
// summed over its columns in a fixed butterfly order; dg_reduce_kernel adds
// a row's tiles in order.
constexpr int kTC = 64;    // columns per tile (one per lane)
template <typename TO>
__global__ __launch_bounds__(kT) void swiglu_bwd_t_kernel(
    const float* __restrict__ gu, const float* __restrict__ v, TO* __restrict__ dgu,
    TO* __restrict__ act_t, TO* __restrict__ dgu_t, int64_t ld_t,
    const int32_t* __restrict__ perm, const float* __restrict__ gates,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ kofs, int G,
    int64_t p_limit, int d_ff, float* __restrict__ dg_part, int64_t ld_dg) {
  constexpr int V = 16 / sizeof(TO);           // elements per 16-byte store
  constexpr int PITCH = kTC + 2;               // LDS row pitch (elements)
  __shared__ TO s_t[3][64][PITCH];             // act, dgp, du of [p][c]
  __shared__ int64_t s_row[64];
  __shared__ float s_g[64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t p0 = (int64_t)blockIdx.x * 64;
  const int c0 = blockIdx.y * kTC, ct = blockIdx.y;
  if (tid < 64) {
    const int64_t pp = p0 + tid;
    int64_t r = -1;
    if (pp < kofs[G]) {
      int lo = 0, hi = G;                      // kofs[lo] <= pp < kofs[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (kofs[mid] <= pp) lo = mid; else hi = mid;
      }
      const int64_t local = pp - kofs[lo];
      if (local < offsets[lo + 1] - offsets[lo]) r = offsets[lo] + local;
    }
    s_row[tid] = r;
    s_g[tid] = r >= 0 ? gates[perm[r]] : 0.0f;
  }
  __syncthreads();
  // rows i = w, w + 4, ...: lane = column
  const int c = c0 + lane;
#pragma unroll 4
  for (int i = w; i < 64; i += 4) {
    const int64_t r = s_row[i];
    float a = 0.0f, dgp = 0.0f, du = 0.0f, dot = 0.0f;
    if (r >= 0 && c < d_ff) {
      const float* gr = gu + r * 2 * d_ff;
      const float gp = gr[c], up = gr[d_ff + c], vv = v[r * d_ff + c];
      const float sg = 1.0f / (1.0f + expf(-gp));
      const float si = gp * sg;
      a = si * up;
      dot = vv * a;
      const float dact = s_g[i] * vv;
      dgp = dact * up * sg * (1.0f + gp * (1.0f - sg));
      du = dact * si;
      TO* dr = dgu + r * 2 * d_ff;
      st(dr, c, dgp);
      st(dr, d_ff + c, du);
    }
    s_t[0][i][lane] = from_f32<TO>(a);
    s_t[1][i][lane] = from_f32<TO>(dgp);
    s_t[2][i][lane] = from_f32<TO>(du);
    if (r >= 0) {
      dot = wave_sum(dot);                     // columns past d_ff add 0
      if (lane == 0) dg_part[ct * ld_dg + r] = dot;
    }
  }
  __syncthreads();
  // transposed stores: lane -> (column, V consecutive p); each wave pass
  // covers V columns
  constexpr int LPC = 64 / V;                  // lanes per column
  const int cc_l = lane / LPC, pv = (lane % LPC) * V;
  for (int cb = w * V; cb < kTC; cb += 4 * V) {
    const int cx = cb + cc_l;
    const int col = c0 + cx;
    if (col >= d_ff) continue;
#pragma unroll
    for (int m = 0; m < 3; ++m) {
      TO vals[V];
#pragma unroll
      for (int e = 0; e < V; ++e) vals[e] = s_t[m][pv + e][cx];
      TO* dst = m == 0 ? act_t + (int64_t)col * ld_t
                       : dgu_t + ((int64_t)(m == 1 ? col : d_ff + col)) * ld_t;
      *reinterpret_cast<u32x4*>(dst + p0 + pv) = *reinterpret_cast<const u32x4*>(vals);
    }
  }
}

// The same outputs for bf16 layers (d_ff a multiple of 64) whose fp32
// pre-activations and v are 16-byte aligned (the kernel above serves the
// others and the fp32 layers), with 16-byte loads: a
// lane takes four adjacent columns of a row (16 lanes per row of the 64-column
// tile, four rows per wave and pass), so that each thread has twelve 16-byte
// loads in flight instead of twelve 4-byte ones. The tile's partial
// <v_r, act_r> adds the rounded products v·act (no fused multiply-add) with
// the butterfly of the one-column-per-lane form: columns c and c ^ 32, ^ 16,
// ^ 8, ^ 4 across lanes (lane ^ 8, ^ 4, ^ 2, ^ 1), then ^ 2 and ^ 1 inside
// the lane. Mixtral prefill shape (R = 8192, d_ff = 14,336, 2.6 GB moved):
// 565-575 against 620-675 us.
__global__ __launch_bounds__(kT) void swiglu_bwd_t4_kernel(
    const float* __restrict__ gu, const float* __restrict__ v, bf16_t* __restrict__ dgu,
    bf16_t* __restrict__ act_t, bf16_t* __restrict__ dgu_t, int64_t ld_t,
    const int32_t* __restrict__ perm, const float* __restrict__ gates,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ kofs, int G,
    int64_t p_limit, int d_ff, float* __restrict__ dg_part, int64_t ld_dg) {
  constexpr int PITCH = kTC + 4;               // 8-byte aligned staged rows
  __shared__ __attribute__((aligned(16))) bf16_t s_t[3][64][PITCH];   // act, dgp, du of [p][c]
  __shared__ int64_t s_row[64];
  __shared__ float s_g[64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t p0 = (int64_t)blockIdx.x * 64;
  const int c0 = blockIdx.y * kTC, ct = blockIdx.y;
  if (tid < 64) {
    const int64_t pp = p0 + tid;
    int64_t r = -1;
    if (pp < kofs[G]) {
      int lo = 0, hi = G;                      // kofs[lo] <= pp < kofs[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (kofs[mid] <= pp) lo = mid; else hi = mid;
      }
      const int64_t local = pp - kofs[lo];
      if (local < offsets[lo + 1] - offsets[lo]) r = offsets[lo] + local;
    }
    s_row[tid] = r;
    s_g[tid] = r >= 0 ? gates[perm[r]] : 0.0f;
  }
  __syncthreads();
  const int cl = (lane & 15) * 4;              // first of the lane's four columns
  const int c = c0 + cl;
  const bool cok = c < d_ff;                   // d_ff % 4 == 0: all four or none
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int i = 16 * pass + 4 * w + (lane >> 4);
    const int64_t r = s_row[i];
    f32x4 gp = {0.0f, 0.0f, 0.0f, 0.0f}, up = gp, vv = gp;
    if (r >= 0 && cok) {
      const float* gr = gu + r * 2 * d_ff;
      gp = *reinterpret_cast<const f32x4*>(gr + c);
      up = *reinterpret_cast<const f32x4*>(gr + d_ff + c);
      vv = *reinterpret_cast<const f32x4*>(v + r * d_ff + c);
    }
    const float g = s_g[i];
    float a[4], dgp[4], du[4], dot[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float sg = 1.0f / (1.0f + expf(-gp[j]));
      const float si = gp[j] * sg;
      a[j] = si * up[j];
      dot[j] = __fmul_rn(vv[j], a[j]);
      const float dact = g * vv[j];
      dgp[j] = dact * up[j] * sg * (1.0f + gp[j] * (1.0f - sg));
      du[j] = dact * si;
    }
    const u32x2 pa = {f32_to_bf16(a[0]) | (f32_to_bf16(a[1]) << 16),
                      f32_to_bf16(a[2]) | (f32_to_bf16(a[3]) << 16)};
    const u32x2 pg = {f32_to_bf16(dgp[0]) | (f32_to_bf16(dgp[1]) << 16),
                      f32_to_bf16(dgp[2]) | (f32_to_bf16(dgp[3]) << 16)};
    const u32x2 pu = {f32_to_bf16(du[0]) | (f32_to_bf16(du[1]) << 16),
                      f32_to_bf16(du[2]) | (f32_to_bf16(du[3]) << 16)};
    if (r >= 0 && cok) {
      bf16_t* dr = dgu + r * 2 * d_ff;
      *reinterpret_cast<u32x2*>(dr + c) = pg;
      *reinterpret_cast<u32x2*>(dr + d_ff + c) = pu;
    }
    *reinterpret_cast<u32x2*>(&s_t[0][i][cl]) = pa;
    *reinterpret_cast<u32x2*>(&s_t[1][i][cl]) = pg;
    *reinterpret_cast<u32x2*>(&s_t[2][i][cl]) = pu;
    // every lane of the 16-lane row group takes part (columns past d_ff and
    // padding rows add zeros); only the group's first lane stores
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) dot[j] += __shfl_xor(dot[j], o, kWave);
    const float s = (dot[0] + dot[2]) + (dot[1] + dot[3]);
    if (r >= 0 && (lane & 15) == 0) dg_part[ct * ld_dg + r] = s;
  }
  __syncthreads();
  // transposed stores as in swiglu_bwd_t_kernel: lane -> (column, 8
  // consecutive p); each wave pass covers 8 columns
  const int cc_l = lane >> 3, pv = (lane & 7) * 8;
  for (int cb = w * 8; cb < kTC; cb += 32) {
    const int cx = cb + cc_l;
    const int col = c0 + cx;
    if (col >= d_ff) continue;
#pragma unroll
    for (int m = 0; m < 3; ++m) {
      bf16_t vals[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) vals[e] = s_t[m][pv + e][cx];
      bf16_t* dst = m == 0 ? act_t + (int64_t)col * ld_t
                           : dgu_t + ((int64_t)(m == 1 ? col : d_ff + col)) * ld_t;
      *reinterpret_cast<u32x4*>(dst + p0 + pv) = *reinterpret_cast<const u32x4*>(vals);
    }
  }
}

// dg_slot[perm[r]] = sum over column tiles ct (in order) of dg_part[ct][r];
// the loads of eight tiles are issued together.
__global__ __launch_bounds__(kT) void dg_reduce_kernel(const float* __restrict__ dg_part,
                                                       int nct, int64_t ld_dg,
                                                       const int32_t* __restrict__ perm,
                                                       const int32_t* __restrict__ offsets,
                                                       int G, float* __restrict__ dg_slot) {
  const int64_t r = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (r >= offsets[G]) return;
  float s = 0.0f;
  int i = 0;
  for (; i + 8 <= nct; i += 8) {
    float q[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = dg_part[(i + j) * ld_dg + r];
#pragma unroll
    for (int j = 0; j < 8; ++j) s += q[j];
  }
  for (; i < nct; ++i) s += dg_part[i * ld_dg + r];
  dg_slot[perm[r]] = s;
}

// One wave per token: router-logit gradient dz_t [N] (fp32 and a bf16 copy
// zero-padded to ldzb columns). z_t is re-formed from the split-K slices in
// the forward's order. Task part through the selected gates (dg of a
// dropped slot is 0); L_aux part (f_i = counts_i / (T k) constant, p_i the
// mean routing probability); z-loss part (2 / T) LSE_t softmax(z_t).
constexpr int kMaxPerLane = 8;   // N <= 512
template <typename TZ>
__global__ __launch_bounds__(64) void route_bwd_kernel(
    const float* __restrict__ z_part, int splits, const float* __restrict__ b_router,
    const int32_t* __restrict__ ids, const float* __restrict__ gates,
    const float* __restrict__ dg_slot, const int32_t* __restrict__ row_of,
    const int32_t* __restrict__ counts, int T, int N, int k, int mode, float alpha,
    float d_laux, float d_zloss, float* __restrict__ dz, TZ* __restrict__ dzb, int ldzb,
    float* __restrict__ dg_out) {
  const int t = blockIdx.x, lane = threadIdx.x;
  const int64_t TN = (int64_t)T * N;
  float z[kMaxPerLane], dzl[kMaxPerLane];
  float m = -INFINITY;
#pragma unroll
  for (int q = 0; q < kMaxPerLane; ++q) {
    const int i = lane + 64 * q;
    float v = -INFINITY;
    if (i < N) {
      // the forward's sum: slices in order, all loads issued first
      const float* zp = z_part + (int64_t)t * N + i;
      float part[kRouterMaxSplits];
#pragma unroll
      for (int s = 0; s < kRouterMaxSplits; ++s) part[s] = s < splits ? zp[s * TN] : 0.0f;
      v = 0.0f;
#pragma unroll
      for (int s = 0; s < kRouterMaxSplits; ++s)
        if (s < splits) v += part[s];
      if (b_router) v += b_router[i];
    }
    z[q] = v;
    dzl[q] = 0.0f;
    m = fmaxf(m, v);
  }
  m = wave_max(m);
  float se = 0.0f;
#pragma unroll
  for (int q = 0; q < kMaxPerLane; ++q) se += (lane + 64 * q < N) ? expf(z[q] - m) : 0.0f;
  se = wave_sum(se);
  const float lse = m + logf(se);
  auto P = [&](int q) { return expf(z[q] - m) / se; };   // softmax probability
  auto sig = [&](float x) { return 1.0f / (1.0f + expf(-x)); };

  // ---- task gradient through the selected gates
  const int64_t f0 = (int64_t)t * k;
  float inner = 0.0f, inner_p = 0.0f;
  for (int j = 0; j < k; ++j) {
    const float dgj = row_of[f0 + j] >= 0 ? dg_slot[f0 + j] : 0.0f;
    inner += gates[f0 + j] * dgj;
    if (dg_out && lane == 0) dg_out[f0 + j] = dgj;
  }
  // per-slot values are uniform across the wave: read them in the loop
  for (int j = 0; j < k; ++j) {
    const int e = ids[f0 + j];
    const float dgj = row_of[f0 + j] >= 0 ? dg_slot[f0 + j] : 0.0f;
    const float gj = gates[f0 + j];
    const int q = e >> 6;
    if (mode == 0) {
      if ((e & 63) == lane) {
#pragma unroll
        for (int qq = 0; qq < kMaxPerLane; ++qq)
          if (qq == q) dzl[qq] += gj * (dgj - inner);
      }
    } else if (mode == 1) {
      // a_i = dg at the selected experts; dz_i = P_i (a_i - sum_l P_l a_l)
      if ((e & 63) == lane) {
#pragma unroll
        for (int qq = 0; qq < kMaxPerLane; ++qq)
          if (qq == q) dzl[qq] += P(qq) * dgj;
      }
    }
  }
  if (mode == 1) {
    for (int j = 0; j < k; ++j) {
      const int e = ids[f0 + j];
      const float dgj = row_of[f0 + j] >= 0 ? dg_slot[f0 + j] : 0.0f;
      float pe = 0.0f;
      if ((e & 63) == lane) {
#pragma unroll
        for (int qq = 0; qq < kMaxPerLane; ++qq)
          if (qq == (e >> 6)) pe = P(qq);
      }
      inner_p += wave_sum(pe) * dgj;
    }
#pragma unroll
    for (int q = 0; q < kMaxPerLane; ++q)
      if (lane + 64 * q < N) dzl[q] -= P(q) * inner_p;
  }
  if (mode == 2) {
    // s_sel = sigmoid of the selected logits, S = their sum
    float S = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int e = ids[f0 + j];
      float ze = 0.0f;
      if ((e & 63) == lane) {
#pragma unroll
        for (int qq = 0; qq < kMaxPerLane; ++qq)
          if (qq == (e >> 6)) ze = z[qq];
      }
      S += sig(wave_sum(ze));
    }
    for (int j = 0; j < k; ++j) {
      const int e = ids[f0 + j];
      const float dgj = row_of[f0 + j] >= 0 ? dg_slot[f0 + j] : 0.0f;
      if ((e & 63) == lane) {
#pragma unroll
        for (int qq = 0; qq < kMaxPerLane; ++qq)
          if (qq == (e >> 6)) {
            const float s = sig(z[qq]);
            dzl[qq] += (dgj - inner) / S * s * (1.0f - s);
          }
      }
    }
  }

  // ---- L_aux: dL/dP_ti = d_laux alpha N f_i / T
  if (d_laux != 0.0f) {
    const float cst = d_laux * alpha * (float)N / ((float)T * (float)T * (float)k);
    float a[kMaxPerLane];
#pragma unroll
    for (int q = 0; q < kMaxPerLane; ++q) {
      const int i = lane + 64 * q;
      a[q] = i < N ? cst * (float)counts[i] : 0.0f;
    }
    if (mode == 2) {
      float S = 0.0f, pa = 0.0f;
#pragma unroll
      for (int q = 0; q < kMaxPerLane; ++q)
        if (lane + 64 * q < N) S += sig(z[q]);
      S = wave_sum(S);
#pragma unroll
      for (int q = 0; q < kMaxPerLane; ++q)
        if (lane + 64 * q < N) pa += sig(z[q]) / S * a[q];
      pa = wave_sum(pa);
#pragma unroll
      for (int q = 0; q < kMaxPerLane; ++q)
        if (lane + 64 * q < N) {
          const float s = sig(z[q]);
          dzl[q] += (a[q] - pa) / S * s * (1.0f - s);
        }
    } else {
      float pa = 0.0f;
#pragma unroll
      for (int q = 0; q < kMaxPerLane; ++q)
        if (lane + 64 * q < N) pa += P(q) * a[q];
      pa = wave_sum(pa);
#pragma unroll
      for (int q = 0; q < kMaxPerLane; ++q)
        if (lane + 64 * q < N) dzl[q] += P(q) * (a[q] - pa);
    }
  }
  // ---- z-loss
  if (d_zloss != 0.0f) {
    const float c = d_zloss * 2.0f / (float)T * lse;
#pragma unroll
    for (int q = 0; q < kMaxPerLane; ++q)
      if (lane + 64 * q < N) dzl[q] += c * P(q);
  }
#pragma unroll
  for (int q = 0; q < kMaxPerLane; ++q) {
    const int i = lane + 64 * q;
    if (i < N) dz[(int64_t)t * N + i] = dzl[q];
    if (i < ldzb) st(dzb, (int64_t)t * ldzb + i, i < N ? dzl[q] : 0.0f);
  }
}

// db[i] = sum_t dz[t][i] in a fixed order, in two passes: partial sums over
// chunks of kColChunk tokens (grid: columns / 64 x chunks; four waves each
// take a quarter of the chunk, added in order), then the chunk partials in
// chunk order.
constexpr int kColChunk = 128;
__global__ __launch_bounds__(kT) void colsum_part_kernel(const float* __restrict__ dz, int T, int N,
                                                         float* __restrict__ part) {
  __shared__ float s_part[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i = blockIdx.x * 64 + lane;
  const int t0 = blockIdx.y * kColChunk + w * (kColChunk / 4);
  const int t1 = min(t0 + kColChunk / 4, T);
  float s = 0.0f;
  if (i < N)
    for (int t = t0; t < t1; ++t) s += dz[(int64_t)t * N + i];
  s_part[w][lane] = s;
  __syncthreads();
  if (w == 0 && i < N)
    part[(int64_t)blockIdx.y * N + i] =
        ((s_part[0][lane] + s_part[1][lane]) + s_part[2][lane]) + s_part[3][lane];
}
__global__ __launch_bounds__(kT) void colsum_final_kernel(const float* __restrict__ part,
                                                          int chunks, int N,
                                                          float* __restrict__ db) {
  const int i = blockIdx.x * kT + threadIdx.x;
  if (i >= N) return;
  float s = 0.0f;
  for (int c = 0; c < chunks; ++c) s += part[(int64_t)c * N + i];
  db[i] = s;
}

// dh[t] = sum_j rows[row_of[t k + j]] (kept slots, slot order) + shared[t]
// + router[t], accumulated in fp32 in that order. The token's row indices
// are read once into LDS; VEC: each thread takes 16 bytes of columns (d and
// every pointer allow it; the launcher checks), else one column.
// With dz (N <= kMaxRouterFused experts) the router's term is formed here
// instead of read: sum over i < N, in order, of dz[t][i] · W_r[i][c] in fp32
// (no bf16 rounding of the term or of dz, and no separate GEMM).
constexpr int kMaxTopK = 16;
template <typename TE, bool VEC>
__global__ __launch_bounds__(kT) void dh_combine_kernel(
    const TE* __restrict__ rows, const int32_t* __restrict__ row_of,
    const TE* __restrict__ shared, const TE* __restrict__ router, const float* __restrict__ dz,
    const TE* __restrict__ wr, int N, TE* __restrict__ dh, int k, int d) {
  constexpr int V = VEC ? 16 / sizeof(TE) : 1;
  __shared__ int64_t s_r[kMaxTopK];
  __shared__ float s_dz[kMaxRouterFused];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < k) s_r[threadIdx.x] = row_of[t * k + threadIdx.x];
  if (dz && threadIdx.x < N) s_dz[threadIdx.x] = dz[t * N + threadIdx.x];
  __syncthreads();
  for (int c = threadIdx.x * V; c < d; c += kT * V) {
    float acc[V];
#pragma unroll
    for (int e = 0; e < V; ++e) acc[e] = 0.0f;
    auto add = [&](const TE* src) {
      if constexpr (VEC) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(src);
        const TE* x = reinterpret_cast<const TE*>(&raw);
#pragma unroll
        for (int e = 0; e < V; ++e) acc[e] += ld(x, e);
      } else {
        acc[0] += ld(src, 0);
      }
    };
    for (int j = 0; j < k; ++j) {
      const int64_t r = s_r[j];
      if (r >= 0) add(rows + r * d + c);
    }
    if (shared) add(shared + t * d + c);
    if (dz) {
      float rr[V];
#pragma unroll
      for (int e = 0; e < V; ++e) rr[e] = 0.0f;
      for (int i = 0; i < N; ++i) {
        const float z = s_dz[i];
        if constexpr (VEC) {
          const u32x4 raw = *reinterpret_cast<const u32x4*>(wr + (int64_t)i * d + c);
          const TE* x = reinterpret_cast<const TE*>(&raw);
#pragma unroll
          for (int e = 0; e < V; ++e) rr[e] = fmaf(z, ld(x, e), rr[e]);
        } else {
          rr[0] = fmaf(z, ld(wr, (int64_t)i * d + c), rr[0]);
        }
      }
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] += rr[e];
    } else {
      add(router + t * d + c);
    }
    if constexpr (VEC) {
      TE out[V];
#pragma unroll
      for (int e = 0; e < V; ++e) out[e] = from_f32<TE>(acc[e]);
      *reinterpret_cast<u32x4*>(dh + t * d + c) = *reinterpret_cast<const u32x4*>(out);
    } else {
      st(dh, t * d + c, acc[0]);
    }
  }
}

}  // namespace

hipError_t launch_kofs(const int32_t* offsets, int G, int n_single, int32_t* kofs,
                       hipStream_t st) {
  hipLaunchKernelGGL(kofs_kernel, dim3(1), dim3(kT), 0, st, offsets, G, n_single, kofs);
  return hipGetLastError();
}

hipError_t launch_pack_t(const void* src, int ld_src, int ncols, const int32_t* perm, int kdiv,
                         const float* scale, const int32_t* offsets, const int32_t* kofs, int G,
                         int n_single, int64_t p_limit, void* dst, int64_t ld_dst, int bf16,
                         hipStream_t st, int batch, int64_t src_bstride, int64_t dst_bstride) {
  if (p_limit == 0 || ncols == 0 || batch == 0) return hipSuccess;
  dim3 grid((unsigned)((p_limit + 63) / 64), (unsigned)((ncols + 63) / 64), (unsigned)batch);
  const int V = bf16 ? 8 : 4;
  const bool vec = ld_src % V == 0 && ld_dst % V == 0 && p_limit % V == 0 &&
                   src_bstride % V == 0 && dst_bstride % V == 0 &&
                   (reinterpret_cast<uintptr_t>(src) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(dst) & 15) == 0;
#define MOE_PACK(TE, VEC)                                                                      \
  hipLaunchKernelGGL((pack_t_kernel<TE, VEC>), grid, dim3(kT), 0, st,                          \
                     static_cast<const TE*>(src), ld_src, ncols, perm, kdiv, scale, offsets,   \
                     kofs, G, n_single, p_limit, static_cast<TE*>(dst), ld_dst, src_bstride,   \
                     dst_bstride)
  if (bf16) {
    if (vec) MOE_PACK(bf16_t, true); else MOE_PACK(bf16_t, false);
  } else {
    if (vec) MOE_PACK(float, true); else MOE_PACK(float, false);
  }
#undef MOE_PACK
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const float* gu, const float* v, void* act, void* dgu,
                             const int32_t* perm, const float* gates, float* dg_slot,
                             const int32_t* offsets, int G, int rows_bound, int d_ff, int bf16,
                             hipStream_t st) {
  if (rows_bound == 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(swiglu_bwd_kernel<bf16_t>, dim3(rows_bound), dim3(kT), 0, st, gu, v,
                       static_cast<bf16_t*>(act), static_cast<bf16_t*>(dgu), perm, gates, dg_slot,
                       offsets, G, d_ff);
  else
    hipLaunchKernelGGL(swiglu_bwd_kernel<float>, dim3(rows_bound), dim3(kT), 0, st, gu, v,
                       static_cast<float*>(act), static_cast<float*>(dgu), perm, gates, dg_slot,
                       offsets, G, d_ff);
  return hipGetLastError();
}

int swiglu_bwd_t_tiles(int d_ff) { return (d_ff + kTC - 1) / kTC; }

hipError_t launch_swiglu_bwd_t(const float* gu, const float* v, void* dgu, void* act_t,
                               void* dgu_t, int64_t ld_t, const int32_t* perm,
                               const float* gates, const int32_t* offsets, const int32_t* kofs,
                               int G, int64_t p_limit, int rows_bound, int d_ff,
                               float* dg_part, float* dg_slot, int bf16, hipStream_t st) {
  if (p_limit == 0 || d_ff == 0) return hipSuccess;
  if (p_limit % 64 != 0 || ld_t % 8 != 0 || (reinterpret_cast<uintptr_t>(act_t) & 15) ||
      (reinterpret_cast<uintptr_t>(dgu_t) & 15))
    return hipErrorInvalidValue;
  const int nct = swiglu_bwd_t_tiles(d_ff);
  dim3 grid((unsigned)(p_limit / 64), (unsigned)nct);
  const bool vec4 = bf16 && d_ff % 4 == 0 &&
                    ((reinterpret_cast<uintptr_t>(gu) | reinterpret_cast<uintptr_t>(v)) & 15) == 0 &&
                    (reinterpret_cast<uintptr_t>(dgu) & 7) == 0;
  if (vec4)
    hipLaunchKernelGGL(swiglu_bwd_t4_kernel, grid, dim3(kT), 0, st, gu, v,
                       static_cast<bf16_t*>(dgu), static_cast<bf16_t*>(act_t),
                       static_cast<bf16_t*>(dgu_t), ld_t, perm, gates, offsets, kofs, G, p_limit,
                       d_ff, dg_part, (int64_t)rows_bound);
  else if (bf16)
    hipLaunchKernelGGL(swiglu_bwd_t_kernel<bf16_t>, grid, dim3(kT), 0, st, gu, v,
                       static_cast<bf16_t*>(dgu), static_cast<bf16_t*>(act_t),
                       static_cast<bf16_t*>(dgu_t), ld_t, perm, gates, offsets, kofs, G, p_limit,
                       d_ff, dg_part, (int64_t)rows_bound);
  else
    hipLaunchKernelGGL(swiglu_bwd_t_kernel<float>, grid, dim3(kT), 0, st, gu, v,
                       static_cast<float*>(dgu), static_cast<float*>(act_t),
                       static_cast<float*>(dgu_t), ld_t, perm, gates, offsets, kofs, G, p_limit,
                       d_ff, dg_part, (int64_t)rows_bound);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || rows_bound == 0) return e;
  hipLaunchKernelGGL(dg_reduce_kernel, dim3((unsigned)((rows_bound + kT - 1) / kT)), dim3(kT), 0,
                     st, dg_part, nct, (int64_t)rows_bound, perm, offsets, G, dg_slot);
  return hipGetLastError();
}

hipError_t launch_route_bwd(const float* z_part, int splits, const float* b_router,
                            const int32_t* ids, const float* gates, const float* dg_slot,
                            const int32_t* row_of, const int32_t* counts, int T, int N, int k,
                            int mode, float alpha, float d_laux, float d_zloss, float* dz,
                            void* dzb, int ldzb, int bf16, float* dg_out, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (splits < 1 || splits > kRouterMaxSplits) return hipErrorInvalidValue;
  if (bf16)
    hipLaunchKernelGGL(route_bwd_kernel<bf16_t>, dim3(T), dim3(64), 0, st, z_part, splits,
                       b_router, ids, gates, dg_slot, row_of, counts, T, N, k, mode, alpha,
                       d_laux, d_zloss, dz, static_cast<bf16_t*>(dzb), ldzb, dg_out);
  else
    hipLaunchKernelGGL(route_bwd_kernel<float>, dim3(T), dim3(64), 0, st, z_part, splits,
                       b_router, ids, gates, dg_slot, row_of, counts, T, N, k, mode, alpha,
                       d_laux, d_zloss, dz, static_cast<float*>(dzb), ldzb, dg_out);
  return hipGetLastError();
}

int colsum_chunks(int T) { return (T + kColChunk - 1) / kColChunk; }

hipError_t launch_colsum(const float* dz, int T, int N, float* part, float* db, hipStream_t st) {
  const int chunks = colsum_chunks(T);
  if (chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(colsum_part_kernel, dim3((N + 63) / 64, chunks), dim3(kT), 0, st, dz, T, N,
                     part);
  hipLaunchKernelGGL(colsum_final_kernel, dim3((N + kT - 1) / kT), dim3(kT), 0, st, part, chunks,
                     N, db);
  return hipGetLastError();
}

hipError_t launch_dh_combine(const void* rows, const int32_t* row_of, const void* shared,
                             const void* router, const float* dz, const void* w_router, int N,
                             void* dh, int T, int k, int d, int bf16, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (k > kMaxTopK) return hipErrorInvalidValue;
  if ((dz != nullptr) == (router != nullptr) || (dz && (N > kMaxRouterFused || !w_router)))
    return hipErrorInvalidValue;                 // exactly one form of the router's term
  const int V = bf16 ? 8 : 4;
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  const bool vec = d % V == 0 && al(rows) && al(dh) && (!shared || al(shared)) &&
                   (router ? al(router) : al(w_router));
#define MOE_DHC(TE, VEC)                                                                       \
  hipLaunchKernelGGL((dh_combine_kernel<TE, VEC>), dim3(T), dim3(kT), 0, st,                   \
                     static_cast<const TE*>(rows), row_of, static_cast<const TE*>(shared),     \
                     static_cast<const TE*>(router), dz, static_cast<const TE*>(w_router), N,  \
                     static_cast<TE*>(dh), k, d)
  if (bf16) {
    if (vec) MOE_DHC(bf16_t, true); else MOE_DHC(bf16_t, false);
  } else {
    if (vec) MOE_DHC(float, true); else MOE_DHC(float, false);
  }
#undef MOE_DHC
  return hipGetLastError();
}

}  // namespace moe
