// Grouped expert GEMMs on bf16 MFMA (gfx950), fp32 accumulation.
//
// The experts of a sparse MoE layer are SwiGLU FFNs [page "MOE 专家选择与路由机制"
// (wuhy-notes), §一 expert formula]; after dispatch each expert owns a
// contiguous run of rows and the experts run together as one grouped GEMM
// [wuhy-notes §十二 "小矩阵问题"; page "【大模型】MoE（专家混合模型）简介"
// (horizon.auto), §8 Kernel row], over ragged, unpadded row counts
// [wuhy-notes §六 Dropless MoE].
//
// Two shapes of kernel:
//  * prefill: a persistent, XCD-aware tile loop over (expert m-tile, n-tile)
//    pairs; each 256-thread block stages A (gathered token rows) and B
//    (weight rows, K contiguous) in LDS, double buffered, and four waves
//    run v_mfma_f32_32x32x16_bf16. The gate/up kernel holds the gate and up
//    accumulators of the same output tile and applies SiLU(g)·u in the
//    epilogue.
//  * decode (≤ 64 rows per expert): weight-streaming split-K kernels, B read
//    straight from HBM into registers (no LDS), v_mfma_f32_16x16x32_bf16,
//    four waves reduce through LDS in a fixed order.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxGroups = 512;
constexpr int kXcds = 8;   // MI355X: 8 XCDs; block b runs on XCD b % 8

// ---------------------------------------------------------------- tiling
template <int BM_, int BN_, bool DUAL_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = 64;
  static constexpr bool DUAL = DUAL_;
  static constexpr int NB = DUAL ? 2 : 1;           // gate and up, or one B
  static constexpr int WM = 2, WN = 2;              // 2x2 waves
  static constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  static constexpr int FM = TM / 32, FN = TN / 32;  // 32x32 MFMA tiles per wave
  static constexpr int BROWS = BN * NB;             // B rows staged per K step
  static constexpr int ROWB = BK * 2 + 16;          // LDS row pitch (bytes), +16 pad
  static constexpr int A_BYTES = BM * ROWB;
  static constexpr int B_BYTES = BROWS * ROWB;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int ACH = BM / 32;               // 16B chunks per thread (A)
  static constexpr int BCH = BROWS / 32;            // 16B chunks per thread (B)
  static constexpr int BCH0 = BN / 32;              // chunks that come from B0
  static_assert(FM >= 1 && FN >= 1, "tile too small");
};

enum Epi { EPI_SWIGLU = 0, EPI_STORE_BF16 = 1 };

// Global -> registers for one BK slab. Thread tid loads 16-byte chunk
// (tid & 7) of rows (tid >> 3) + 32 i: eight lanes cover one 128-byte row
// segment, so every load instruction is fully coalesced. Raw buffer loads:
// a 32-bit per-lane byte offset, the K position as a scalar offset, and the
// buffer's extent in the descriptor (reads past it return zero).
template <class C>
__device__ __forceinline__ void load_slab(u32x4 (&ra)[C::ACH], u32x4 (&rb)[C::BCH],
                                          const Rsrc& A, const uint32_t (&aoff)[C::ACH],
                                          const Rsrc& B0, const Rsrc& B1,
                                          const uint32_t (&boff)[C::BCH], int kbytes) {
#pragma unroll
  for (int i = 0; i < C::ACH; ++i) ra[i] = buffer_load16(A, aoff[i], kbytes);
#pragma unroll
  for (int i = 0; i < C::BCH; ++i) rb[i] = buffer_load16((i < C::BCH0) ? B0 : B1, boff[i], kbytes);
}

template <class C>
__device__ __forceinline__ void store_slab(char* __restrict__ stage,
                                           const u32x4 (&ra)[C::ACH],
                                           const u32x4 (&rb)[C::BCH]) {
  const int tid = threadIdx.x;
  char* a = stage + (tid >> 3) * C::ROWB + (tid & 7) * 16;
  char* b = a + C::A_BYTES;
#pragma unroll
  for (int i = 0; i < C::ACH; ++i)
    *reinterpret_cast<u32x4*>(a + i * 32 * C::ROWB) = ra[i];
#pragma unroll
  for (int i = 0; i < C::BCH; ++i)
    *reinterpret_cast<u32x4*>(b + i * 32 * C::ROWB) = rb[i];
}

template <class C>
__device__ __forceinline__ void mma_slab(const char* __restrict__ stage,
                                         f32x16 (&acc)[C::NB][C::FM][C::FN]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int lr = lane & 31, lh = lane >> 5;
  const char* a = stage + (wm * C::TM + lr) * C::ROWB + lh * 16;
  const char* b = stage + C::A_BYTES + (wn * C::TN + lr) * C::ROWB + lh * 16;
#pragma unroll
  for (int ks = 0; ks < C::BK / 16; ++ks) {
    u32x4 af[C::FM];
    u32x4 bfr[C::NB][C::FN];
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
      af[fm] = *reinterpret_cast<const u32x4*>(a + fm * 32 * C::ROWB + ks * 32);
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
        bfr[nb][fn] = *reinterpret_cast<const u32x4*>(
            b + (nb * C::BN + fn * 32) * C::ROWB + ks * 32);
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
          acc[nb][fm][fn] = mfma_32x32x16(af[fm], bfr[nb][fn], acc[nb][fm][fn]);
  }
}

// acc += A[rows] · B[cols]^T over k in [k_begin, k_begin + k_len), k_len a
// multiple of 64. Two register stages of global loads are in flight: the
// slab for step kt+2 is issued when step kt starts and reaches LDS at the
// end of step kt+1, so a load has two steps of MFMA work to arrive. LDS is
// double buffered; one __syncthreads per step.
template <class C>
__device__ __forceinline__ void mainloop(char* __restrict__ lds, const Rsrc& A,
                                         const uint32_t (&aoff)[C::ACH], const Rsrc& B0,
                                         const Rsrc& B1, const uint32_t (&boff)[C::BCH],
                                         int k_begin, int k_len,
                                         f32x16 (&acc)[C::NB][C::FM][C::FN]) {
  constexpr int STEP = C::BK * 2;  // bytes per slab along K
  const int KT = k_len / C::BK;
  const int kb = k_begin * 2;
  char* L0 = lds;
  char* L1 = lds + C::STAGE;
  u32x4 ra0[C::ACH], rb0[C::BCH], ra1[C::ACH], rb1[C::BCH];
  load_slab<C>(ra0, rb0, A, aoff, B0, B1, boff, kb);
  if (KT > 1) load_slab<C>(ra1, rb1, A, aoff, B0, B1, boff, kb + STEP);
  store_slab<C>(L0, ra0, rb0);
  __syncthreads();
  int kt = 0;
  for (; kt + 1 < KT; kt += 2) {
    // even step: L0 holds slab kt, registers 1 hold slab kt+1
    if (kt + 2 < KT) load_slab<C>(ra0, rb0, A, aoff, B0, B1, boff, kb + (kt + 2) * STEP);
    mma_slab<C>(L0, acc);
    store_slab<C>(L1, ra1, rb1);
    __syncthreads();
    // odd step: L1 holds slab kt+1, registers 0 hold slab kt+2
    if (kt + 3 < KT) load_slab<C>(ra1, rb1, A, aoff, B0, B1, boff, kb + (kt + 3) * STEP);
    mma_slab<C>(L1, acc);
    if (kt + 2 < KT) store_slab<C>(L0, ra0, rb0);
    __syncthreads();
  }
  if (kt < KT) {   // odd number of steps: the last slab is in L0
    mma_slab<C>(L0, acc);
    __syncthreads();
  }
}

// Write the tile's outputs through LDS so that global stores are 16-byte,
// row-contiguous. Each lane holds one column of 16 rows per 32x32 block;
// neighbouring lanes swap values so every LDS write carries two adjacent
// columns. EPI_SWIGLU stores SiLU(gate)·up, EPI_STORE_BF16 stores acc.
template <class C, int EPI>
__device__ __forceinline__ void epilogue_bf16(char* __restrict__ lds,
                                              const f32x16 (&acc)[C::NB][C::FM][C::FN],
                                              bf16_t* __restrict__ Cout, int64_t ldc,
                                              int64_t row0_out, int rows_valid, int n0,
                                              int Ncols) {
  constexpr int PITCH = C::BN * 2 + 16;   // bytes per LDS output row
  static_assert(C::BM * PITCH <= C::LDS, "output tile does not fit in LDS");
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int lr = lane & 31, lh = lane >> 5;
  const bool odd = lane & 1;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const int col = wn * C::TN + fn * 32 + lr;
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        float v0, v1;
        if (EPI == EPI_SWIGLU) {
          v0 = silu_fast(acc[0][fm][fn][i]) * acc[C::NB - 1][fm][fn][i];
          v1 = silu_fast(acc[0][fm][fn][i + 1]) * acc[C::NB - 1][fm][fn][i + 1];
        } else {
          v0 = acc[0][fm][fn][i];
          v1 = acc[0][fm][fn][i + 1];
        }
        // even lane keeps row i (cols lr, lr+1); odd lane keeps row i+1 (cols lr-1, lr)
        const float send = odd ? v0 : v1;
        const float recv = __shfl_xor(send, 1, 64);
        const int ii = odd ? i + 1 : i;
        const int r = wm * C::TM + fm * 32 + 8 * (ii >> 2) + 4 * lh + (ii & 3);
        const uint32_t packed = odd ? pack_bf16x2(recv, v1) : pack_bf16x2(v0, recv);
        *reinterpret_cast<uint32_t*>(lds + r * PITCH + (col & ~1) * 2) = packed;
      }
    }
  __syncthreads();
  constexpr int CPR = C::BN / 8;            // 16-byte chunks per row
  for (int c = tid; c < C::BM * CPR; c += kThreads) {
    const int r = c / CPR, ch = c % CPR;
    const int col = n0 + ch * 8;
    if (r < rows_valid && col < Ncols) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(lds + r * PITCH + ch * 16);
      *reinterpret_cast<u32x4*>(Cout + (row0_out + r) * ldc + col) = v;
    }
  }
  __syncthreads();
}

template <class C>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[C::NB][C::FM][C::FN]) {
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[nb][fm][fn][i] = 0.0f;
}

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// Persistent grouped GEMM. Every block first builds the exclusive prefix of
// m-tiles per group in LDS, then walks its share of the tile list:
//  * XCD-aware split: block b runs on XCD b % 8, and XCD x takes the
//    contiguous tile range [x·n/8, (x+1)·n/8), so the ~32 tiles in flight
//    on one XCD share A rows and B columns in that XCD's L2;
//  * tile order: groups of 8 n-tiles, m-tiles (all experts) inside, so 4
//    m-tiles × 8 n-tiles run together.
template <class C, int EPI>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(GroupedProblem p) {
  __shared__ __attribute__((aligned(16))) char lds[C::LDS];
  __shared__ int s_pref[kMaxGroups + 1];
  const int tid = threadIdx.x;
  const int G = p.offsets ? p.groups : 1;

  if (tid < 64) {
    int loc[kMaxGroups / 64];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kMaxGroups / 64; ++i) {
      const int g = tid * (kMaxGroups / 64) + i;
      int c = 0;
      if (g < G) {
        const int rows = p.offsets ? (p.offsets[g + 1] - p.offsets[g]) : p.M;
        c = (rows + C::BM - 1) / C::BM;
      }
      loc[i] = c;
      sum += c;
    }
    const int incl = wave_incl_scan(sum);
    int run = incl - sum;
#pragma unroll
    for (int i = 0; i < kMaxGroups / 64; ++i) {
      const int g = tid * (kMaxGroups / 64) + i;
      if (g < G) s_pref[g] = run;
      run += loc[i];
    }
    if (tid == 63) s_pref[G] = incl;
  }
  __syncthreads();

  const int total_mt = s_pref[G];
  const int nt_n = (p.Ncols + C::BN - 1) / C::BN;
  const int64_t total = (int64_t)total_mt * nt_n;
  if (total == 0) return;

  const int nblk = gridDim.x, b = blockIdx.x;
  int64_t t_begin, t_end, t_step;
  if (nblk >= kXcds && nblk % kXcds == 0) {
    const int xcd = b % kXcds;
    t_begin = total * xcd / kXcds + b / kXcds;
    t_end = total * (xcd + 1) / kXcds;
    t_step = nblk / kXcds;
  } else {
    t_begin = b;
    t_end = total;
    t_step = nblk;
  }

  const Rsrc rA = make_rsrc(p.A, p.a_bytes);
  const int row0 = tid >> 3, c16 = tid & 7;
  constexpr int GN = 8;

  for (int64_t t = t_begin; t < t_end; t += t_step) {
    // ---- tile -> (m-tile, n-tile)
    const int64_t sg = (int64_t)total_mt * GN;
    const int nsup = (int)(t / sg);
    const int within = (int)(t - (int64_t)nsup * sg);
    const int width = min(GN, nt_n - nsup * GN);
    const int mt = within / width;
    const int nt = nsup * GN + within % width;
    // ---- m-tile -> group (binary search in the prefix)
    int lo = 0, hi = G;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pref[mid] <= mt) lo = mid; else hi = mid;
    }
    const int g = lo;
    const int gbase = p.offsets ? p.offsets[g] : 0;
    const int gend = p.offsets ? p.offsets[g + 1] : p.M;
    const int m0 = gbase + (mt - s_pref[g]) * C::BM;
    const int m_end = min(m0 + C::BM, gend);
    const int n0 = nt * C::BN;

    uint32_t aoff[C::ACH];
#pragma unroll
    for (int i = 0; i < C::ACH; ++i) {
      const int r = min(m0 + row0 + 32 * i, m_end - 1);
      const int src = p.perm ? p.perm[r] / p.kdiv : r;
      aoff[i] = (uint32_t)(src * p.lda + c16 * 8) * 2u;
    }
    uint32_t boff[C::BCH];
#pragma unroll
    for (int i = 0; i < C::BCH; ++i) {
      const int rr = (row0 + 32 * i) % C::BN;
      const int col = min(n0 + rr, p.Ncols - 1);
      boff[i] = (uint32_t)(col * p.ldb + c16 * 8) * 2u;
    }
    const uint32_t bbytes = (uint32_t)((int64_t)p.Ncols * p.ldb * 2);
    const Rsrc rB0 = make_rsrc(static_cast<const bf16_t*>(p.B0) + (int64_t)g * p.b_gstride, bbytes);
    const Rsrc rB1 = C::DUAL ? make_rsrc(static_cast<const bf16_t*>(p.B1) + (int64_t)g * p.b_gstride, bbytes) : rB0;

    f32x16 acc[C::NB][C::FM][C::FN];
    zero_acc<C>(acc);
    mainloop<C>(lds, rA, aoff, rB0, rB1, boff, 0, p.K, acc);

    epilogue_bf16<C, EPI>(lds, acc, static_cast<bf16_t*>(p.C), p.ldc, p.c_row0 + m0,
                          m_end - m0, n0, p.Ncols);
  }
}

// Router logits as a split-K GEMM: z_part[s][T][N] = h[:, Ks] · W_r[:, Ks]^T.
// The selection kernel sums the partial slices in a fixed order.
template <class C>
__global__ __launch_bounds__(kThreads, 1) void router_gemm_kernel(
    const bf16_t* __restrict__ h, const bf16_t* __restrict__ w, float* __restrict__ z_part,
    int T, int d, int N, int splits) {
  __shared__ __attribute__((aligned(16))) char lds[C::LDS];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.x * C::BM, n0 = blockIdx.y * C::BN, s = blockIdx.z;
  // split s covers K steps [kt*s/splits, kt*(s+1)/splits): never empty when
  // kt >= splits, so every partial slice is written
  const int kt = d / C::BK;
  const int k_begin = (kt * s / splits) * C::BK;
  const int k_len = (kt * (s + 1) / splits) * C::BK - k_begin;
  const int row0 = tid >> 3, c16 = tid & 7;
  uint32_t aoff[C::ACH];
#pragma unroll
  for (int i = 0; i < C::ACH; ++i) aoff[i] = (uint32_t)(min(m0 + row0 + 32 * i, T - 1) * d + c16 * 8) * 2u;
  uint32_t boff[C::BCH];
#pragma unroll
  for (int i = 0; i < C::BCH; ++i) boff[i] = (uint32_t)(min(n0 + row0 + 32 * i, N - 1) * d + c16 * 8) * 2u;
  f32x16 acc[C::NB][C::FM][C::FN];
  zero_acc<C>(acc);
  const Rsrc rh = make_rsrc(h, (uint32_t)((int64_t)T * d * 2));
  const Rsrc rw = make_rsrc(w, (uint32_t)((int64_t)N * d * 2));
  mainloop<C>(lds, rh, aoff, rw, rw, boff, k_begin, k_len, acc);
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int lr = lane & 31, lh = lane >> 5;
  float* out = z_part + (int64_t)s * T * N;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const int col = n0 + wn * C::TN + fn * 32 + lr;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = m0 + wm * C::TM + fm * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
        if (r < T && col < N) out[(int64_t)r * N + col] = acc[0][fm][fn][i];
      }
    }
}

// ------------------------------------------------------- decode (skinny)
// Block (group g, column block): rows of group g (at most 16·MT), 16·CT
// output columns (of gate and up when DUAL), the four waves split K into
// 64-wide chunks (chunk c goes to wave c % 4). Lane (i = l % 16, q = l / 16)
// loads 32 contiguous bytes of weight row i at k = 64c + 16q, so each group
// of four lanes reads one full 128-byte line; the A fragments use the same
// k mapping.
template <int MT, int CT, bool DUAL>
__global__ __launch_bounds__(kThreads) void skinny_gemm_kernel(GroupedProblem p) {
  constexpr int NB = DUAL ? 2 : 1;
  constexpr int NACC = NB * MT * CT;
  __shared__ f32x4 red[4][NACC][64];
  const int g = blockIdx.x;
  int r0, cnt;
  if (p.offsets) {
    r0 = p.offsets[g];
    cnt = p.offsets[g + 1] - r0;
  } else {
    r0 = g * 16 * MT;
    cnt = min(p.M - r0, 16 * MT);
  }
  if (cnt <= 0) return;
  cnt = min(cnt, 16 * MT);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, lq = lane >> 4;
  const int n0 = blockIdx.y * 16 * CT;

  const bf16_t* __restrict__ A = static_cast<const bf16_t*>(p.A);
  const bf16_t* arow[MT];
  bool aval[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + li;
    aval[mt] = m < cnt;
    const int r = r0 + min(m, cnt - 1);
    const int src = p.perm ? p.perm[r] / p.kdiv : r;
    arow[mt] = A + (int64_t)src * p.lda + lq * 16;
  }
  const bf16_t* brow[NB][CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int col = min(n0 + ct * 16 + li, p.Ncols - 1);
    brow[0][ct] = static_cast<const bf16_t*>(p.B0) + (int64_t)g * p.b_gstride +
                  (int64_t)col * p.ldb + lq * 16;
    if (DUAL)
      brow[NB - 1][ct] = static_cast<const bf16_t*>(p.B1) + (int64_t)g * p.b_gstride +
                         (int64_t)col * p.ldb + lq * 16;
  }

  f32x4 acc[NB][MT][CT];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) acc[nb][mt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KT = p.K / 64;
  u32x4 bc[NB][CT][2], bn[NB][CT][2];
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  auto loadB = [&](u32x4 (&dst)[NB][CT][2], int c) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int s = 0; s < 2; ++s)
          dst[nb][ct][s] = *reinterpret_cast<const u32x4*>(brow[nb][ct] + c * 64 + s * 8);
  };
  int c = w;
  if (c < KT) loadB(bc, c);
  for (; c < KT; c += 4) {
    if (c + 4 < KT) loadB(bn, c + 4);
    u32x4 af[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int s = 0; s < 2; ++s)
        af[mt][s] = aval[mt] ? *reinterpret_cast<const u32x4*>(arow[mt] + c * 64 + s * 8) : zero4;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
            acc[nb][mt][ct] = mfma_16x16x32(af[mt][s], bc[nb][ct][s], acc[nb][mt][ct]);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int s = 0; s < 2; ++s) bc[nb][ct][s] = bn[nb][ct][s];
  }

#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        red[w][(nb * MT + mt) * CT + ct][lane] = acc[nb][mt][ct];
  __syncthreads();

  bf16_t* __restrict__ Cout = static_cast<bf16_t*>(p.C);
  for (int q = w; q < MT * CT; q += 4) {
    const int mt = q / CT, ct = q % CT;
    const f32x4 a0 = red[0][q][lane] + red[1][q][lane] + red[2][q][lane] + red[3][q][lane];
    f32x4 a1 = a0;
    if (DUAL) {
      const int q1 = (MT + mt) * CT + ct;
      a1 = red[0][q1][lane] + red[1][q1][lane] + red[2][q1][lane] + red[3][q1][lane];
    }
    const int col = n0 + ct * 16 + li;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mt * 16 + lq * 4 + i;
      if (m < cnt && col < p.Ncols) {
        const float v = DUAL ? silu_fast(a0[i]) * a1[i] : a0[i];
        Cout[(p.c_row0 + r0 + m) * (int64_t)p.ldc + col] = (bf16_t)f32_to_bf16(v);
      }
    }
  }
}

template <int MT, bool DUAL>
hipError_t launch_skinny(const GroupedProblem& p, hipStream_t st) {
  constexpr int CT = (MT == 1) ? 4 : (MT == 2 ? 2 : 1);
  const int G = p.offsets ? p.groups : (p.M + 16 * MT - 1) / (16 * MT);
  dim3 grid(G, (p.Ncols + 16 * CT - 1) / (16 * CT));
  if (G == 0) return hipSuccess;
  hipLaunchKernelGGL((skinny_gemm_kernel<MT, CT, DUAL>), grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

template <bool DUAL>
hipError_t launch_skinny_any(const GroupedProblem& p, hipStream_t st) {
  if (p.max_rows <= 16) return launch_skinny<1, DUAL>(p, st);
  if (p.max_rows <= 32) return launch_skinny<2, DUAL>(p, st);
  return launch_skinny<4, DUAL>(p, st);
}

template <class C, int EPI>
hipError_t launch_grouped(const GroupedProblem& p, int num_cu, hipStream_t st) {
  // Upper bound on tiles, to avoid idle blocks on tiny problems.
  const int G = p.offsets ? p.groups : 1;
  const int64_t mt_bound = (int64_t)(p.M + C::BM - 1) / C::BM + (p.offsets ? G : 0);
  const int64_t tiles = mt_bound * ((p.Ncols + C::BN - 1) / C::BN);
  int nblk = num_cu;
  if (tiles < nblk) nblk = (int)tiles;
  if (nblk >= kXcds) nblk -= nblk % kXcds;
  if (nblk <= 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_gemm_kernel<C, EPI>), dim3(nblk), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace

// Rows per expert at most 64: weight streaming. Otherwise tiles of 256 rows
// when experts average at least 1024 rows, else 128.
hipError_t launch_gateup_bf16(const GroupedProblem& p, int num_cu, hipStream_t st) {
  if (p.max_rows <= 64) return launch_skinny_any<true>(p, st);
  const int G = p.offsets ? p.groups : 1;
  if (p.M >= 1024 * G) return launch_grouped<TileCfg<256, 128, true>, EPI_SWIGLU>(p, num_cu, st);
  return launch_grouped<TileCfg<128, 128, true>, EPI_SWIGLU>(p, num_cu, st);
}

hipError_t launch_down_bf16(const GroupedProblem& p, int num_cu, hipStream_t st) {
  if (p.max_rows <= 64) return launch_skinny_any<false>(p, st);
  const int G = p.offsets ? p.groups : 1;
  if (p.M >= 1024 * G) return launch_grouped<TileCfg<256, 256, false>, EPI_STORE_BF16>(p, num_cu, st);
  return launch_grouped<TileCfg<128, 256, false>, EPI_STORE_BF16>(p, num_cu, st);
}

// Split-K factor of the router GEMM: enough blocks to fill about 256 CUs,
// at least four K steps per split, at most kRouterMaxSplits. It depends on
// the shape only, so results do not depend on the device.
int router_splits(int T, int d, int N) {
  using C = TileCfg<128, 128, false>;
  const int64_t tiles = (int64_t)((T + C::BM - 1) / C::BM) * ((N + C::BN - 1) / C::BN);
  int s = 1;
  while (s < kRouterMaxSplits && tiles * s * 2 <= 256 && (d / 64) >= s * 2 * 4) s *= 2;
  return s;
}

hipError_t launch_router_gemm_bf16(const void* h, const void* w, float* z_part, int T, int d,
                                   int N, int splits, hipStream_t st) {
  using C = TileCfg<128, 128, false>;
  dim3 grid((T + C::BM - 1) / C::BM, (N + C::BN - 1) / C::BN, splits);
  hipLaunchKernelGGL((router_gemm_kernel<C>), grid, dim3(kThreads), 0, st,
                     static_cast<const bf16_t*>(h), static_cast<const bf16_t*>(w), z_part, T, d,
                     N, splits);
  return hipGetLastError();
}

}  // namespace moe
