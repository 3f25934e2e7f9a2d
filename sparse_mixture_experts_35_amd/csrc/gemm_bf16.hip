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
//    four waves reduce through LDS in a fixed order; the down GEMM can run
//    the combine in its last blocks.
// The backward pass adds down-type tiles whose B is given as [K rows][N
// columns] (the weights as stored; LDS transpose reads for its fragments)
// and the weight-gradient GEMMs over per-expert K ranges.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxGroups = 512;
constexpr int kXcds = 8;   // MI355X: 8 XCDs; block b runs on XCD b % 8

// ---------------------------------------------------------------- tiling
// Block tile BM rows x BN output columns (gate and up columns both when
// DUAL), four waves in a 2x2 grid, each wave TM x TN with 32x32x16 MFMAs.
// K advances in slabs of BK = 32. A slab of the block tile lives in LDS as
// BM + BROWS rows of 64 bytes (A rows, then B rows), 16-byte chunks XOR-
// swizzled per row. STAGES such stages form a ring; OCC blocks share a CU
// (two blocks: two waves per SIMD, each hides the other's waits).
// (64-deep slabs, whose loads cover whole cache lines, were measured too:
// they halve the L1-to-L2 requests but did not make the kernel faster.)
// NN: B is given as [K rows][N columns] (N contiguous, the weights' own
// layout in the backward pass) and staged as BK rows of BN columns; its
// MFMA fragments are read with the LDS transpose read (one B, no DUAL).
// BK_ = 64: 64-deep K slabs, so that each staged row is one whole 128-byte
// line (a 32-deep slab loads half a line per row and slab). Rows of 128 B
// stream into LDS about 1.5x faster than rows of 64 B (HBM: 6.3 against
// 4.3 TB/s with 512 rows a slab); the 64 KB stages leave room for two.
template <int BM_, int BN_, bool DUAL_, int STAGES_, int OCC_, bool NN_ = false, int BK_ = 32>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr bool DUAL = DUAL_;
  static constexpr int STAGES = STAGES_;             // LDS ring depth (3 or 4)
  static constexpr int OCC = OCC_;                   // blocks per CU (1 or 2)
  static constexpr int NB = DUAL ? 2 : 1;           // gate and up, or one B
  static constexpr int WM = 2, WN = 2;              // 2x2 waves
  static constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  static constexpr int FM = TM / 32, FN = TN / 32;  // 32x32 MFMA tiles per wave
  static constexpr int BROWS = BN * NB;             // B rows staged per slab
  static constexpr int ROWB = BK * 2;               // 64 bytes per staged row
  static constexpr int CH = ROWB / 16;              // 16-byte chunks per row
  static constexpr int RPI = 64 / CH;               // rows per 1 KiB load instruction
  static constexpr int A_BYTES = BM * ROWB;
  static constexpr int STAGE = (BM + BROWS) * ROWB;
  static constexpr int NAW = BM / (4 * RPI);        // A load blocks per wave
  static constexpr int NBW = BROWS / (4 * RPI);     // B load blocks per wave
  static constexpr int NLW = NAW + NBW;             // direct-to-LDS loads per wave per slab
  static_assert(FM >= 1 && FN >= 1, "tile too small");
  static_assert(BM % (4 * RPI) == 0 && BROWS % (4 * RPI) == 0, "tile rows vs load blocks");
  static_assert((BK == 32 && (STAGES == 3 || STAGES == 4)) ||
                (BK == 64 && (STAGES == 2 || STAGES == 3)), "pipeline shape");
  static constexpr bool NN = NN_;
  // three-stage 64-deep tiles: each wave loads the A rows of its own row
  // range and skips row blocks past the tile's last row (the two-stage
  // 256-row tiles keep interleaved rows: with per-wave rows the Mixtral-
  // shaped gate/up GEMM missed L2 for 7.49 instead of 6.72 GB, 1-2% slower)
  static constexpr bool WAVE_ROWS = BK == 64 && STAGES == 3;
  static constexpr int BROWB = BN * 2;              // NN: bytes of one staged B row (one k)
  static_assert(!NN || (!DUAL && BK * BROWB == BROWS * ROWB && BROWB % 256 == 0),
                "NN: one B, the same stage size, whole 16-chunk groups per row");
};

// NN: chunk swizzle of staged B row r. A transpose read takes, in each group
// of 16 lanes, 8 bytes from each of four consecutive rows at the same two
// logical chunks; XOR-ing the chunk index with 4 (r & 3) puts the four
// rows' chunk pairs on distinct banks.
__device__ __forceinline__ int nn_swz(int r) { return 4 * (r & 3); }

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16* lds_v4i16_t;

// Chunk swizzle of staged row r: logical 16-byte chunk c lives at c ^ swz(r).
// ds_read_b128 serves 16 consecutive lanes per pass from 64 four-byte banks.
// A fragment read has lane = row and one logical chunk, so a lane's bank
// quad is (r & 3, chunk), and (r & 3, (r >> 2) & 3) is distinct over any 16
// consecutive rows. Measured conflict-free with the LDS bank-conflict
// counter on gfx950 (where ((r >> 1) + (r >> 3)) & 3, for instance, still
// costs 4 stall cycles per read).
// With 128-byte rows (BK = 64, eight chunks) rows r and r + 2 share banks,
// so the chunk is XOR-ed with (r >> 1) & 7 instead: distinct over any 16
// consecutive rows of the same parity. Both forms repeat every 16 rows, so a
// fragment row's swizzle is that of its lane row.
template <class C>
__device__ __forceinline__ int swz(int r) {
  if constexpr (C::CH == 8) return (r >> 1) & 7;
  return (r >> 2) & 3;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Issue the direct-to-LDS loads of one slab (byte offset kbytes along K)
// into stage `st`. Wave w fills A blocks w, w+4, ... and B blocks w, w+4, ...
// (RPI rows, 1 KiB each); lane l of a block writes bytes [16 l, 16 l + 16)
// of the block, i.e. row l / CH, physical chunk l % CH, so it loads logical
// chunk (l % CH) ^ swz(row).
// PART selects the loads: all of them (-1), the first (0) or second (1)
// half of the wave's list (A blocks, then B blocks), or the A (2) or B (3)
// blocks only.
// NN: B0 is this slab's B source and kbytes_b the byte offset of its first
// row (A still advances by kbytes).
// WAVE_ROWS tiles: wave w fills A blocks NAW w .. NAW w + NAW - 1 instead
// (the rows BM/4 w .. BM/4 (w + 1) - 1, inside its own row range), and
// issues only the first NA of them: blocks wholly past the tile's last row
// would load zeros, which costs the fill path as much as loading data.
template <class C, int PART = -1, int NA = C::NAW>
__device__ __forceinline__ void dma_slab(char* __restrict__ st, Rsrc A, const uint32_t* aoff,
                                         Rsrc B0, Rsrc B1, const uint32_t* boff, int kbytes,
                                         int kbytes_b) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: LDS address in SALU
  const int kb = C::NN ? kbytes_b : kbytes;                          // B's offset along K
#pragma unroll
  for (int q = 0; q < C::NLW; ++q) {
    if ((PART == 0 || PART == 1) && (q < C::NLW / 2) != (PART == 0)) continue;
    if ((PART == 2 && q >= C::NAW) || (PART == 3 && q < C::NAW)) continue;
    if (q < C::NAW) {
      if (q >= NA) continue;
      const int slot = C::WAVE_ROWS ? C::NAW * w + q : w + 4 * q;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(A, (lds_ptr_t)(st + slot * 1024), 16,
                                               aoff[q], kbytes, 0, 0);
    } else {
      const int j = q - C::NAW;
      const bool up = C::DUAL && 4 * j * C::RPI >= C::BN;   // B block w + 4j holds up rows
      __builtin_amdgcn_raw_ptr_buffer_load_lds(up ? B1 : B0,
                                               (lds_ptr_t)(st + C::A_BYTES + (w + 4 * j) * 1024),
                                               16, boff[j], kb, 0, 0);
    }
  }
}

template <class C>
struct Frags {
  u32x4 a[C::FM];
  u32x4 b[C::NB][C::FN];
};

// Fragments of MFMA k-step ks (0 or 1) of the slab in stage `st`, for the
// first V of the wave's FM row blocks (the others hold only padding rows).
template <class C, int V>
__device__ __forceinline__ void read_frags(const char* __restrict__ st, int ks, Frags<C>& f) {
  if constexpr (V == 0) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int lr = lane & 31, lh = lane >> 5;
  const int co = (((ks * 2 + lh) ^ swz<C>(lr)) << 4);
  const char* a = st + (wm * C::TM + lr) * C::ROWB + co;
  const char* b = st + C::A_BYTES + (wn * C::TN + lr) * C::ROWB + co;
#pragma unroll
  for (int fm = 0; fm < V; ++fm)
    f.a[fm] = *reinterpret_cast<const u32x4*>(a + fm * 32 * C::ROWB);
  if constexpr (C::NN) {
    // lane j of 16-lane group q gets the four k values of column j from the
    // 8-byte reads of the group's lanes 4c + j/4 (row c, columns 4 (j % 4)..);
    // groups 0/1 and 2/3 take columns 0-15 / 16-31 of the block, and the two
    // k halves; two reads give the eight k values of the fragment
    const int i = lane & 15, g16 = (lane >> 4) & 1;
    const char* bb = st + C::A_BYTES;
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const int n = wn * C::TN + fn * 32 + 16 * g16 + 4 * (i & 3);
      v4i16 hv[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = 16 * ks + 8 * lh + 4 * h + (i >> 2);
        const char* q = bb + row * C::BROWB + (((n >> 3) ^ nn_swz(row)) << 4) + ((n & 7) << 1);
        hv[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t)q);
      }
      const u32x2 lo = __builtin_bit_cast(u32x2, hv[0]), hi = __builtin_bit_cast(u32x2, hv[1]);
      f.b[0][fn] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
    return;
  }
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
      f.b[nb][fn] = *reinterpret_cast<const u32x4*>(b + (nb * C::BN + fn * 32) * C::ROWB);
}

template <class C, int V>
__device__ __forceinline__ void mma(const Frags<C>& f, f32x16 (&acc)[C::NB][C::FM][C::FN]) {
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int fm = 0; fm < V; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
        acc[nb][fm][fn] = mfma_32x32x16(f.a[fm], f.b[nb][fn], acc[nb][fm][fn]);
}

// s_waitcnt vmcnt(n) (n < 64) leaving the other counters alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt(((N >> 4) << 14) | (0xF << 8) | (0x7 << 4) | (N & 15));
}

// s_waitcnt vmcnt(n) lgkmcnt(0): also every LDS read of this wave is done,
// so that once all waves pass the following barrier, a stage they read can
// be overwritten by loads.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt(((N >> 4) << 14) | (0x0 << 8) | (0x7 << 4) | (N & 15));
}

// Scheduling hints for one MFMA k-step (one wave per SIMD): the next
// k-step's fragment reads go between the first MFMAs, and `LOADS`
// direct-to-LDS loads are spread evenly over all MFMAs (SPREAD) or over the
// ones after the reads. A wave that issues loads back to back waits behind
// the other waves' loads at the CU's load unit and leaves its MFMA pipe idle;
// one load every few MFMAs measured fastest. The MFMAs of a k-step use
// distinct accumulators, so any order is valid.
template <class C, int V, int LOADS, bool READS, bool SPREAD = false>
__device__ __forceinline__ void weave() {
  constexpr int NMF = C::NB * V * C::FN;          // MFMAs per k-step
  // LDS reads of a k-step: one per A fragment, one per B fragment (two with
  // the NN transpose reads)
  constexpr int NRD = READS && V > 0 ? V + C::NB * C::FN * (C::NN ? 2 : 1) : 0;
  if constexpr (NMF == 0) return;
  constexpr int FIRST = (!SPREAD && LOADS > 0 && NRD < NMF) ? NRD : 0;   // first slot with loads
#pragma unroll
  for (int i = 0; i < NMF; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                      // MFMA
    if (i < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);         // LDS read
    if (LOADS > 0 && i >= FIRST) {
      const int n = (i - FIRST + 1) * LOADS / (NMF - FIRST) - (i - FIRST) * LOADS / (NMF - FIRST);
#pragma unroll
      for (int q = 0; q < n; ++q) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // load
    }
  }
}

// One K step k on stage S[j]: frags f0 (k-step 0) are already in registers.
//  1. read frags f1 (k-step 1) of S[j]; MFMAs on f0, with the first half of
//     the loads of slab k+STAGES-1 (clamped to the last slab) into the stage
//     slab k-1 occupied (free since the previous barrier)
//  2. wait until this wave's loads of slab k+1 are done and its LDS reads
//     too; barrier: slab k+1 is complete in its stage and every wave has
//     read all of S[j]
//  3. read frags f0 of slab k+1; MFMAs on f1, with the second half of the
//     loads. Spreading the loads over both halves keeps any one wave from
//     queueing several loads behind the other waves' between two MFMAs.
template <class C, int V>
__device__ __forceinline__ void k_step(char* __restrict__ cur, char* __restrict__ nxt,
                                       char* __restrict__ dst, int kload_bytes, int kload_b,
                                       Rsrc B0, Frags<C>& f0, Frags<C>& f1, Rsrc A,
                                       const uint32_t* aoff, Rsrc B1, const uint32_t* boff,
                                       f32x16 (&acc)[C::NB][C::FM][C::FN]) {
  read_frags<C, V>(cur, 1, f1);
  mma<C, V>(f0, acc);
  dma_slab<C, 0>(dst, A, aoff, B0, B1, boff, kload_bytes, kload_b);
  weave<C, V, C::NLW / 2, true, true>();
  wait_vmcnt_lds<(C::STAGES - 2) * C::NLW - C::NLW / 2>();
  __builtin_amdgcn_s_barrier();
  read_frags<C, V>(nxt, 0, f0);
  mma<C, V>(f1, acc);
  dma_slab<C, 1>(dst, A, aoff, B0, B1, boff, kload_bytes, kload_b);
  weave<C, V, C::NLW - C::NLW / 2, true, true>();
}

// ------------------------------------------------- 64-deep slabs, 2 stages
// One slab (4 MFMA k-steps) computed from `cur`. The next slab's loads into
// `nxt` went out in two halves: the first right after the previous slab's
// barrier (when `nxt`, read last before that barrier, became free), the
// second with this slab's first k-step; the wait for them (and for this
// wave's reads of `cur`) and the barrier come after the third k-step, and
// the last k-step, which reads the next slab's first fragments, issues the
// first half of the slab after next into `cur`. No branch inside: loads
// past the last slab re-load it into the free stage. The first half is the
// A blocks (NA of them issued), the second the B blocks.
template <class C, int V, int NA>
__device__ __forceinline__ void slab_k64(char* __restrict__ cur, char* __restrict__ nxt,
                                         int knext, int knext2, Frags<C>& f0, Frags<C>& f1,
                                         Rsrc A, const uint32_t* aoff, Rsrc B0, Rsrc B1,
                                         const uint32_t* boff,
                                         f32x16 (&acc)[C::NB][C::FM][C::FN]) {
  read_frags<C, V>(cur, 1, f1);
  mma<C, V>(f0, acc);
  dma_slab<C, 1>(nxt, A, aoff, B0, B1, boff, knext, knext);
  weave<C, V, C::NLW - C::NLW / 2, true, true>();
  read_frags<C, V>(cur, 2, f0);
  mma<C, V>(f1, acc);
  weave<C, V, 0, true, true>();
  read_frags<C, V>(cur, 3, f1);
  mma<C, V>(f0, acc);
  weave<C, V, 0, true, true>();
  wait_vmcnt_lds<0>();
  __builtin_amdgcn_s_barrier();
  read_frags<C, V>(nxt, 0, f0);
  mma<C, V>(f1, acc);
  dma_slab<C, 0, NA>(cur, A, aoff, B0, B1, boff, knext2, knext2);
  weave<C, V, NA, true, true>();
}

// A blocks wave (wm, wn) must load for V valid row blocks of its wave row:
// those that start below row 32 V of the wave row (WAVE_ROWS tiles; all of
// them otherwise).
template <class C>
constexpr int na_k64(int V, int wn) {
  if (!C::WAVE_ROWS) return C::NAW;
  const int n = (32 * V - wn * C::NAW * C::RPI) / C::RPI;
  return n < 0 ? 0 : (n > C::NAW ? C::NAW : n);
}

// pre: the first slab's loads into S0 were issued already (by the
// persistent weight-gradient kernel, before the previous tile's epilogue).
template <class C, int V, int NA>
__device__ __forceinline__ void mainloop_k64(char* __restrict__ S0, char* __restrict__ S1, Rsrc A,
                                             const uint32_t* aoff, Rsrc B0, Rsrc B1,
                                             const uint32_t* boff, int k_begin, int k_len,
                                             f32x16 (&acc)[C::NB][C::FM][C::FN],
                                             bool pre = false) {
  static_assert(C::BK == 64 && C::STAGES == 2 && !C::NN, "64-deep slabs: two stages");
  static_assert(C::NAW == C::NBW, "A blocks are the first half of a wave's loads");
  constexpr int STEP = C::BK * 2;
  const int KT = k_len / C::BK;
  const int kb = k_begin * 2;
  auto kbyte = [&](int k) { return kb + min(k, KT - 1) * STEP; };
  Frags<C> f0, f1;
  if (!pre) dma_slab<C, -1, NA>(S0, A, aoff, B0, B1, boff, kb, kb);
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  read_frags<C, V>(S0, 0, f0);
  dma_slab<C, 0, NA>(S1, A, aoff, B0, B1, boff, kbyte(1), kbyte(1));
  int k = 0;
  for (; k + 2 <= KT; k += 2) {
    slab_k64<C, V, NA>(S0, S1, kbyte(k + 1), kbyte(k + 2), f0, f1, A, aoff, B0, B1, boff, acc);
    slab_k64<C, V, NA>(S1, S0, kbyte(k + 2), kbyte(k + 3), f0, f1, A, aoff, B0, B1, boff, acc);
  }
  if (k < KT)
    slab_k64<C, V, NA>(S0, S1, kbyte(k + 1), kbyte(k + 2), f0, f1, A, aoff, B0, B1, boff, acc);
  wait_vmcnt<0>();
  __syncthreads();
}

// ------------------------------------------------- 64-deep slabs, 3 stages
// Loads run two slabs ahead, so twice the bytes are in flight: for tiles of
// few rows the weight columns come from HBM at every slab, and one slab in
// flight per CU leaves HBM latency-bound. Slab k computes from stage k % 3;
// its first k-step issues the B blocks of slab k + 2, its second the A
// blocks, into the stage slab k - 1 used (its reads ended before the
// barrier that closed slab k - 1). After the third k-step a wave waits until
// at most slab k + 2's loads are outstanding (loads complete in issue
// order), then the barrier; the fourth k-step reads slab k + 1's first
// fragments. Loads past the last slab re-load it into the free stage.
template <class C, int V, int NA>
__device__ __forceinline__ void slab_k64_3(char* __restrict__ cur, char* __restrict__ nxt,
                                           char* __restrict__ dst, int kload, Frags<C>& f0,
                                           Frags<C>& f1, Rsrc A, const uint32_t* aoff, Rsrc B0,
                                           Rsrc B1, const uint32_t* boff,
                                           f32x16 (&acc)[C::NB][C::FM][C::FN]) {
  read_frags<C, V>(cur, 1, f1);
  mma<C, V>(f0, acc);
  dma_slab<C, 3>(dst, A, aoff, B0, B1, boff, kload, kload);
  weave<C, V, C::NBW, true, true>();
  read_frags<C, V>(cur, 2, f0);
  mma<C, V>(f1, acc);
  dma_slab<C, 2, NA>(dst, A, aoff, B0, B1, boff, kload, kload);
  weave<C, V, NA, true, true>();
  read_frags<C, V>(cur, 3, f1);
  mma<C, V>(f0, acc);
  weave<C, V, 0, true, true>();
  wait_vmcnt_lds<NA + C::NBW>();
  __builtin_amdgcn_s_barrier();
  read_frags<C, V>(nxt, 0, f0);
  mma<C, V>(f1, acc);
  weave<C, V, 0, true, true>();
}

template <class C, int V, int NA>
__device__ __forceinline__ void mainloop_k64_3(char* __restrict__ S0, char* __restrict__ S1,
                                               char* __restrict__ S2, Rsrc A,
                                               const uint32_t* aoff, Rsrc B0, Rsrc B1,
                                               const uint32_t* boff, int k_begin, int k_len,
                                               f32x16 (&acc)[C::NB][C::FM][C::FN]) {
  static_assert(C::BK == 64 && C::STAGES == 3 && !C::NN, "64-deep slabs: three stages");
  static_assert(C::WN * C::NAW * C::RPI == C::TM, "a wave row's waves load its rows");
  constexpr int STEP = C::BK * 2;
  const int KT = k_len / C::BK;
  const int kb = k_begin * 2;
  auto kbyte = [&](int k) { return kb + min(k, KT - 1) * STEP; };
  Frags<C> f0, f1;
  dma_slab<C, -1, NA>(S0, A, aoff, B0, B1, boff, kb, kb);
  dma_slab<C, -1, NA>(S1, A, aoff, B0, B1, boff, kbyte(1), kbyte(1));
  wait_vmcnt<NA + C::NBW>();
  __builtin_amdgcn_s_barrier();
  read_frags<C, V>(S0, 0, f0);
  int k = 0;
  for (; k + 3 <= KT; k += 3) {
    slab_k64_3<C, V, NA>(S0, S1, S2, kbyte(k + 2), f0, f1, A, aoff, B0, B1, boff, acc);
    slab_k64_3<C, V, NA>(S1, S2, S0, kbyte(k + 3), f0, f1, A, aoff, B0, B1, boff, acc);
    slab_k64_3<C, V, NA>(S2, S0, S1, kbyte(k + 4), f0, f1, A, aoff, B0, B1, boff, acc);
  }
  if (k < KT)
    slab_k64_3<C, V, NA>(S0, S1, S2, kbyte(k + 2), f0, f1, A, aoff, B0, B1, boff, acc);
  if (k + 1 < KT)
    slab_k64_3<C, V, NA>(S1, S2, S0, kbyte(k + 3), f0, f1, A, aoff, B0, B1, boff, acc);
  wait_vmcnt<0>();
  __syncthreads();
}

// acc += A[rows] · B[cols]^T over k in [k_begin, k_begin + k_len) (k_len a
// multiple of 32). Loads run STAGES-1 slabs ahead of the MFMAs through a
// ring of LDS stages; the loop is unrolled by STAGES so that every stage is
// a distinct LDS object. Loads past the last slab re-load the last slab, so
// every step issues the same number of loads and the vmcnt accounting holds.
// NN: B rows (K) are ldb_bytes apart; rows at and past nn_k1 (when > 0) come
// from B1 at row - nn_k1, the others from B0.
template <class C, int V = C::FM>
__device__ __forceinline__ void mainloop(char* __restrict__ S0, char* __restrict__ S1,
                                         char* __restrict__ S2, char* __restrict__ S3,
                                         Rsrc A, const uint32_t* aoff, Rsrc B0, Rsrc B1,
                                         const uint32_t* boff, int k_begin, int k_len,
                                         f32x16 (&acc)[C::NB][C::FM][C::FN],
                                         int ldb_bytes = 0, int nn_k1 = 0, bool pre = false) {
  constexpr int STEP = C::BK * 2;
  const int KT = k_len / C::BK;
  const int kb = k_begin * 2;
  auto kbyte = [&](int k) { return kb + min(k, KT - 1) * STEP; };
  // this slab's B source and the byte offset of its first B row
  auto brow = [&](int k) { return k_begin + min(k, KT - 1) * C::BK; };
  auto bsrc = [&](int k) {
    if constexpr (C::NN) return (nn_k1 > 0 && brow(k) >= nn_k1) ? B1 : B0;
    return B0;
  };
  auto kbyte_b = [&](int k) {
    if constexpr (C::NN) {
      const int r = brow(k);
      return (nn_k1 > 0 && r >= nn_k1 ? r - nn_k1 : r) * ldb_bytes;
    }
    return kbyte(k);
  };
  if constexpr (C::BK == 64) {
    // the wave's A block count depends on its column in the wave grid too
    constexpr int NA0 = na_k64<C>(V, 0), NA1 = na_k64<C>(V, 1);
    const bool first = NA0 == NA1 || __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) % C::WN == 0;
    if constexpr (C::STAGES == 3) {
      if (first)
        mainloop_k64_3<C, V, NA0>(S0, S1, S2, A, aoff, B0, B1, boff, k_begin, k_len, acc);
      else
        mainloop_k64_3<C, V, NA1>(S0, S1, S2, A, aoff, B0, B1, boff, k_begin, k_len, acc);
    } else {
      if (first)
        mainloop_k64<C, V, NA0>(S0, S1, A, aoff, B0, B1, boff, k_begin, k_len, acc, pre);
      else
        mainloop_k64<C, V, NA1>(S0, S1, A, aoff, B0, B1, boff, k_begin, k_len, acc, pre);
    }
    return;
  }
  Frags<C> f0, f1;
  // (the k_step calls are spelled out: wrapping them in a lambda changed the
  // register allocation and doubled the NN tiles' time)
  if constexpr (C::STAGES == 4) {
    dma_slab<C>(S0, A, aoff, bsrc(0), B1, boff, kbyte(0), kbyte_b(0));
    dma_slab<C>(S1, A, aoff, bsrc(1), B1, boff, kbyte(1), kbyte_b(1));
    dma_slab<C>(S2, A, aoff, bsrc(2), B1, boff, kbyte(2), kbyte_b(2));
    wait_vmcnt<2 * C::NLW>();
    __builtin_amdgcn_s_barrier();
    read_frags<C, V>(S0, 0, f0);
    int k = 0;
    for (; k + 4 <= KT; k += 4) {
      k_step<C, V>(S0, S1, S3, kbyte(k + 3), kbyte_b(k + 3), bsrc(k + 3), f0, f1, A, aoff, B1, boff, acc);
      k_step<C, V>(S1, S2, S0, kbyte(k + 4), kbyte_b(k + 4), bsrc(k + 4), f0, f1, A, aoff, B1, boff, acc);
      k_step<C, V>(S2, S3, S1, kbyte(k + 5), kbyte_b(k + 5), bsrc(k + 5), f0, f1, A, aoff, B1, boff, acc);
      k_step<C, V>(S3, S0, S2, kbyte(k + 6), kbyte_b(k + 6), bsrc(k + 6), f0, f1, A, aoff, B1, boff, acc);
    }
    if (k < KT) k_step<C, V>(S0, S1, S3, kbyte(k + 3), kbyte_b(k + 3), bsrc(k + 3), f0, f1, A, aoff, B1, boff, acc);
    if (k + 1 < KT) k_step<C, V>(S1, S2, S0, kbyte(k + 4), kbyte_b(k + 4), bsrc(k + 4), f0, f1, A, aoff, B1, boff, acc);
    if (k + 2 < KT) k_step<C, V>(S2, S3, S1, kbyte(k + 5), kbyte_b(k + 5), bsrc(k + 5), f0, f1, A, aoff, B1, boff, acc);
  } else if constexpr (C::STAGES == 3) {
    dma_slab<C>(S0, A, aoff, bsrc(0), B1, boff, kbyte(0), kbyte_b(0));
    dma_slab<C>(S1, A, aoff, bsrc(1), B1, boff, kbyte(1), kbyte_b(1));
    wait_vmcnt<C::NLW>();
    __builtin_amdgcn_s_barrier();
    read_frags<C, V>(S0, 0, f0);
    int k = 0;
    for (; k + 3 <= KT; k += 3) {
      k_step<C, V>(S0, S1, S2, kbyte(k + 2), kbyte_b(k + 2), bsrc(k + 2), f0, f1, A, aoff, B1, boff, acc);
      k_step<C, V>(S1, S2, S0, kbyte(k + 3), kbyte_b(k + 3), bsrc(k + 3), f0, f1, A, aoff, B1, boff, acc);
      k_step<C, V>(S2, S0, S1, kbyte(k + 4), kbyte_b(k + 4), bsrc(k + 4), f0, f1, A, aoff, B1, boff, acc);
    }
    if (k < KT) k_step<C, V>(S0, S1, S2, kbyte(k + 2), kbyte_b(k + 2), bsrc(k + 2), f0, f1, A, aoff, B1, boff, acc);
    if (k + 1 < KT) k_step<C, V>(S1, S2, S0, kbyte(k + 3), kbyte_b(k + 3), bsrc(k + 3), f0, f1, A, aoff, B1, boff, acc);
  }
  wait_vmcnt<0>();
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

// SWIGLU: SiLU(gate)·up; STORE_BF16: the accumulator; STORE_DUAL: the gate
// and up accumulators side by side, gate in columns [0, Ncols) and up in
// [Ncols, 2 Ncols) of each output row (the backward pass's recompute of the
// pre-activations).
// STORE_F32 / STORE_DUAL_F32: the same as fp32 (the backward pass's
// intermediates that feed a reduction).
// SWIGLU_SAVE: SWIGLU, and the fp32 gate and up accumulators side by side
// in a second output (the training forward keeps them for the backward).
enum Epi { EPI_SWIGLU = 0, EPI_STORE_BF16 = 1, EPI_STORE_DUAL = 2, EPI_STORE_F32 = 3,
           EPI_STORE_DUAL_F32 = 4, EPI_SWIGLU_SAVE = 5 };

// Output column of MFMA block fn, lane column lr, in a wave's TN-wide strip:
// B rows are staged so that blocks 2j and 2j+1 hold the even and odd columns
// of the 64-column group j. Each lane then owns two adjacent output columns
// of the same rows, stored as one packed bf16 pair.
__device__ __forceinline__ int strip_col(int fn, int lr) {
  return (fn >> 1) * 64 + 2 * lr + (fn & 1);
}

// Epilogue: SiLU(gate)·up (SWIGLU) or the accumulator, rounded to bf16
// (hardware round-to-nearest-even), stored straight from registers as 4-byte
// column pairs: a store instruction writes two full 128-byte row segments.
// Raw buffer stores over the tile's valid rows: rows past the group's end
// fall outside the descriptor and are dropped, columns past Ncols get an
// out-of-range offset, so there are no branches.
template <class C, int EPI>
__device__ __forceinline__ void epilogue_bf16(const f32x16 (&acc)[C::NB][C::FM][C::FN],
                                              void* __restrict__ Cout, int64_t ldc,
                                              int64_t row0_out, int rows_valid, int n0,
                                              int Ncols, float* __restrict__ C2 = nullptr,
                                              int64_t ldc2_el = 0) {
  static_assert(C::FN % 2 == 0, "column pairs need an even number of MFMA blocks");
  constexpr bool F32 = EPI == EPI_STORE_F32 || EPI == EPI_STORE_DUAL_F32;
  constexpr bool TWO = EPI == EPI_STORE_DUAL || EPI == EPI_STORE_DUAL_F32;
  constexpr int ES = F32 ? 4 : 2;      // output element bytes
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index, tile origin and extent are uniform: keep them scalar (they
  // can come back from spill slots as vector values, and a buffer store with
  // a vector descriptor or soffset turns into a loop over lanes)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int lr = lane & 31, lh = lane >> 5;
  rows_valid = __builtin_amdgcn_readfirstlane(rows_valid);
  n0 = __builtin_amdgcn_readfirstlane(n0);
  const uint32_t r0lo = __builtin_amdgcn_readfirstlane((uint32_t)row0_out);
  const uint32_t r0hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)row0_out >> 32));
  row0_out = (int64_t)(((uint64_t)r0hi << 32) | r0lo);
  // Row stride in bytes, made opaque so the compiler recomputes the row
  // offsets per tile instead of hoisting (and spilling) all of them.
  int ldc2 = (int)ldc * ES;
  asm volatile("" : "+s"(ldc2));
  const Rsrc out = make_rsrc(static_cast<char*>(Cout) + row0_out * ldc * ES,
                             (uint32_t)rows_valid * (uint32_t)ldc2);
  const uint32_t lane_row = (uint32_t)(4 * lh) * (uint32_t)ldc2;
  // second output (SWIGLU_SAVE): fp32 rows of 2 Ncols
  int ldcs = (int)ldc2_el * 4;
  asm volatile("" : "+s"(ldcs));
  Rsrc out2 = out;
  uint32_t lane_row2 = 0;
  if constexpr (EPI == EPI_SWIGLU_SAVE) {
    out2 = make_rsrc(C2 + row0_out * ldc2_el, (uint32_t)rows_valid * (uint32_t)ldcs);
    lane_row2 = (uint32_t)(4 * lh) * (uint32_t)ldcs;
  }
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
    const int rb = wm * C::TM + fm * 32;
    if (rb >= rows_valid) break;             // the rest of this wave's rows are padding
    if constexpr (C::NN) {
      // NN tiles keep plain columns (MFMA block fn, lane column lr -> fn·32 +
      // lr): one store per element
      static_assert(EPI == EPI_STORE_BF16 || EPI == EPI_STORE_F32, "NN: plain stores only");
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) {
        const int col = n0 + wn * C::TN + fn * 32 + lr;
        const uint32_t voff = col < Ncols ? lane_row + (uint32_t)col * ES : 0xC0000000u;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int rrow = rb + 8 * (i >> 2) + (i & 3);   // + 4*lh (in voff)
          if constexpr (F32)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[0][fm][fn][i]), out, voff,
                                                  rrow * ldc2, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b16(
                (unsigned short)(pack_bf16x2_hw(acc[0][fm][fn][i], 0.0f) & 0xffffu), out, voff,
                rrow * ldc2, 0);
        }
      }
      continue;
    }
#pragma unroll
    for (int fe = 0; fe < C::FN; fe += 2) {
      const int col = n0 + wn * C::TN + strip_col(fe, lr);
      const uint32_t voff = col < Ncols ? lane_row + (uint32_t)col * ES : 0xC0000000u;
      const uint32_t voff_up = col < Ncols ? voff + (uint32_t)Ncols * ES : 0xC0000000u;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rrow = rb + 8 * (i >> 2) + (i & 3);   // + 4*lh (in voff)
        static_assert(!TWO || C::DUAL, "storing gate and up needs both");
        if constexpr (F32) {
          // two 4-byte stores per column pair (a 2-vector 8-byte store built
          // here was compiled to store one row's data to every row)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[0][fm][fe + h2][i]), out,
                                                  voff + 4 * h2, rrow * ldc2, 0);
            if constexpr (TWO)
              __builtin_amdgcn_raw_buffer_store_b32(
                  __float_as_uint(acc[C::NB - 1][fm][fe + h2][i]), out, voff_up + 4 * h2,
                  rrow * ldc2, 0);
          }
          continue;
        }
        if constexpr (TWO) {
          __builtin_amdgcn_raw_buffer_store_b32(
              pack_bf16x2_hw(acc[0][fm][fe][i], acc[0][fm][fe + 1][i]), out, voff, rrow * ldc2, 0);
          __builtin_amdgcn_raw_buffer_store_b32(
              pack_bf16x2_hw(acc[C::NB - 1][fm][fe][i], acc[C::NB - 1][fm][fe + 1][i]), out,
              voff_up, rrow * ldc2, 0);
          continue;
        }
        if constexpr (EPI == EPI_SWIGLU_SAVE) {
          const uint32_t v2 = col < Ncols ? lane_row2 + (uint32_t)col * 4u : 0xC0000000u;
          const uint32_t v2u = col < Ncols ? v2 + (uint32_t)Ncols * 4u : 0xC0000000u;
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[0][fm][fe + h2][i]), out2,
                                                  v2 + 4 * h2, rrow * ldcs, 0);
            __builtin_amdgcn_raw_buffer_store_b32(
                __float_as_uint(acc[C::NB - 1][fm][fe + h2][i]), out2, v2u + 4 * h2,
                rrow * ldcs, 0);
          }
        }
        float v0, v1;
        if (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_SAVE) {
          v0 = silu_fast(acc[0][fm][fe][i]) * acc[C::NB - 1][fm][fe][i];
          v1 = silu_fast(acc[0][fm][fe + 1][i]) * acc[C::NB - 1][fm][fe + 1][i];
        } else {
          v0 = acc[0][fm][fe][i];
          v1 = acc[0][fm][fe + 1][i];
        }
        __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2_hw(v0, v1), out, voff,
                                              rrow * ldc2, 0);
      }
    }
  }
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

// Per-lane load offsets of the DMA blocks of wave w: A block w + 4j holds
// tile rows RPI(w + 4j) .. +RPI-1 (WAVE_ROWS tiles: block NAW w + j, rows
// RPI(NAW w + j) .. +RPI-1); lane l loads the block's row l/CH, logical
// chunk (l % CH) ^ swz(row). Rows past the group's end load zeros: their
// MFMAs then work on zero operands, which draws less power than repeating a
// real row (the GEMMs run at the power limit), and they are never stored.
template <class C>
__device__ __forceinline__ void dma_offsets(uint32_t (&aoff)[C::NAW], uint32_t (&boff)[C::NBW],
                                            const int32_t* perm, int kdiv, int lda, int m0,
                                            int m_end, int ldb, int n0, int Ncols) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rl = lane / C::CH, ch = lane % C::CH;
#pragma unroll
  for (int j = 0; j < C::NAW; ++j) {
    const int row = C::RPI * (C::WAVE_ROWS ? C::NAW * w + j : w + 4 * j) + rl;
    const int r = m0 + row;
    if (r >= m_end) {
      aoff[j] = 0x80000000u;    // past the descriptor's extent: the load returns zeros
    } else {
      const int src = perm ? perm[r] / kdiv : r;
      aoff[j] = (uint32_t)(src * lda * 2 + ((ch ^ swz<C>(row)) << 4));
    }
  }
  if constexpr (C::NN) {
    // B block w + 4j covers bytes [1 KiB (w + 4j), +1 KiB) of the B part:
    // staged row (k) r, physical chunk c holds columns n0 + 8 (c ^ nn_swz(r));
    // columns past Ncols read zeros
#pragma unroll
    for (int j = 0; j < C::NBW; ++j) {
      const int byte = 1024 * (w + 4 * j) + 16 * lane;
      const int r = byte / C::BROWB, c = (byte % C::BROWB) / 16;
      const int col = n0 + 8 * (c ^ nn_swz(r));
      boff[j] = col < Ncols ? (uint32_t)(r * ldb * 2 + col * 2) : 0x80000000u;
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < C::NBW; ++j) {
    const int row = C::RPI * (w + 4 * j) + rl;  // B row within the stage's B part
    const int q = row % C::BN;                  // staged row -> output column (strip_col)
    const int col = min(n0 + (q & ~63) + 2 * (q & 31) + ((q >> 5) & 1), Ncols - 1);
    boff[j] = (uint32_t)(col * ldb * 2 + ((ch ^ swz<C>(C::BM + row)) << 4));
  }
}

// Tile t of the tile list -> expert g, rows [m0, m_end), first column n0.
// Tile order: groups of GN n-tiles, m-tiles (all experts) inside, so the
// blocks of one XCD that run at the same time (neighbouring tiles) cover
// many m-tiles of few experts and share their B columns in L2, and pairs of
// them share A rows. GN = 2: narrower groups measured faster than 4, 8 or 16 on the
// Mixtral, Qwen3-30B and DeepSeek-V3 shapes (fewer weight re-reads), except
// where the experts average at most 1.5 m-tiles: then an expert's B columns
// are read by one tile anyway, and the down-type GEMM is faster with groups
// of GN = 8 n-tiles sharing the A rows (DeepSeek-V3 shape: 2.05 -> 1.94 ms).
// Past the offsets' G groups, group G is the problem's extra group (X0):
// its A rows x_a_row0 + r are read in order, its output rows are
// x_c_row0 + r. c0 is the output row of the tile's first row.
struct TileInfo {
  int g, m0, m_end, n0;
  int64_t c0;
  bool x;
};
template <class C>
__device__ __forceinline__ int tile_group_width(int total_mt, int G) {
  // 128-row tiles on 64-deep slabs: at most 2 m-tiles per expert on average
  // (DeepSeek-V3 shape, down: 2.04 -> 1.93 ms; the Qwen3-30B shape, 4.5
  // m-tiles per expert, measured no gain)
  if constexpr (C::BK == 64 && C::STAGES == 3) return (!C::DUAL && total_mt <= 2 * G) ? 8 : 2;
  return (!C::DUAL && 2 * total_mt <= 3 * G) ? 8 : 2;
}
template <class C>
__device__ __forceinline__ TileInfo tile_info(const GroupedProblem& p, const int* s_pref, int G,
                                              int total_mt, int nt_n, int64_t t, int GN) {
  const int64_t sg = (int64_t)total_mt * GN;
  const int nsup = (int)(t / sg);
  const int within = (int)(t - (int64_t)nsup * sg);
  const int width = min(GN, nt_n - nsup * GN);
  const int mt = within / width;
  const int nt = nsup * GN + within % width;
  // m-tile -> group (binary search in the prefix)
  int lo = 0, hi = G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_pref[mid] <= mt) lo = mid; else hi = mid;
  }
  // every lane computed the same values from LDS; say so to the compiler,
  // so that descriptors and bounds live in scalar registers
  TileInfo ti;
  ti.g = __builtin_amdgcn_readfirstlane(lo);
  const int lm0 = (mt - __builtin_amdgcn_readfirstlane(s_pref[ti.g])) * C::BM;
  ti.n0 = nt * C::BN;
  ti.x = p.X0 && ti.g == (p.offsets ? p.groups : 1);
  if (ti.x) {
    const int a0 = (int)p.x_a_row0;
    ti.m0 = a0 + lm0;
    ti.m_end = a0 + min(lm0 + C::BM, p.x_rows);
    ti.c0 = p.x_c_row0 + lm0;
    return ti;
  }
  const int gbase = p.offsets ? __builtin_amdgcn_readfirstlane(p.offsets[ti.g]) : 0;
  const int gend = p.offsets ? __builtin_amdgcn_readfirstlane(p.offsets[ti.g + 1]) : p.M;
  ti.m0 = gbase + lm0;
  ti.m_end = min(ti.m0 + C::BM, gend);
  ti.c0 = p.c_row0 + ti.m0;
  return ti;
}

// mainloop<C, v> for the run-time v in [0, W] (a wave-uniform branch).
template <class C, int W>
__device__ __forceinline__ void mainloop_rows(int v, char* S0, char* S1, char* S2, char* S3,
                                              Rsrc A, const uint32_t* aoff, Rsrc B0, Rsrc B1,
                                              const uint32_t* boff, int k_begin, int k_len,
                                              f32x16 (&acc)[C::NB][C::FM][C::FN],
                                              int ldb_bytes = 0, int nn_k1 = 0,
                                              bool pre = false) {
  if (v == W || W == 0) {
    mainloop<C, W>(S0, S1, S2, S3, A, aoff, B0, B1, boff, k_begin, k_len, acc, ldb_bytes, nn_k1,
                   pre);
    return;
  }
  if constexpr (W > 0)
    mainloop_rows<C, W - 1>(v, S0, S1, S2, S3, A, aoff, B0, B1, boff, k_begin, k_len, acc,
                            ldb_bytes, nn_k1, pre);
}

// acc = A[tile rows] · B[tile columns]^T over k in [k_begin, k_begin + k_len).
template <class C>
__device__ __forceinline__ void tile_mainloop(const GroupedProblem& p, const TileInfo& ti, Rsrc rA,
                                              char* S0, char* S1, char* S2, char* S3,
                                              int k_begin, int k_len,
                                              f32x16 (&acc)[C::NB][C::FM][C::FN]) {
  uint32_t aoff[C::NAW], boff[C::NBW];
  dma_offsets<C>(aoff, boff, ti.x ? nullptr : p.perm, p.kdiv, p.lda, ti.m0, ti.m_end, p.ldb,
                 ti.n0, p.Ncols);
  Rsrc rB0, rB1;
  if constexpr (C::NN) {
    // B0 holds K rows [0, k1) (all K when k1 = 0), B1 rows [k1, K)
    const int k1 = p.b_k1 > 0 ? p.b_k1 : p.K;
    const int64_t rowb = (int64_t)p.ldb * 2;
    rB0 = make_rsrc(static_cast<const bf16_t*>(p.B0) + (int64_t)ti.g * p.b_gstride,
                    (uint32_t)(k1 * rowb));
    rB1 = p.b_k1 > 0 ? make_rsrc(static_cast<const bf16_t*>(p.B1) + (int64_t)ti.g * p.b_gstride,
                                 (uint32_t)((p.K - k1) * rowb))
                     : rB0;
  } else {
    const uint32_t bbytes = (uint32_t)((int64_t)p.Ncols * p.ldb * 2);
    const bf16_t* b0 = ti.x ? static_cast<const bf16_t*>(p.X0)
                            : static_cast<const bf16_t*>(p.B0) + (int64_t)ti.g * p.b_gstride;
    rB0 = make_rsrc(b0, bbytes);
    if constexpr (C::DUAL) {
      const bf16_t* b1 = ti.x ? static_cast<const bf16_t*>(p.X1)
                              : static_cast<const bf16_t*>(p.B1) + (int64_t)ti.g * p.b_gstride;
      rB1 = make_rsrc(b1, bbytes);
    } else {
      rB1 = rB0;
    }
  }
  zero_acc<C>(acc);
  // row blocks of this wave that hold rows of the group: the MFMAs of the
  // others would only multiply padding (zeros), so they are not issued
  const int wm = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) / C::WN;
  const int v = min(max((ti.m_end - ti.m0 - wm * C::TM + 31) / 32, 0), C::FM);
  mainloop_rows<C, C::FM>(v, S0, S1, S2, S3, rA, aoff, rB0, rB1, boff, k_begin, k_len, acc,
                          p.ldb * 2, p.b_k1);
}

// A tile's fp32 partial sums in the split-K workspace, element-major
// ([element][thread]) so that every wave instruction covers 1 KiB. Splits of
// one tile may run on different XCDs, each with its own L2, so partials are
// written and read with agent-scope coherent accesses (sc1, the form of a
// relaxed agent-scope atomic load or store): no cache-wide write-back or
// invalidate is needed, only the completion of the stores before the
// arrival counter (an agent-scope atomic) is bumped.
constexpr int kSc1 = 16;   // buffer cache-policy bit: agent-scope coherent
template <class C>
struct Partial {
  static constexpr int FLOATS = C::BM * C::BN * C::NB;
};
template <class C>
__device__ __forceinline__ void store_partial(Rsrc r, int soff,
                                              const f32x16 (&acc)[C::NB][C::FM][C::FN]) {
  int e = 0;
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int i = 0; i < 16; i += 4, ++e) {
          const f32x4 v = {acc[nb][fm][fn][i], acc[nb][fm][fn][i + 1], acc[nb][fm][fn][i + 2],
                           acc[nb][fm][fn][i + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r,
                                                 threadIdx.x * 16u, soff + e * kThreads * 16,
                                                 kSc1);
        }
}
// acc = partial (FIRST) or acc += partial, element by element.
template <class C, bool FIRST>
__device__ __forceinline__ void add_partial(Rsrc r, int soff, f32x16 (&acc)[C::NB][C::FM][C::FN]) {
  int e = 0;
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int i = 0; i < 16; i += 4, ++e) {
          const f32x4 v = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, threadIdx.x * 16u,
                                                           soff + e * kThreads * 16, kSc1));
#pragma unroll
          for (int c = 0; c < 4; ++c)
            acc[nb][fm][fn][i + c] = FIRST ? v[c] : acc[nb][fm][fn][i + c] + v[c];
        }
}

constexpr int kMaxSplit = 8;        // K splits of one tail tile
constexpr int kMinSplitK = 2048;    // K per split at least
constexpr int kQueueCounters = (kSplitCounters - kXcds) / kXcds;   // tail tiles per queue

// Work plan of one queue: n tiles for B blocks. The tiles past the last
// full round (n mod B of them) are cut into S K-ranges each, so that the
// last round is made of short units instead of a few whole tiles.
struct QueuePlan {
  int64_t base, n, dp, items;   // first tile, tiles, whole tiles, work items
  int S;
};
template <class C>
__device__ __forceinline__ QueuePlan queue_plan(int64_t total, int x, int Q, int B, int KT,
                                                int64_t cap_floats) {
  QueuePlan q;
  q.base = total * x / Q;
  q.n = total * (x + 1) / Q - q.base;
  q.dp = q.n;
  q.S = 1;
  const int rem = (int)(q.n % B);
  if (rem > 0 && rem <= kQueueCounters) {
    int sp = min(B / rem, min(KT / (kMinSplitK / C::BK), kMaxSplit));
    sp = (int)min((int64_t)sp, cap_floats / ((int64_t)Partial<C>::FLOATS * rem));
    if (sp >= 2) {
      q.S = sp;
      q.dp = q.n - rem;
    }
  }
  q.items = q.dp + (q.n - q.dp) * q.S;
  return q;
}

// Persistent grouped GEMM. Every block first builds the exclusive prefix of
// m-tiles per group in LDS, then takes work from queues:
//  * XCD-aware queues: block b runs on XCD b % 8, and queue x holds the
//    contiguous tile range [x·n/8, (x+1)·n/8), so the ~32 tiles in flight
//    on one XCD share A rows and B columns in that XCD's L2. A block takes
//    the next item of its own queue with an atomic counter, and once that
//    queue is empty, items of the other queues; tile speed varies from CU
//    to CU, and dynamic assignment evens it out.
//  * split-K tail: each queue's last partial round of tiles is cut into S
//    K-ranges per tile. Every split stores its fp32 partial sums; the block
//    that arrives last at the tile's counter adds the S partials in split
//    order and runs the epilogue. No block waits on another, and each tile's
//    arithmetic is the same whichever blocks run it, so results do not
//    depend on timing.
// Without a workspace (p.part == NULL) the blocks walk a static schedule.
template <class C, int EPI>
__global__ __launch_bounds__(kThreads, C::OCC) void grouped_gemm_kernel(GroupedProblem p) {
  __shared__ __attribute__((aligned(1024))) char S0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char S1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char S2[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char S3[C::STAGES == 4 ? C::STAGE : 1024];
  __shared__ int s_pref[kMaxGroups + 1];
  __shared__ int s_item;
  __shared__ int s_last;
  const int tid = threadIdx.x;
  // the offsets' groups, then the extra group (launchers keep G <= kMaxGroups)
  const int G0 = p.offsets ? p.groups : 1;
  const int G = G0 + (p.X0 ? 1 : 0);

  if (tid < 64) {
    int loc[kMaxGroups / 64];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kMaxGroups / 64; ++i) {
      const int g = tid * (kMaxGroups / 64) + i;
      int c = 0;
      if (g < G) {
        const int rows = g == G0 ? p.x_rows
                                 : (p.offsets ? (p.offsets[g + 1] - p.offsets[g]) : p.M);
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

  const int total_mt = __builtin_amdgcn_readfirstlane(s_pref[G]);
  const int gn = tile_group_width<C>(total_mt, G);
  const int nt_n = (p.Ncols + C::BN - 1) / C::BN;
  const int64_t total = (int64_t)total_mt * nt_n;
  if (total == 0) return;

  const int nblk = gridDim.x, b = blockIdx.x;
  const bool xcd_split = nblk >= kXcds && nblk % kXcds == 0;
  const Rsrc rA = make_rsrc(p.A, p.a_bytes);
  const bool dynamic = p.part != nullptr;
  const int Q = xcd_split ? kXcds : 1;
  const int BQ = nblk / Q;                       // blocks per queue
  const int KT = p.K / C::BK;                    // K slabs
  const int64_t cap_q = p.part_floats / Q;       // partial floats per queue
  constexpr int64_t TF = Partial<C>::FLOATS;

  // static schedule: block b takes tiles t_next, t_next + t_step, ... < t_end
  int64_t t_next = b, t_end = total, t_step = nblk;
  if (xcd_split) {
    const int xcd = b % kXcds;
    t_next = total * xcd / kXcds + b / kXcds;
    t_end = total * (xcd + 1) / kXcds;
    t_step = nblk / kXcds;
  }
  // dynamic schedule: the next item of queue x is fetched with one atomic,
  // issued for item i+1 before item i's epilogue so that its latency hides
  // behind the stores
  int qi = 0, x = b % Q;
  QueuePlan q;
  int64_t it = 0;
  if (dynamic) {
    q = queue_plan<C>(total, x, Q, BQ, KT, cap_q);
    if (tid == 0) s_item = atomicAdd(p.part_cnt + x, 1);
    __syncthreads();
    it = __builtin_amdgcn_readfirstlane(s_item);
  }
  for (;;) {
    // ---- work item: tile t over K range [k0, k1); split s of S
    int64_t t;
    int S = 1, s = 0, j = 0;
    if (dynamic) {
      while (it >= q.items && qi < Q) {          // queue x is empty: next queue
        if (++qi == Q) break;
        x = (b % Q + qi) % Q;
        q = queue_plan<C>(total, x, Q, BQ, KT, cap_q);
        __syncthreads();                         // every thread has read s_item
        if (tid == 0) s_item = atomicAdd(p.part_cnt + x, 1);
        __syncthreads();
        it = __builtin_amdgcn_readfirstlane(s_item);
      }
      if (qi == Q) break;
      if (it < q.dp) {
        t = q.base + it;
      } else {
        const int u = (int)(it - q.dp);
        S = q.S;
        j = u / S;
        s = u - j * S;
        t = q.base + q.dp + j;
      }
    } else {
      if (t_next >= t_end) break;
      t = t_next;
      t_next += t_step;
    }
    const int k0 = (KT * s / S) * C::BK, k1 = (KT * (s + 1) / S) * C::BK;

    const TileInfo ti = tile_info<C>(p, s_pref, G, total_mt, nt_n, t, gn);
    f32x16 acc[C::NB][C::FM][C::FN];
    tile_mainloop<C>(p, ti, rA, S0, S1, S2, S3, k0, k1 - k0, acc);
    int nxt = 0;
    if (dynamic && tid == 0) nxt = atomicAdd(p.part_cnt + x, 1);
    bool write = true;
    if (S > 1) {
      // store this split's partial; the last split of the tile to arrive
      // sums all of them in split order and writes the tile
      const Rsrc rp = make_rsrc(p.part + (int64_t)x * cap_q + (int64_t)j * S * TF,
                                (uint32_t)(S * TF * sizeof(float)));
      store_partial<C>(rp, s * (int)(TF * sizeof(float)), acc);
      wait_vmcnt<0>();                 // this wave's partial stores are complete
      __syncthreads();
      if (tid == 0) s_last = atomicAdd(p.part_cnt + kXcds + x * kQueueCounters + j, 1) == S - 1;
      __syncthreads();
      write = __builtin_amdgcn_readfirstlane(s_last);
      if (write) {
        add_partial<C, true>(rp, 0, acc);
        for (int r = 1; r < S; ++r) add_partial<C, false>(rp, r * (int)(TF * sizeof(float)), acc);
      }
    }
    if (write)
      epilogue_bf16<C, EPI>(acc, p.C, p.ldc, ti.c0, ti.m_end - ti.m0, ti.n0, p.Ncols, p.C2,
                            p.ldc2);
    if (dynamic) {
      __syncthreads();                 // every thread has read s_item / s_last
      if (tid == 0) s_item = nxt;
      __syncthreads();
      it = __builtin_amdgcn_readfirstlane(s_item);
    }
  }
}

__global__ void zero_i32_kernel(int32_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

// Weight gradients: C_g = A[:, K_g] · B[:, K_g]^T for every group g, with
// K_g = [kofs[g], kofs[g+1]) (whole slabs of the tile configuration,
// possibly empty) a column range of the K-contiguous operands A [M rows,
// lda] and B [Ncols rows, ldb] (the backward pass's transposed activations,
// one padded K range per expert). C_g is [M, Ncols] at C + g * c_gstride, row-major with ldc,
// written as bf16 or fp32. Grid: (m-tiles x n-tiles, groups).
template <class C, bool F32OUT>
__global__ __launch_bounds__(kThreads, C::OCC) void kgroup_gemm_kernel(
    const bf16_t* __restrict__ A, int lda, uint32_t a_bytes, const bf16_t* __restrict__ B,
    int ldb, uint32_t b_bytes, const int32_t* __restrict__ kofs, int M, int Ncols,
    void* __restrict__ Cout, int64_t c_gstride, int ldc) {
  __shared__ __attribute__((aligned(1024))) char S0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char S1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char S2[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char S3[C::STAGES == 4 ? C::STAGE : 1024];
  const int g = blockIdx.y;
  const int nt_n = (Ncols + C::BN - 1) / C::BN;
  const int m0 = (int)(blockIdx.x / nt_n) * C::BM, n0 = (int)(blockIdx.x % nt_n) * C::BN;
  const int k_begin = __builtin_amdgcn_readfirstlane(kofs[g]);
  const int k_len = __builtin_amdgcn_readfirstlane(kofs[g + 1]) - k_begin;
  f32x16 acc[C::NB][C::FM][C::FN];
  zero_acc<C>(acc);
  if (k_len > 0) {
    uint32_t aoff[C::NAW], boff[C::NBW];
    dma_offsets<C>(aoff, boff, nullptr, 1, lda, m0, M, ldb, n0, Ncols);
    const Rsrc rA = make_rsrc(A, a_bytes), rB = make_rsrc(B, b_bytes);
    const int wm = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) / C::WN;
    const int v = min(max((M - m0 - wm * C::TM + 31) / 32, 0), C::FM);
    mainloop_rows<C, C::FM>(v, S0, S1, S2, S3, rA, aoff, rB, rB, boff, k_begin, k_len, acc);
  }
  if constexpr (F32OUT) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int lr = lane & 31, lh = lane >> 5;
    float* out = static_cast<float*>(Cout) + (int64_t)g * c_gstride;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) {
        const int col = n0 + wn * C::TN + strip_col(fn, lr);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = m0 + wm * C::TM + fm * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
          if (r < M && col < Ncols) out[(int64_t)r * ldc + col] = acc[0][fm][fn][i];
        }
      }
  } else {
    epilogue_bf16<C, EPI_STORE_BF16>(acc, static_cast<bf16_t*>(Cout) + (int64_t)g * c_gstride,
                                     ldc, m0, min(C::BM, M - m0), n0, Ncols);
  }
}

// The weight gradients of kgroup_gemm_kernel (bf16 out) on two-stage 64-deep
// tiles, persistent, one block per CU. An expert's K range is short (about
// 16 slabs at the Mixtral prefill shape), so a tile's first-slab wait and a
// block's start weigh on every tile: here the next tile's first slab goes out
// into stage S0 as soon as the main loop has freed both stages (its closing
// barrier; the epilogue stores from registers), ahead of the current tile's
// stores. Block b runs on XCD x = b % 8. With mx > 0 (P blocks, a multiple of
// 8, and at least mx m-tiles and 8 / mx n-tiles), XCD x takes, expert by
// expert, the m-tiles m = x % mx (mod mx) and the n-tiles n = x / mx
// (mod 8 / mx), m-tile major, its P / 8 blocks taking every (P / 8)-th of
// them; mx = 1 is the order of the one-tile-per-block grid whenever the
// n-tiles are a multiple of 8. Otherwise block b takes tiles b, b + P, ...
// of that grid's order (group, m-tile, n-tile). Each output tile is computed
// as in kgroup_gemm_kernel: the results are its results bit for bit.
template <class C>
__global__ __launch_bounds__(kThreads, 1) void kgroup_gemm_persist_kernel(
    const bf16_t* __restrict__ A, int lda, uint32_t a_bytes, const bf16_t* __restrict__ B,
    int ldb, uint32_t b_bytes, const int32_t* __restrict__ kofs, int G, int M, int Ncols,
    bf16_t* __restrict__ Cout, int64_t c_gstride, int ldc, int mx) {
  static_assert(C::BK == 64 && C::STAGES == 2 && !C::NN && !C::DUAL && !C::WAVE_ROWS,
                "two-stage 64-deep tiles, every A block loaded");
  __shared__ __attribute__((aligned(1024))) char S0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char S1[C::STAGE];
  const int nt_m = (M + C::BM - 1) / C::BM;
  const int nt_n = (Ncols + C::BN - 1) / C::BN;
  const int nblk = gridDim.x, b = blockIdx.x;
  const int nx = mx > 0 ? kXcds / mx : 0;
  const bool xg = mx > 0 && kXcds % mx == 0 && nblk % kXcds == 0 && nt_m >= mx && nt_n >= nx;
  // tile sequence of this block: index u = u0, u0 + du, ... < un over
  // (group, m class index, n class index)
  int xm = 0, xn = 0, sm = 1, sn = 1, cm = nt_m, cn = nt_n;
  int64_t u = b, du = nblk;
  if (xg) {
    const int x = b % kXcds;
    xm = x % mx;
    xn = x / mx;
    sm = mx;
    sn = nx;
    cm = (nt_m - xm + mx - 1) / mx;
    cn = (nt_n - xn + nx - 1) / nx;
    u = b / kXcds;
    du = nblk / kXcds;
  }
  const int per_g = cm * cn;
  const int64_t un = (int64_t)per_g * G;
  const Rsrc rA = make_rsrc(A, a_bytes), rB = make_rsrc(B, b_bytes);
  const int wm = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) / C::WN;
  struct Tile {
    int g, m0, n0, k_begin, k_len;
  };
  auto tile = [&](int64_t v) {
    Tile t;
    t.g = (int)(v / per_g);
    const int r = (int)(v - (int64_t)t.g * per_g);
    t.m0 = (xm + sm * (r / cn)) * C::BM;
    t.n0 = (xn + sn * (r % cn)) * C::BN;
    t.k_begin = __builtin_amdgcn_readfirstlane(kofs[t.g]);
    t.k_len = __builtin_amdgcn_readfirstlane(kofs[t.g + 1]) - t.k_begin;
    return t;
  };
  if (u >= un) return;
  Tile cur = tile(u);
  uint32_t aoff[C::NAW], boff[C::NBW];
  dma_offsets<C>(aoff, boff, nullptr, 1, lda, cur.m0, M, ldb, cur.n0, Ncols);
  bool pre = false;                    // the current tile's first slab is in flight
  for (;;) {
    f32x16 acc[C::NB][C::FM][C::FN];
    zero_acc<C>(acc);
    if (cur.k_len > 0) {
      const int v = min(max((M - cur.m0 - wm * C::TM + 31) / 32, 0), C::FM);
      mainloop_rows<C, C::FM>(v, S0, S1, S0, S0, rA, aoff, rB, rB, boff, cur.k_begin, cur.k_len,
                              acc, 0, 0, pre);
    }
    const int64_t un_next = u + du;
    Tile nxt = cur;
    pre = false;
    if (un_next < un) {
      nxt = tile(un_next);
      dma_offsets<C>(aoff, boff, nullptr, 1, lda, nxt.m0, M, ldb, nxt.n0, Ncols);
      if (nxt.k_len > 0) {
        dma_slab<C, -1, C::NAW>(S0, rA, aoff, rB, rB, boff, nxt.k_begin * 2, nxt.k_begin * 2);
        pre = true;
      }
    }
    epilogue_bf16<C, EPI_STORE_BF16>(acc, Cout + (int64_t)cur.g * c_gstride, ldc, cur.m0,
                                     min(C::BM, M - cur.m0), cur.n0, Ncols);
    if (un_next >= un) break;
    u = un_next;
    cur = nxt;
  }
}

// Router logits as a split-K GEMM: z_part[s][T][N] = h[:, Ks] · W_r[:, Ks]^T.
// The selection kernel sums the partial slices in a fixed order.
template <class C>
__global__ __launch_bounds__(kThreads, 1) void router_gemm_kernel(
    const bf16_t* __restrict__ h, const bf16_t* __restrict__ w, float* __restrict__ z_part,
    int T, int d, int N, int splits) {
  __shared__ __attribute__((aligned(1024))) char S0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char S1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char S2[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char S3[C::STAGES == 4 ? C::STAGE : 1024];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.x * C::BM, n0 = blockIdx.y * C::BN, s = blockIdx.z;
  // split s covers K slabs [kt*s/splits, kt*(s+1)/splits): never empty when
  // kt >= splits, so every partial slice is written
  const int kt = d / C::BK;
  const int k_begin = (kt * s / splits) * C::BK;
  const int k_len = (kt * (s + 1) / splits) * C::BK - k_begin;
  uint32_t aoff[C::NAW], boff[C::NBW];
  dma_offsets<C>(aoff, boff, nullptr, 1, d, m0, T, d, n0, N);
  const Rsrc rh = make_rsrc(h, (uint32_t)((int64_t)T * d * 2));
  const Rsrc rw = make_rsrc(w, (uint32_t)((int64_t)N * d * 2));
  f32x16 acc[C::NB][C::FM][C::FN];
  zero_acc<C>(acc);
  mainloop<C>(S0, S1, S2, S3, rh, aoff, rw, rw, boff, k_begin, k_len, acc);
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int lr = lane & 31, lh = lane >> 5;
  float* out = z_part + (int64_t)s * T * N;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const int col = n0 + wn * C::TN + strip_col(fn, lr);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = m0 + wm * C::TM + fm * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
        if (r < T && col < N) out[(int64_t)r * N + col] = acc[0][fm][fn][i];
      }
    }
}

// ------------------------------------------------------- decode (skinny)
// Block b runs on XCD b % 8. Normally block b takes group b mod G and
// column block b / G, so XCD x streams the weights of groups x, x + 8, ...
// With at most 64 groups of which at most six hold rows (a few tokens),
// that order leaves XCDs idle; then the work items (used group, column
// block), group-major, are cut into eight contiguous ranges, XCD x taking
// the x-th (one token: 0.330 -> 0.163 ms per step, four tokens 0.419 ->
// 0.392 ms). With seven used groups of eight that measured 5% slower than
// leaving one XCD idle, and spreading an XCD's blocks over many groups
// (consecutive blocks taking different used groups, or consecutive column
// blocks of one group) 6-12% slower. Surplus blocks of the launch (sized
// for all groups) return at once. Rows of group g (at most 16·MT), 16·CT
// output columns (of gate and up when DUAL), the four waves split K into
// 64-wide chunks (chunk c goes to wave c % 4). Lane (i = l % 16, q = l / 16)
// loads 32 contiguous bytes of weight row i at k = 64c + 16q, so each group
// of four lanes reads one full 128-byte line; the A fragments use the same
// k mapping.
template <int MT, int CT, bool DUAL, bool CMB, int PD>
__device__ __forceinline__ void skinny_tile(const GroupedProblem& p, int g, int cb, int r0,
                                            int cnt,
                                            f32x4 (&red)[4][(DUAL ? 2 : 1) * MT * CT][64]) {
  constexpr int NB = DUAL ? 2 : 1;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, lq = lane >> 4;
  const int n0 = cb * 16 * CT;

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
  auto loadA = [&](u32x4 (&dst)[MT][2], int c) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int s = 0; s < 2; ++s)
        dst[mt][s] = aval[mt] ? *reinterpret_cast<const u32x4*>(arow[mt] + c * 64 + s * 8) : zero4;
  };
  auto chunk_mfma = [&](const u32x4 (&a)[MT][2], const u32x4 (&b)[NB][CT][2]) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
            acc[nb][mt][ct] = mfma_16x16x32(a[mt][s], b[nb][ct][s], acc[nb][mt][ct]);
  };
  if constexpr (PD == 1) {
    // A and B of chunk c + 4 are loaded together, one chunk ahead of the
    // MFMAs: loads complete in issue order, so the MFMAs' wait for chunk c
    // leaves all of chunk c + 4 in flight
    u32x4 bc[NB][CT][2], bn[NB][CT][2];
    u32x4 ac[MT][2], an[MT][2];
    int c = w;
    if (c < KT) {
      loadB(bc, c);
      loadA(ac, c);
    }
    for (; c < KT; c += 4) {
      if (c + 4 < KT) {
        loadB(bn, c + 4);
        loadA(an, c + 4);
      }
      chunk_mfma(ac, bc);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int s = 0; s < 2; ++s) bc[nb][ct][s] = bn[nb][ct][s];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int s = 0; s < 2; ++s) ac[mt][s] = an[mt][s];
    }
  } else {
    // a ring of PD + 1 register sets: while a wave computes chunk c, chunks
    // c + 4, ..., c + 4 PD are in flight. The loop is unrolled over the ring,
    // so every slot is a fixed register set (copying from a slot whose loads
    // are in flight would wait for them), at the cost of more live
    // registers; used for 16-column blocks, whose chunks are small.
    u32x4 bq[PD + 1][NB][CT][2];
    u32x4 aq[PD + 1][MT][2];
#pragma unroll
    for (int j = 0; j < PD; ++j) {
      const int cj = w + 4 * j;
      if (cj < KT) {
        loadB(bq[j], cj);
        loadA(aq[j], cj);
      }
    }
    for (int c0 = w; c0 < KT; c0 += 4 * (PD + 1)) {
#pragma unroll
      for (int j = 0; j <= PD; ++j) {
        const int c = c0 + 4 * j;
        if (c < KT) {
          const int cl = c + 4 * PD;
          if (cl < KT) {
            loadB(bq[(j + PD) % (PD + 1)], cl);
            loadA(aq[(j + PD) % (PD + 1)], cl);
          }
          chunk_mfma(aq[j], bq[j]);
        }
      }
    }
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
  __shared__ __attribute__((aligned(16))) bf16_t s_out[CMB ? 16 * MT : 1][16 * CT];
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
        if constexpr (CMB)
          s_out[m][ct * 16 + li] = (bf16_t)f32_to_bf16(v);
        else
          Cout[(p.c_row0 + r0 + m) * (int64_t)p.ldc + col] = (bf16_t)f32_to_bf16(v);
      }
    }
  }
  if constexpr (CMB) {
    // 16-byte agent-coherent stores of the tile's rows (byte offsets below
    // 2^31: checked by the launcher)
    __syncthreads();
    constexpr int CPR = 2 * CT;                  // 8-column chunks per row
    const Rsrc rc = make_rsrc(Cout, 0x7fffffffu);
    for (int i = tid; i < cnt * CPR; i += kThreads) {
      const int m = i / CPR, ch = i % CPR;
      const int col = n0 + ch * 8;
      if (col < p.Ncols) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(&s_out[m][ch * 8]);
        const int64_t off = ((p.c_row0 + r0 + m) * (int64_t)p.ldc + col) * 2;
        __builtin_amdgcn_raw_buffer_store_b128(v, rc, (uint32_t)off, 0, kSc1);
      }
    }
  }
}

// The combine of one column range [n0, n0 + 16 CT) by the last block of the
// range to arrive; rows are read with agent-coherent loads.
template <int CT>
__device__ __forceinline__ void skinny_combine(const GroupedProblem& p, const CombineFuse& cf,
                                               int cb, int ngroups) {
  __shared__ int s_last;
  const int tid = threadIdx.x;
  wait_vmcnt<0>();                    // this wave's row stores are complete
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(cf.cnt + cb, 1) == ngroups - 1;
  __syncthreads();
  if (!__builtin_amdgcn_readfirstlane(s_last)) return;
  constexpr int CPR = 2 * CT;
  const int n0 = cb * 16 * CT;
  const int64_t R = (int64_t)cf.T * cf.k;
  const Rsrc rc = make_rsrc(p.C, 0x7fffffffu);
  bf16_t* __restrict__ y = static_cast<bf16_t*>(cf.y);
  for (int i = tid; i < cf.T * CPR; i += kThreads) {
    const int t = i / CPR, col = n0 + (i % CPR) * 8;
    if (col >= p.Ncols) continue;
    float acc[8];
    if (cf.has_shared) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(
          rc, (uint32_t)(((R + t) * p.ldc + col) * 2), 0, kSc1);
      unpack_bf16x8(v, acc);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
    }
    for (int j = 0; j < cf.k; ++j) {
      const int64_t r = cf.row_of[(int64_t)t * cf.k + j];
      if (r < 0) continue;
      const float gt = cf.gates[(int64_t)t * cf.k + j];
      float v[8];
      unpack_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(rc, (uint32_t)((r * p.ldc + col) * 2),
                                                          0, kSc1),
                    v);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(gt, v[e], acc[e]);
    }
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(acc[2 * e], acc[2 * e + 1]);
    *reinterpret_cast<u32x4*>(y + (int64_t)t * p.Ncols + col) = o;
  }
}

// CMB (down GEMM with the combine fused): rows are written with
// agent-coherent stores, then every block of a column range bumps that
// range's arrival counter (the blocks of experts without rows too); the
// last to arrive sums each token's rows over those columns into y, with the
// separate combine kernel's arithmetic and order (same bits).
template <int MT, int CT, bool DUAL, bool CMB, int PD>
__global__ __launch_bounds__(kThreads) void skinny_gemm_kernel(GroupedProblem p, CombineFuse cf) {
  constexpr int NB = DUAL ? 2 : 1;
  constexpr int NACC = NB * MT * CT;
  __shared__ f32x4 red[4][NACC][64];
  // one-dimensional grid of 8·⌈G·ncb / 8⌉ blocks
  const int G = p.offsets ? p.groups : (p.M + 16 * MT - 1) / (16 * MT);
  const int ncb = (p.Ncols + 16 * CT - 1) / (16 * CT);
  uint64_t m = 0;
  int ngroups = G;
  if (p.offsets && G <= 64) {
    const int lane = threadIdx.x & 63;
    const bool used = lane < G && p.offsets[lane + 1] > p.offsets[lane];
    m = __ballot(used);
    // no group with rows: group 0 stands in (no rows; the combine still runs)
    if (m == 0) m = 1;
    ngroups = __popcll(m);
  }
  int g, cb;
  if (m && ngroups <= 6) {
    const int64_t items = (int64_t)ngroups * ncb;
    const int64_t per = (items + kXcds - 1) / kXcds;      // items per XCD
    const int64_t j = blockIdx.x / kXcds;
    const int64_t item = (int64_t)(blockIdx.x % kXcds) * per + j;
    if (j >= per || item >= items) return;
    const int a = (int)(item / ncb);
    cb = (int)(item % ncb);
    for (int i = 0; i < a; ++i) m &= m - 1;
    g = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)m) - 1);
  } else {
    ngroups = G;
    g = (int)(blockIdx.x % G);
    cb = (int)(blockIdx.x / G);
    if (cb >= ncb) return;
  }
  int r0, cnt;
  if (p.offsets) {
    r0 = p.offsets[g];
    cnt = p.offsets[g + 1] - r0;
  } else {
    r0 = g * 16 * MT;
    cnt = min(p.M - r0, 16 * MT);
  }
  // at most 16·MT rows per pass; more only when a caller's ids name one
  // expert twice for a token (the row bound of the launch assumes not)
  for (int base = 0; base < cnt; base += 16 * MT) {
    if (base > 0) __syncthreads();          // the previous pass's LDS reads are done
    skinny_tile<MT, CT, DUAL, CMB, PD>(p, g, cb, r0 + base, min(cnt - base, 16 * MT), red);
  }
  if constexpr (CMB) skinny_combine<CT>(p, cf, cb, ngroups);
}

// PD chunks in flight per wave: 3 for 16-column blocks (a wave's chunk is
// 2 or 4 KB of weights, and one token's down GEMM has two blocks per CU),
// else 1.
template <int MT, int CT, bool DUAL, bool CMB>
hipError_t launch_skinny_ct(const GroupedProblem& p, hipStream_t st, const CombineFuse& cf) {
  const int G = p.offsets ? p.groups : (p.M + 16 * MT - 1) / (16 * MT);
  if (G == 0) return hipSuccess;
  const int64_t items = (int64_t)G * ((p.Ncols + 16 * CT - 1) / (16 * CT));
  const dim3 grid((unsigned)((items + kXcds - 1) / kXcds * kXcds));
  constexpr int PD = CT == 1 ? 3 : 1;
  hipLaunchKernelGGL((skinny_gemm_kernel<MT, CT, DUAL, CMB, PD>), grid, dim3(kThreads), 0, st, p,
                     cf);
  return hipGetLastError();
}

// 64 columns per block (CT = 4): the block's activation rows are read once
// per 64 columns (narrower blocks for 33-64 rows made those L2 reads
// outweigh the weights: at T = 64, 0.659 against 0.518 ms per step). At
// most 16 rows per expert and fewer work items than two per CU (the
// experts that can hold rows, at most min(groups, rows), times the column
// blocks), narrower blocks, so that every CU streams weights: one token
// touches two experts, and 64-column blocks gave its down GEMM 128 blocks
// for 256 CUs. 32 columns when that gives at least four items per CU, else
// 16 (one token's gate/up: 1,792 items, seven per CU, instead of 3.5 rounds
// of 32-column items; the step 0.154 -> 0.148 ms).
template <int MT, bool DUAL, bool CMB = false>
hipError_t launch_skinny(const GroupedProblem& p, int num_cu, hipStream_t st,
                         const CombineFuse& cf = CombineFuse{}) {
  if constexpr (MT == 1) {
    const int64_t used = p.offsets ? std::min<int64_t>(p.groups, p.M) : (p.M + 15) / 16;
    auto items = [&](int ct) { return used * ((p.Ncols + 16 * ct - 1) / (16 * ct)); };
    if (items(4) < 2 * (int64_t)num_cu)
      return items(2) >= 4 * (int64_t)num_cu ? launch_skinny_ct<1, 2, DUAL, CMB>(p, st, cf)
                                             : launch_skinny_ct<1, 1, DUAL, CMB>(p, st, cf);
  }
  return launch_skinny_ct<MT, 4, DUAL, CMB>(p, st, cf);
}

template <bool DUAL, bool CMB = false>
hipError_t launch_skinny_any(const GroupedProblem& p, int num_cu, hipStream_t st,
                             const CombineFuse& cf = CombineFuse{}) {
  if (p.max_rows <= 16) return launch_skinny<1, DUAL, CMB>(p, num_cu, st, cf);
  if (p.max_rows <= 32) return launch_skinny<2, DUAL, CMB>(p, num_cu, st, cf);
  return launch_skinny<4, DUAL, CMB>(p, num_cu, st, cf);
}

template <class C, int EPI>
hipError_t launch_grouped(const GroupedProblem& p, int num_cu, hipStream_t st) {
  // Upper bound on tiles, to avoid idle blocks on tiny problems.
  const int G = p.offsets ? p.groups : 1;
  const int64_t xr = p.X0 ? p.x_rows : 0;
  const int64_t mt_bound = ((int64_t)p.M + xr + C::BM - 1) / C::BM + (p.offsets ? G : 0) +
                           (p.X0 ? 1 : 0);
  const int64_t tiles = mt_bound * ((p.Ncols + C::BN - 1) / C::BN);
  // with a split-K workspace, small problems may use more blocks than tiles
  const int64_t units = p.part ? tiles * kMaxSplit : tiles;
  int nblk = num_cu * C::OCC;
  if (units < nblk) nblk = (int)units;
  if (nblk >= kXcds) nblk -= nblk % kXcds;
  if (nblk <= 0) return hipSuccess;
  if (p.part) {
    hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(kThreads), 0, st, p.part_cnt, kSplitCounters);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((grouped_gemm_kernel<C, EPI>), dim3(nblk), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace

// Tile configurations of the prefill kernels.
using GateUp256 = TileCfg<256, 128, true, 4, 1>;    // 256 rows, 1 block per CU
using GateUp128 = TileCfg<128, 128, true, 3, 2>;    // 128 rows, 2 blocks per CU
using Down128 = TileCfg<128, 256, false, 3, 2>;
using Down256 = TileCfg<256, 256, false, 4, 1>;
using Router = TileCfg<128, 128, false, 4, 1>;
using Down128NN = TileCfg<128, 256, false, 3, 2, true>;
using Down256NN = TileCfg<256, 256, false, 4, 1, true>;
// the 256-row tiles on 64-deep slabs (two 64 KB stages)
using GateUp256K = TileCfg<256, 128, true, 2, 1, false, 64>;
using Down256K = TileCfg<256, 256, false, 2, 1, false, 64>;
// few rows per expert: 128-row tiles, 64-deep slabs, three stages (144 KB)
using GateUpMid = TileCfg<128, 128, true, 3, 1, false, 64>;
using DownMid = TileCfg<128, 256, false, 3, 1, false, 64>;

// Rows per expert at most 64: weight streaming. Otherwise 256-row tiles (one
// block per CU) when experts average at least 1024 rows or the 256-row tile
// list still gives every CU about four tiles, else 128-row tiles (two blocks
// per CU). A 256-row tile reads an expert's weight columns once for up to 256
// of its rows, where 128-row tiles read them once per 128 rows and rely on L2
// to share the rest; padding rows cost no loads and their MFMAs are skipped.
// Rows and groups of a launch, its extra group included.
static int64_t all_rows(const GroupedProblem& p) { return (int64_t)p.M + (p.X0 ? p.x_rows : 0); }
static int64_t all_groups(const GroupedProblem& p) {
  return (p.offsets ? p.groups : 1) + (p.X0 ? 1 : 0);
}

static bool tall_tiles(const GroupedProblem& p, int bn, int num_cu) {
  const int64_t G = all_groups(p), M = all_rows(p);
  if (M >= 1024 * G) return true;
  const int64_t nt = (p.Ncols + bn - 1) / bn;
  const int64_t est = (M / 256 + G / 2) * nt;   // 256-row tiles, about
  return est >= 4 * (int64_t)num_cu;
}

// 64-deep slabs for the 256-row tiles whenever K allows: whole 128-byte
// lines per row and slab, half the load requests of 32-deep slabs for the
// same bytes. Measured 1-2% faster on the Mixtral- and Qwen3-30B-shaped
// layers, the same on the DeepSeek-V3 shape (every shape runs at or near
// the board's power limit, so fewer requests buy a little clock).
static bool k64_tiles(const GroupedProblem& p) { return p.K % 64 == 0; }

// Fewer than 768 rows per expert on average: many tiles hold few rows and
// stream their expert's weight columns from HBM at every slab. 128-row tiles
// with three 64-deep stages keep two slabs in flight per CU instead of one
// (DeepSeek-V3 shape, 128 rows per expert: gate/up 3.90 -> 3.40 ms; the
// Qwen3-30B shape, 512 Zipf-skewed: 3% faster; the Mixtral shape, 1,024:
// 5% slower, so it keeps the 256-row tiles).
static bool mid_tiles(const GroupedProblem& p) {
  return p.K % 64 == 0 && all_rows(p) < 768 * all_groups(p);
}

// The extra group (X0) runs in the launch of the other groups, on their
// tiles, unless those take the weight-streaming kernels (at most 64 rows per
// group; skinny = true) or there is no room for one more group: then it runs
// after them as a launch of its own.
static GroupedProblem without_extra(const GroupedProblem& p) {
  GroupedProblem q = p;
  q.X0 = q.X1 = nullptr;
  q.x_rows = 0;
  return q;
}
static GroupedProblem extra_alone(const GroupedProblem& p) {
  GroupedProblem q = without_extra(p);
  const int64_t skip = p.x_a_row0 * p.lda * 2;
  q.A = static_cast<const char*>(p.A) + skip;
  q.a_bytes = (uint32_t)(p.a_bytes - skip);
  q.perm = nullptr;
  q.kdiv = 1;
  q.offsets = nullptr;
  q.groups = 1;
  q.M = q.max_rows = p.x_rows;
  q.B0 = p.X0;
  q.B1 = p.X1;
  q.b_gstride = 0;
  q.c_row0 = p.x_c_row0;
  return q;
}
template <class F>
static hipError_t with_extra(const GroupedProblem& p, bool skinny, F launch) {
  if (!p.X0 || (!skinny && (p.offsets ? p.groups : 1) < kMaxGroups)) return launch(p);
  const hipError_t e = launch(without_extra(p));
  if (e != hipSuccess || p.x_rows == 0) return e;
  return launch(extra_alone(p));
}

hipError_t launch_gateup_bf16(const GroupedProblem& p_, int num_cu, hipStream_t st) {
  if (p_.C2) {
    // keeping the pre-activations: the grouped tiles at any row count, the
    // same tiles and schedule as the backward's recompute
    return with_extra(p_, false, [&](const GroupedProblem& p) {
      if (mid_tiles(p)) return launch_grouped<GateUpMid, EPI_SWIGLU_SAVE>(p, num_cu, st);
      if (tall_tiles(p, GateUp256::BN, num_cu))
        return k64_tiles(p) ? launch_grouped<GateUp256K, EPI_SWIGLU_SAVE>(p, num_cu, st)
                            : launch_grouped<GateUp256, EPI_SWIGLU_SAVE>(p, num_cu, st);
      return launch_grouped<GateUp128, EPI_SWIGLU_SAVE>(p, num_cu, st);
    });
  }
  return with_extra(p_, p_.max_rows <= 64, [&](const GroupedProblem& p) {
    if (p.max_rows <= 64) return launch_skinny_any<true>(p, num_cu, st);
    if (mid_tiles(p)) return launch_grouped<GateUpMid, EPI_SWIGLU>(p, num_cu, st);
    if (tall_tiles(p, GateUp256::BN, num_cu))
      return k64_tiles(p) ? launch_grouped<GateUp256K, EPI_SWIGLU>(p, num_cu, st)
                          : launch_grouped<GateUp256, EPI_SWIGLU>(p, num_cu, st);
    return launch_grouped<GateUp128, EPI_SWIGLU>(p, num_cu, st);
  });
}

int combine_counters(int d) { return (d + 15) / 16; }

bool down_combine_ok(const GroupedProblem& p, const CombineFuse& cf) {
  const int64_t rows = (int64_t)cf.T * cf.k + (cf.has_shared ? cf.T : 0);
  return p.max_rows <= 64 && p.offsets && p.c_row0 == 0 && p.ldc == p.Ncols &&
         p.Ncols % 8 == 0 && rows * p.ldc * 2 <= 0x7fffffffLL;
}

hipError_t launch_down_combine_bf16(const GroupedProblem& p, const CombineFuse& cf, int num_cu,
                                    hipStream_t st) {
  if (!down_combine_ok(p, cf)) return hipErrorNotSupported;
  return launch_skinny_any<false, true>(p, num_cu, st, cf);
}

hipError_t launch_down_bf16(const GroupedProblem& p_, int num_cu, hipStream_t st) {
  return with_extra(p_, p_.max_rows <= 64, [&](const GroupedProblem& p) {
    if (p.max_rows <= 64) return launch_skinny_any<false>(p, num_cu, st);
    if (mid_tiles(p)) return launch_grouped<DownMid, EPI_STORE_BF16>(p, num_cu, st);
    if (tall_tiles(p, Down256::BN, num_cu))
      return k64_tiles(p) ? launch_grouped<Down256K, EPI_STORE_BF16>(p, num_cu, st)
                          : launch_grouped<Down256, EPI_STORE_BF16>(p, num_cu, st);
    return launch_grouped<Down128, EPI_STORE_BF16>(p, num_cu, st);
  });
}

// NN (B as [K rows][N columns]): the grouped tiles at more than 64 rows per
// group; at most 64 the weight-streaming kernels need K-contiguous weights
bool down_nn_ok(const GroupedProblem& p) {
  const int k1 = p.b_k1 > 0 ? p.b_k1 : p.K;
  return p.max_rows > 64 && p.Ncols % 8 == 0 && p.ldb % 8 == 0 && p.K % 32 == 0 &&
         k1 % 32 == 0 && (int64_t)(k1 > p.K - k1 ? k1 : p.K - k1) * p.ldb * 2 <= 0x7fffffffLL;
}

template <int EPI>
static hipError_t launch_down_nn(const GroupedProblem& p, int num_cu, hipStream_t st) {
  if (!down_nn_ok(p)) return hipErrorNotSupported;
  if (tall_tiles(p, Down256NN::BN, num_cu)) return launch_grouped<Down256NN, EPI>(p, num_cu, st);
  return launch_grouped<Down128NN, EPI>(p, num_cu, st);
}

hipError_t launch_down_nn_bf16(const GroupedProblem& p, int num_cu, hipStream_t st) {
  return launch_down_nn<EPI_STORE_BF16>(p, num_cu, st);
}

hipError_t launch_down_nn_f32out_bf16(const GroupedProblem& p, int num_cu, hipStream_t st) {
  return launch_down_nn<EPI_STORE_F32>(p, num_cu, st);
}

// Gate and up pre-activations of the routed rows as fp32, side by side in C
// (ldc = 2 Ncols): the same tiles and schedule as the SwiGLU launch, any row
// count.
hipError_t launch_gateup_preact_bf16(const GroupedProblem& p_, int num_cu, hipStream_t st) {
  return with_extra(p_, false, [&](const GroupedProblem& p) {
    if (mid_tiles(p)) return launch_grouped<GateUpMid, EPI_STORE_DUAL_F32>(p, num_cu, st);
    if (tall_tiles(p, GateUp256::BN, num_cu))
      return k64_tiles(p) ? launch_grouped<GateUp256K, EPI_STORE_DUAL_F32>(p, num_cu, st)
                          : launch_grouped<GateUp256, EPI_STORE_DUAL_F32>(p, num_cu, st);
    return launch_grouped<GateUp128, EPI_STORE_DUAL_F32>(p, num_cu, st);
  });
}

// C = A·B0^T stored as fp32, any row count (the grouped tiles only).
hipError_t launch_down_f32out_bf16(const GroupedProblem& p, int num_cu, hipStream_t st) {
  if (tall_tiles(p, Down256::BN, num_cu))
    return launch_grouped<Down256, EPI_STORE_F32>(p, num_cu, st);
  return launch_grouped<Down128, EPI_STORE_F32>(p, num_cu, st);
}

hipError_t launch_kgroup_bf16(const void* A_, int lda, int64_t a_rows, const void* B_, int ldb,
                              int64_t b_rows, const int32_t* kofs, int groups, int M, int Ncols,
                              void* C, int64_t c_gstride, int ldc, bool f32out, int num_cu,
                              hipStream_t st) {
  if (groups == 0 || M == 0 || Ncols == 0) return hipSuccess;
  const bf16_t* A = static_cast<const bf16_t*>(A_);
  const bf16_t* B = static_cast<const bf16_t*>(B_);
  const uint32_t ab = (uint32_t)(a_rows * lda * 2), bb = (uint32_t)(b_rows * ldb * 2);
  if (f32out) {
    using K = Router;
    dim3 grid((unsigned)(((M + K::BM - 1) / K::BM) * ((Ncols + K::BN - 1) / K::BN)), groups);
    hipLaunchKernelGGL((kgroup_gemm_kernel<K, true>), grid, dim3(kThreads), 0, st, A, lda, ab, B,
                       ldb, bb, kofs, M, Ncols, C, c_gstride, ldc);
  } else if (M >= 512) {
    // 256 x 256 tiles: half the operand traffic per flop of 128 x 256; the
    // K ranges are whole 64-deep slabs. Persistent, one block per CU.
    using K = Down256K;
    const int64_t tiles =
        (int64_t)((M + K::BM - 1) / K::BM) * ((Ncols + K::BN - 1) / K::BN) * groups;
    int64_t nblk = std::min<int64_t>(tiles, num_cu > 0 ? num_cu : 256);
    if (nblk >= kXcds) nblk -= nblk % kXcds;
    // 2 m-tile classes x 4 n-tile classes over the XCDs: measured faster
    // than the grid's own order (1 x 8), 4 x 2 and 8 x 1 at the Mixtral
    // prefill shape, for all three weight gradients alike
    const int mx = 2;
    hipLaunchKernelGGL((kgroup_gemm_persist_kernel<K>), dim3((unsigned)nblk), dim3(kThreads), 0,
                       st, A, lda, ab, B, ldb, bb, kofs, groups, M, Ncols,
                       static_cast<bf16_t*>(C), c_gstride, ldc, mx);
  } else {
    using K = Down128;
    dim3 grid((unsigned)(((M + K::BM - 1) / K::BM) * ((Ncols + K::BN - 1) / K::BN)), groups);
    hipLaunchKernelGGL((kgroup_gemm_kernel<K, false>), grid, dim3(kThreads), 0, st, A, lda, ab, B,
                       ldb, bb, kofs, M, Ncols, C, c_gstride, ldc);
  }
  return hipGetLastError();
}

int64_t split_part_floats(int64_t M, int G, int Ncols, bool dual) {
  // kMaxSplit partial tiles per tile at most (tiles of up to 256 rows and
  // 256 columns); the cap covers one 256 KiB partial per block of a launch
  // on 256 CUs
  const int64_t cols = ((int64_t)Ncols + 255) / 256 * 256;
  const int64_t f = (M + (int64_t)G * 256) * cols * (dual ? 2 : 1) * kMaxSplit;
  return f < kSplitMaxFloats ? f : kSplitMaxFloats;
}

// Split-K factor of the router GEMM: enough blocks to fill about 256 CUs,
// at least four K steps per split, at most kRouterMaxSplits. It depends on
// the shape only, so results do not depend on the device.
int router_splits(int T, int d, int N) {
  using C = Router;
  const int64_t tiles = (int64_t)((T + C::BM - 1) / C::BM) * ((N + C::BN - 1) / C::BN);
  int s = 1;
  while (s < kRouterMaxSplits && tiles * s * 2 <= 256 && (d / 64) >= s * 2 * 4) s *= 2;
  return s;
}

hipError_t launch_router_gemm_bf16(const void* h, const void* w, float* z_part, int T, int d,
                                   int N, int splits, hipStream_t st) {
  using C = Router;
  dim3 grid((T + C::BM - 1) / C::BM, (N + C::BN - 1) / C::BN, splits);
  hipLaunchKernelGGL((router_gemm_kernel<C>), grid, dim3(kThreads), 0, st,
                     static_cast<const bf16_t*>(h), static_cast<const bf16_t*>(w), z_part, T, d,
                     N, splits);
  return hipGetLastError();
}

}  // namespace moe
