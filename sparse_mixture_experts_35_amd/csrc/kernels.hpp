// Host-side launchers of the MoE HIP kernels (one translation unit each).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------- routing
constexpr int kRouterMaxSplits = 8;
// Split-K partial logits z_part[s][T][N] (fp32) = h[:, K_s] · w_router[:, K_s]^T,
// s < router_splits(T, d, N) (bf16), or one slice with the fp32 kernel.
int router_splits(int T, int d, int N);
hipError_t launch_router_gemm_bf16(const void* h, const void* w_router,
                                   float* z_part, int T, int d, int N,
                                   int splits, hipStream_t st);
hipError_t launch_router_logits_f32(const float* h, const float* w_router,
                                    float* z, int T, int d, int N,
                                    hipStream_t st);
// Group-limited candidates: n_groups contiguous groups (0 = no limit), the
// keep best by the sum of their topm largest selection scores.
struct GroupLimit {
  int n_groups, keep, topm;
};
// z = sum of the partial slices + b_router; scores, top-k, gates, and
// per-block sums of the routing probabilities
int route_select_blocks(int T, int N);
// (zl_part, when given: per-block sums of the squared log-sum-exp of the
// logits and of the routing entropy, 2 floats per block)
// Final statistics written by the selection kernel itself when it runs as
// a single block (on = request; the launcher clears it otherwise): sum / T,
// which equals the reduction kernel's result bit for bit.
struct RouteFinal {
  float* p_mean;
  float* z_loss;
  float* entropy;
  int on;
};
// Outputs of the dispatch when the selection kernel also dispatches (see
// launch_dispatch; p_mean is fin.p_mean)
struct DispatchOut {
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm_src;
  int32_t* row_of;
  float* f_out;
  float* l_aux;
  float alpha;
  int cap;
  float* cap_stats;
  int32_t* zero;
  int zero_n;
};
// dq != NULL: one block selects and then dispatches (T fits one selection
// block and T·k one dispatch chunk, else hipErrorInvalidValue)
hipError_t launch_route_select(const float* z_part, int splits,
                               const float* b_router, const float* b_select,
                               int32_t* ids, float* gates, float* p_part,
                               float* zl_part, int T, int N, int k, int mode,
                               GroupLimit gl, RouteFinal fin, hipStream_t st,
                               const DispatchOut* dq = nullptr);
// small T·N: router logits by a GEMV kernel (one slice, splits = 1)
bool router_use_gemv(int T, int N);
hipError_t launch_router_gemv_bf16(const void* h, const void* w, float* z,
                                   int T, int d, int N, hipStream_t st);
// p_mean (nullable) from p_part; z_loss / entropy (nullable) from zl_part
hipError_t launch_p_reduce(const float* p_part, float* p_mean,
                           const float* zl_part, float* z_loss, float* entropy,
                           int blocks, int T, int N, hipStream_t st);

// --------------------------------------------------------------- dispatch
// cap: expert capacity C >= 1, or 0 for none; cap_stats nullable; hist:
// dispatch_hist_ints(T, k, N) int32 of scratch, 16-byte aligned (per-chunk
// expert counts); zero_n int32 at zero are cleared (counters of a later
// kernel)
int dispatch_chunks(int T, int k);
int64_t dispatch_hist_ints(int T, int k, int N);
hipError_t launch_dispatch(const int32_t* ids, int T, int k, int N,
                           int32_t* counts, int32_t* offsets,
                           int32_t* perm_src, int32_t* row_of,
                           const float* p_mean, float* f_out, float* l_aux,
                           float alpha, int cap, float* cap_stats,
                           int32_t* hist, hipStream_t st,
                           int32_t* zero = nullptr, int zero_n = 0);

// ---------------------------------------------------------------- experts
// One grouped problem: rows of A gathered through perm (token = perm[r] /
// kdiv, or r when perm is NULL), groups given by offsets (NULL: one group
// of M rows), B rows of group g at B + g*b_gstride.
struct GroupedProblem {
  const void* A;
  int lda;
  const int32_t* perm;
  int kdiv;
  const int32_t* offsets;
  int groups;
  int M;          // rows when offsets == NULL; upper bound of rows otherwise
  int max_rows;   // upper bound on the rows of any one group
  const void* B0;
  const void* B1;  // up projection (gate/up GEMM only)
  int64_t b_gstride;
  int ldb;
  int Ncols;
  int K;
  void* C;
  int ldc;
  int64_t c_row0;
  uint32_t a_bytes;  // extent of A in bytes (rows of A times lda times element size)
  // Work queues and split-K of the last, partial round of tiles (bf16
  // prefill kernels; NULL: static schedule, no split). part holds
  // part_floats fp32 partial sums, part_cnt kSplitCounters queue heads and
  // arrival counters, zeroed by the launcher before every launch.
  float* part;
  int32_t* part_cnt;
  int64_t part_floats;
  // gate/up GEMM only, nullable: also store the fp32 gate and up
  // pre-activations of each row at C2 + (c_row0 + r) * ldc2, gate in columns
  // [0, Ncols), up in [Ncols, 2 Ncols) (kept for the backward pass)
  float* C2;
  int64_t ldc2;
  // B given as [K rows][ldb] (N contiguous; the down-type NN launchers
  // only): rows [0, b_k1) at B0, rows [b_k1, K) at B1 (b_k1 = 0: all at B0)
  int b_k1;
  // One more group after the offsets' groups, nullable (the grouped bf16
  // gate/up and down launchers only): x_rows rows with weights X0 (and X1,
  // gate/up) of the same shape as one expert's, A rows x_a_row0 + r read in
  // order (no perm), output rows x_c_row0 + r (in C, and C2 when given).
  // The shared expert runs as this group in the routed experts' launch.
  const void* X0;
  const void* X1;
  int x_rows;
  int64_t x_a_row0;
  int64_t x_c_row0;
};

constexpr int kSplitCounters = 1024;
constexpr int64_t kSplitMaxFloats = int64_t(16) << 20;   // 64 MiB of partials
// fp32 partial-sum capacity for the split-K tail of a grouped launch over
// at most M rows in G groups and Ncols output columns (gate and up both
// when dual), capped at kSplitMaxFloats. The kernel never uses more than it
// is given: it lowers the split count to fit.
int64_t split_part_floats(int64_t M, int G, int Ncols, bool dual);

// Act = SiLU(A·B0^T) ⊙ (A·B1^T)   (bf16 in/out, fp32 accumulate)
hipError_t launch_gateup_bf16(const GroupedProblem& p, int num_cu,
                              hipStream_t st);
// C = A·B0^T                        (bf16 in/out, fp32 accumulate)
hipError_t launch_down_bf16(const GroupedProblem& p, int num_cu,
                            hipStream_t st);
// Combine fused into the weight-streaming down GEMM (at most 64 rows per
// expert): y[t] = (shared row) + sum_j gates[t k + j] rows[row_of[t k + j]],
// rows being the GEMM's own output C (c_row0 0, ldc = Ncols = d; the shared
// expert's rows [T k, T k + T) written before the launch). cnt:
// combine_counters(d) int32, zero at launch.
struct CombineFuse {
  const int32_t* row_of;
  const float* gates;
  void* y;
  int T, k;
  int has_shared;
  int32_t* cnt;
};
int combine_counters(int d);
bool down_combine_ok(const GroupedProblem& p, const CombineFuse& cf);
// hipErrorNotSupported unless down_combine_ok
hipError_t launch_down_combine_bf16(const GroupedProblem& p, const CombineFuse& cf, int num_cu,
                                    hipStream_t st);
// gate and up pre-activations side by side as fp32: C [rows, 2 Ncols] float,
// ldc = 2 Ncols
hipError_t launch_gateup_preact_bf16(const GroupedProblem& p, int num_cu,
                                     hipStream_t st);
// C = A·B0^T (bf16 in, fp32 out)
hipError_t launch_down_f32out_bf16(const GroupedProblem& p, int num_cu,
                                   hipStream_t st);
// C = A·B with B given as [K rows][ldb] (the weights' own layout; rows past
// b_k1 from B1), bf16 or fp32 out; hipErrorNotSupported unless down_nn_ok
// (more than 64 rows per group, sizes multiples of 8 / 32)
bool down_nn_ok(const GroupedProblem& p);
hipError_t launch_down_nn_bf16(const GroupedProblem& p, int num_cu, hipStream_t st);
hipError_t launch_down_nn_f32out_bf16(const GroupedProblem& p, int num_cu, hipStream_t st);
// C_g = A[:, kofs[g]:kofs[g+1]] · B[:, kofs[g]:kofs[g+1]]^T for g < groups
// (A [a_rows, lda] and B [b_rows, ldb] bf16, K ranges multiples of 64);
// C_g [M, Ncols] at C + g * c_gstride elements, bf16 or fp32 (f32out);
// num_cu sizes the persistent grid of the 256 x 256 tiles
hipError_t launch_kgroup_bf16(const void* A, int lda, int64_t a_rows,
                              const void* B, int ldb, int64_t b_rows,
                              const int32_t* kofs, int groups, int M, int Ncols,
                              void* C, int64_t c_gstride, int ldc, bool f32out, int num_cu,
                              hipStream_t st);
// fp32 versions (plain FMA kernels)
hipError_t launch_gateup_f32(const GroupedProblem& p, hipStream_t st);
hipError_t launch_down_f32(const GroupedProblem& p, hipStream_t st);

hipError_t launch_gateup_preact_f32(const GroupedProblem& p, hipStream_t st);

// ---------------------------------------------------------------- backward
// Padded K ranges: kofs[e] = sum over e' < e of round64(kept rows of e'),
// kofs[G] the total; offsets NULL: kofs = {0, round64(n_single)}.
hipError_t launch_kofs(const int32_t* offsets, int G, int n_single,
                       int32_t* kofs, hipStream_t st);
// dst[c][kofs[e] + i] = scale * src[row][c] for the i-th kept row of expert
// e (row = perm[r] / kdiv or r; scale from scale[perm[r]] or scale[r]);
// zeros in the padding, for padded indices below p_limit
hipError_t launch_pack_t(const void* src, int ld_src, int ncols,
                         const int32_t* perm, int kdiv, const float* scale,
                         const int32_t* offsets, const int32_t* kofs, int G,
                         int n_single, int64_t p_limit, void* dst,
                         int64_t ld_dst, int bf16, hipStream_t st,
                         int batch = 1, int64_t src_bstride = 0,
                         int64_t dst_bstride = 0);
// gu [rows, 2 d_ff] = [gp | up] and v [rows, d_ff] fp32 in; act [rows, d_ff]
// and dgu [rows, 2 d_ff] = [dgp | du] out (bf16 or fp32); dg_slot[perm[r]]
// = <v_r, act_r> (nullable; gates NULL: gate 1)
hipError_t launch_swiglu_bwd(const float* gu, const float* v, void* act,
                             void* dgu, const int32_t* perm, const float* gates,
                             float* dg_slot, const int32_t* offsets, int G,
                             int rows_bound, int d_ff, int bf16, hipStream_t st);
// The routed rows' SwiGLU backward (launch_swiglu_bwd's values): dgu
// [rows, 2 d_ff] row-major, and act^T [d_ff][ld_t] and [dgp | du]^T
// [2 d_ff][ld_t] in launch_pack_t's transposed, padded layout (kofs; p_limit
// a multiple of 64, ld_t of 8, 16-byte aligned); dg_slot[perm[r]] = <v_r,
// act_r> through dg_part (swiglu_bwd_t_tiles(d_ff) x rows_bound floats).
int swiglu_bwd_t_tiles(int d_ff);
hipError_t launch_swiglu_bwd_t(const float* gu, const float* v, void* dgu, void* act_t,
                               void* dgu_t, int64_t ld_t, const int32_t* perm,
                               const float* gates, const int32_t* offsets, const int32_t* kofs,
                               int G, int64_t p_limit, int rows_bound, int d_ff,
                               float* dg_part, float* dg_slot, int bf16, hipStream_t st);
hipError_t launch_route_bwd(const float* z_part, int splits,
                            const float* b_router, const int32_t* ids,
                            const float* gates, const float* dg_slot,
                            const int32_t* row_of, const int32_t* counts, int T,
                            int N, int k, int mode, float alpha, float d_laux,
                            float d_zloss, float* dz, void* dzb, int ldzb,
                            int bf16, float* dg_out, hipStream_t st);
// db[i] = sum_t dz[t][i] (fixed order); part holds colsum_chunks(T) x N floats
int colsum_chunks(int T);
hipError_t launch_colsum(const float* dz, int T, int N, float* part, float* db,
                         hipStream_t st);
// the router's term either as rows (router, [T, d]) or formed from the
// fp32 dz [T, N] and w_router [N, d] (N <= kMaxRouterFused); exactly one
constexpr int kMaxRouterFused = 16;
hipError_t launch_dh_combine(const void* rows, const int32_t* row_of,
                             const void* shared, const void* router, const float* dz,
                             const void* w_router, int N, void* dh,
                             int T, int k, int d, int bf16, hipStream_t st);
hipError_t launch_kgroup_f32(const float* A, int lda, const float* B, int ldb,
                             const int32_t* kofs, int groups, int M, int Ncols,
                             float* C, int64_t c_gstride, int ldc,
                             hipStream_t st);

// ---------------------------------------------------------------- combine
hipError_t launch_combine(const void* out_rows, const int32_t* row_of,
                          const float* gates, void* y, int T, int k, int d,
                          int has_shared, int bf16, hipStream_t st);

}  // namespace moe
