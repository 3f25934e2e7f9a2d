/*
 * moe.h — C ABI of the HIP (gfx950 / MI355X) forward pass of one sparse
 * Mixture-of-Experts FFN layer.
 *
 * The layer, as the pages define it:
 *   router logits   z_t = W_r h_t (+ b_r)
 *       [page "MOE 专家选择与路由机制" (wuhy-notes), §二 第一步;
 *        page "MoE：router 怎样选 expert" (cooking-agi), first section]
 *   scores          softmax over the N experts [wuhy-notes §二 第二步], or a
 *                   sigmoid per expert [cooking-agi, first section]
 *   top-k + gates   S_t = TopK(score_t, k) [wuhy-notes §二 第三步], with one of
 *                   three gate modes (moe_gate_mode)
 *   dispatch        stable regroup of the (token, slot) pairs by expert
 *                   [wuhy-notes §三 "Token Dispatch";
 *                    page "【大模型】MoE（专家混合模型）简介" (horizon.auto) §3 ②]
 *   experts         E_i(h) = W_down^(i) (SiLU(W_gate^(i) h) ⊙ W_up^(i) h)
 *                   [wuhy-notes §一], run as a grouped GEMM [wuhy-notes §十二
 *                   "小矩阵问题"; horizon.auto §8 Kernel row], plus an optional
 *                   always-on shared expert [wuhy-notes §八]
 *   combine         y_t = Σ_{i∈S_t} g_ti E_i(h_t) (+ shared), a sum, never an
 *                   overwrite [cooking-agi, "选好以后，token 怎么过去，输出怎么回来？"]
 *   load statistics f_i, p_i, L_aux = α·N·Σ f_i p_i
 *                   [page "拆解 MoE：单个 Token 如何经过专家层" (feinterview),
 *                    load-balance section]
 *   capacity        optional: each expert keeps at most C = ⌈cf·T·k/N⌉ slots,
 *                   the earliest in token order; the rest are dropped
 *                   [wuhy-notes §六 Expert Capacity]
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless noted; `stream` is a hipStream_t
 *    passed as void* (NULL = the default stream). Launches are asynchronous
 *    on `stream`; results are valid once the caller synchronises it.
 *  - The caller owns every buffer. The library never allocates, frees or
 *    keeps a pointer after the call returns, and has no mutable global state
 *    other than a per-thread error message and a per-device cache of the
 *    compute-unit count.
 *  - Tensors are contiguous and row-major. Activations (h, y, expert rows)
 *    and weights have the element type `dtype` (fp32 or bf16); biases,
 *    gates and statistics are fp32; indices are int32. Weights use the
 *    [out, in] layout: w_router [N, d]; w_gate, w_up [N, d_ff, d];
 *    w_down [N, d, d_ff]; shared sh_gate, sh_up [d_ff_shared, d],
 *    sh_down [d, d_ff_shared].
 *  - Every pointer that is read or written with vector loads (activations,
 *    weights, expert rows, y) must be 16-byte aligned.
 *  - Arithmetic: fp32 accumulation everywhere. On the bf16 path the SwiGLU
 *    activations and the expert output rows are stored as bf16 (round to
 *    nearest even) and y is rounded to bf16 at the end; the fp32 path
 *    stores fp32 throughout. Ties in top-k go to the lower expert index.
 *  - Errors: every error the host can detect is returned BEFORE anything is
 *    launched, and no HIP call is made before argument validation succeeds:
 *      MOE_ERR_INVALID_ARG  bad shape (T<0, d/N/k/d_ff<1, d_ff_shared<0),
 *                           k > N or k above the kept groups' experts (not
 *                           enough candidates), a group limit that does not
 *                           fit N (see moe_shape), unknown dtype or
 *                           mode, a required pointer NULL, b_select given in
 *                           modes A/B or missing in mode C, misaligned
 *                           pointer, non-finite aux_alpha, capacity_factor
 *                           not finite or outside [0, N];
 *      MOE_ERR_UNSUPPORTED  N > 512, k > 16, more than 64 groups or a group
 *                           score over more than 8 experts, bf16 with d, d_ff or d_ff_shared
 *                           not a multiple of 64, or sizes whose element
 *                           counts exceed 2^31-1 per tensor;
 *      MOE_ERR_WORKSPACE    ws_bytes below the size this call needs (or ws
 *                           NULL when that size is non-zero);
 *      MOE_ERR_HIP          a HIP launch or runtime error.
 *    T = 0 is a valid no-op that still validates its arguments.
 *    moe_last_error() returns a human-readable detail for the calling thread.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 6
#define MOE_MAX_EXPERTS 512
#define MOE_MAX_TOPK 16
#define MOE_MAX_GROUPS 64
#define MOE_MAX_GROUP_TOPM 8

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE = 3,
  MOE_ERR_HIP = 4
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum {
  /* Mode A: top-k by softmax probability, gates renormalised over the k
   * selected (equal to a softmax over the selected logits).
   * [wuhy-notes §二 第三步 gate formula; cooking-agi, first section] */
  MOE_GATE_SOFTMAX_RENORM = 0,
  /* Mode B: top-k by softmax probability, each gate keeps its full-softmax
   * probability, no renormalisation (Switch Transformer top-1; any k).
   * [cooking-agi, first section (Switch remark); pwwt.cn §2.1 route()] */
  MOE_GATE_SOFTMAX_FULL = 1,
  /* Mode C: s = sigmoid(z); select the top-k of s + b_select; gates are the
   * UNBIASED s of the selected, renormalised to sum 1. The bias acts on
   * selection only. [cooking-agi, first section (DeepSeek-V3 remark);
   * feinterview load-balance section (bias placement left open)] */
  MOE_GATE_SIGMOID_BIAS_RENORM = 2
} moe_gate_mode;

/* Host struct describing one layer call. */
typedef struct {
  int32_t T;            /* tokens (rows of h)                                  */
  int32_t d;            /* model width                                         */
  int32_t N;            /* routed experts, 1..512                              */
  int32_t k;            /* experts selected per token, 1..min(N,16)            */
  int32_t d_ff;         /* routed expert hidden width                          */
  int32_t d_ff_shared;  /* shared expert hidden width, 0 = no shared expert    */
  int32_t dtype;        /* moe_dtype of activations and weights               */
  int32_t mode;         /* moe_gate_mode                                       */
  float aux_alpha;      /* α of L_aux = α·N·Σ f_i p_i                          */
  /* Group-limited selection [cooking-agi, section on choosing groups first
   * across devices]: the N experts form n_groups contiguous groups of
   * N / n_groups; a group's score is the sum of its group_topm largest
   * selection scores (softmax probability in modes A/B, sigmoid + b_select
   * in mode C; group_topm = 1 is the group maximum); only the topk_groups
   * best groups (ties to the lower group index) keep their experts as
   * candidates for the top-k. Gates and statistics are unchanged (mode B
   * still uses the full softmax). All three 0 = no group limit. */
  int32_t n_groups;     /* 0, or 1..64 dividing N                              */
  int32_t topk_groups;  /* 1..n_groups, with topk_groups·N/n_groups >= k      */
  int32_t group_topm;   /* 1..min(8, N/n_groups)                               */
  /* Expert capacity [wuhy-notes §六 Expert Capacity]: 0 = dropless; else
   * each expert keeps at most C = ceil(capacity_factor·T·k/N) slots
   * (evaluated in double precision), the first C in token order, and
   * the later slots are dropped: they get no expert row and add nothing to
   * y. f_i, p_i and L_aux still describe the routing (dropped slots count
   * in f_i). Must lie in [0, N]; any factor >= N/k keeps every slot. */
  float capacity_factor;
} moe_shape;

/* ABI version of the loaded library (MOE_ABI_VERSION). */
int moe_abi_version(void);

/* Static string for a status code. */
const char* moe_status_string(moe_status s);

/* Detail of the last non-OK status returned on the calling thread ("" if
 * none). Valid until the next call on this thread. */
const char* moe_last_error(void);

/* Host, pure: workspace bytes that suffice for EVERY call below with this
 * shape (the fused layer needs the most). 0 for an invalid shape.
 * moe_combine uses no workspace; moe_dispatch keeps per-chunk expert counts
 * at the start of its workspace (none when T·k <= 1024, else N rows of
 * ceil(T·k / 256) int32 rounded up to a multiple of 4). moe_route keeps the
 * router's partial logits and per-block probability sums there;
 * moe_expert_ffn keeps the SwiGLU activations (T·k·d_ff + T·d_ff_shared
 * elements) and, on the bf16 path, up to 64 MiB of fp32 split-K partial
 * sums plus 4 KiB of work-queue counters. The workspace needs no
 * initialisation, its contents are undefined after a call, and one
 * workspace serves one call at a time (calls in flight on different
 * streams need separate workspaces). */
size_t moe_workspace_bytes(const moe_shape* s);

/* Router: logits, scores, top-k and gates (steps 1-4).
 *   h          [T, d]   dtype
 *   w_router   [N, d]   dtype
 *   b_router   [N] fp32, nullable (router bias b_r)
 *   b_select   [N] fp32, mode C only (must be NULL in modes A and B)
 *   topk_ids   [T, k] int32 out: slot j holds the (j+1)-th best expert
 *   topk_gates [T, k] fp32  out: gate of that slot
 *   p_mean     [N] fp32 out, nullable: p_i = mean_t P_ti (modes A/B: the
 *              softmax probability; mode C: s_ti / Σ_j s_tj), reduced in a
 *              fixed order (bit-reproducible).
 *   z_loss     [1] fp32 out, nullable: router z-loss (1/T) Σ_t (log Σ_i e^z_ti)²
 *              over the logits z (with b_r) [wuhy-notes §五 Router z-loss]
 *   entropy    [1] fp32 out, nullable: (1/T) Σ_t −Σ_i P_ti log P_ti, the mean
 *              entropy of the routing distribution P (as for p_mean)
 *              [wuhy-notes, monitoring list: routing entropy]
 *   Both scalars are reduced in a fixed order (bit-reproducible).
 * [wuhy-notes §二 第一步–第三步; cooking-agi first section] */
moe_status moe_route(const moe_shape* s, const void* h, const void* w_router,
                     const float* b_router, const float* b_select,
                     int32_t* topk_ids, float* topk_gates, float* p_mean,
                     float* z_loss, float* entropy, void* ws, size_t ws_bytes,
                     void* stream);

/* Dispatch: stable regroup of the T·k flat slots f = t·k + j by expert.
 *   topk_ids [T, k] int32 in, every id in [0, N) (precondition; not checked
 *            on the device)
 *   counts   [N]   int32 out: slots routed to each expert (before capacity)
 *   offsets  [N+1] int32 out: exclusive prefix of the KEPT counts
 *            kept_e = min(counts_e, C) (no capacity: kept = counts and
 *            offsets[N] = T·k)
 *   perm_src [T·k] int32 out: bucket row r -> flat slot for r < offsets[N];
 *            expert e's rows are offsets[e]..offsets[e+1]-1, in ascending
 *            slot (= token) order; entries from offsets[N] on are untouched
 *   row_of   [T·k] int32 out: flat slot -> bucket row (inverse of perm_src),
 *            -1 for a slot dropped by the capacity
 *   p_mean   [N] fp32 in, nullable (needed only for l_aux)
 *   f_out    [N] fp32 out, nullable: f_i = counts_i / (T·k)
 *   l_aux    [1] fp32 out, nullable (requires p_mean): α·N·Σ f_i p_i
 *   cap_stats [2] fp32 out, nullable: capacity usage Σ_e kept_e / (N·C) and
 *            the dropped fraction (T·k − Σ_e kept_e) / (T·k), each the fp32
 *            rounding of the exact ratio; both 0 without a capacity
 *            [wuhy-notes, monitoring list: capacity usage, dropped tokens]
 *   ws       workspace of at least moe_workspace_bytes(s) bytes (it uses the
 *            per-chunk counts described there)
 * Deterministic: no atomic decides any order or any float sum.
 * [wuhy-notes §三 Token Dispatch, §六 Expert Capacity; horizon.auto §3 ②;
 *  feinterview load-balance section] */
moe_status moe_dispatch(const moe_shape* s, const int32_t* topk_ids,
                        int32_t* counts, int32_t* offsets, int32_t* perm_src,
                        int32_t* row_of, const float* p_mean, float* f_out,
                        float* l_aux, float* cap_stats, void* ws,
                        size_t ws_bytes, void* stream);

/* Experts: grouped SwiGLU FFN over the dispatched rows (steps 5-6).
 *   out_rows [T·k (+T if d_ff_shared), d] dtype out:
 *     out_rows[r] = E_e(h[perm_src[r] / k]) for bucket row r of expert e;
 *     out_rows[T·k + t] = E_shared(h[t]) when a shared expert is present.
 *   sh_gate/sh_up/sh_down must be given iff d_ff_shared > 0.
 *   offsets [N+1] as written by moe_dispatch with the same shape
 *   (non-decreasing, offsets[0] = 0, offsets[N] <= T·k, at most min(T, C)
 *   rows per expert; precondition, not checked on the device). Rows from
 *   offsets[N] to T·k−1 of out_rows are not written.
 * Bitwise reproducible: work is spread over the GPU dynamically, but every
 * output element is computed by the same sequence of operations; K-split
 * partial sums are added in split order.
 * [wuhy-notes §一 expert formula, §八 shared expert, §十二 小矩阵问题] */
moe_status moe_expert_ffn(const moe_shape* s, const void* h,
                          const int32_t* perm_src, const int32_t* offsets,
                          const void* w_gate, const void* w_up,
                          const void* w_down, const void* sh_gate,
                          const void* sh_up, const void* sh_down,
                          void* out_rows, void* ws, size_t ws_bytes,
                          void* stream);

/* Combine: y[t] = out_rows[T·k + t] (shared, if any) +
 *          Σ_{j<k} topk_gates[t, j] · out_rows[row_of[t·k + j]],
 * accumulated in fp32 in that order, stored as dtype; a slot with
 * row_of = -1 (dropped by the capacity) adds nothing.
 * [cooking-agi, "选好以后，token 怎么过去，输出怎么回来？"; horizon.auto §3 ④] */
moe_status moe_combine(const moe_shape* s, const void* out_rows,
                       const int32_t* row_of, const float* topk_gates,
                       void* y, void* stream);

/* The whole layer in one call (route, dispatch, experts, combine, stats),
 * no host synchronisation inside.
 *   y [T, d] dtype out (required).
 *   topk_ids, topk_gates, counts, f_out, p_out, l_aux, z_loss, entropy,
 *   cap_stats: nullable outputs as in moe_route / moe_dispatch (the
 *   workspace holds whatever is not returned). */
moe_status moe_layer_fused(const moe_shape* s, const void* h,
                           const void* w_router, const float* b_router,
                           const float* b_select, const void* w_gate,
                           const void* w_up, const void* w_down,
                           const void* sh_gate, const void* sh_up,
                           const void* sh_down, void* y, int32_t* topk_ids,
                           float* topk_gates, int32_t* counts, float* f_out,
                           float* p_out, float* l_aux, float* z_loss,
                           float* entropy, float* cap_stats, void* ws,
                           size_t ws_bytes, void* stream);

/* For callers that cannot allocate: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. moe_layer_fused with no
 * workspace argument: its scratch is a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES (64 MiB) that each GPU the library runs on holds
 * from the first call until the process ends. The call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine); the caller still
 * passes inputs and outputs, with the arguments, layouts and results of
 * moe_layer_fused (the same bits). The layout is moe_layer_fused's without
 * the split-K partial region when no tiled GEMM runs (bf16 with at most 64
 * rows per expert and a shared expert over at most 64 tokens, or fp32), so
 * every decode batch of the layer shapes here fits; a shape that needs more
 * returns MOE_ERR_WORKSPACE before any HIP call.
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's contents (each call clears the counters it uses itself): calls that
 * overlap on one GPU (concurrent streams or threads) race, so serialise
 * them. Errors: as moe_layer_fused; MOE_ERR_HIP if the scratch's device
 * address cannot be obtained. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_layer_fused_noalloc(const moe_shape* s, const void* h,
                                   const void* w_router, const float* b_router,
                                   const float* b_select, const void* w_gate,
                                   const void* w_up, const void* w_down,
                                   const void* sh_gate, const void* sh_up,
                                   const void* sh_down, void* y,
                                   int32_t* topk_ids, float* topk_gates,
                                   int32_t* counts, float* f_out, float* p_out,
                                   float* l_aux, float* z_loss, float* entropy,
                                   float* cap_stats, void* stream);

/* moe_layer_fused that also records caller-created hipEvent_t handles on
 * `stream` at the stage boundaries, for timing: events[0] before routing,
 * [1] after routing, [2] after dispatch, [3] after the gate/up GEMM
 * (SwiGLU), [4] after the down GEMM, [5] after combine. `events` is a host
 * array of 6 hipEvent_t (as void*); a NULL entry records nothing at that
 * boundary. Where one kernel does two stages, the boundary between them is
 * recorded back to back: [1] and [2] when a batch that fits one selection
 * block and one dispatch chunk is selected and dispatched by one kernel, [4]
 * and [5] when the combine runs inside the down GEMM (bf16, at most 64 rows
 * per expert). */
moe_status moe_layer_fused_marked(const moe_shape* s, const void* h,
                                  const void* w_router, const float* b_router,
                                  const float* b_select, const void* w_gate,
                                  const void* w_up, const void* w_down,
                                  const void* sh_gate, const void* sh_up,
                                  const void* sh_down, void* y,
                                  int32_t* topk_ids, float* topk_gates,
                                  int32_t* counts, float* f_out, float* p_out,
                                  float* l_aux, float* z_loss, float* entropy,
                                  float* cap_stats, void* ws, size_t ws_bytes,
                                  void* stream, void* const* events);

/* The forward pass for training: moe_layer_fused that also returns what
 * moe_layer_backward takes, so that the backward neither re-routes nor (with
 * preact) recomputes the gate/up GEMM.
 *   topk_ids, topk_gates [T, k], counts [N], offsets [N+1], perm_src [T·k],
 *   row_of [T·k]: required outputs, as moe_route / moe_dispatch define them;
 *   preact fp32 out, nullable: the gate and up pre-activations of every kept
 *     row, [T·k, 2·d_ff] in bucket order (row r of expert e = the bucket row
 *     of moe_dispatch; gate in columns [0, d_ff), up in [d_ff, 2·d_ff); rows
 *     from offsets[N] on are not written), then, with a shared expert,
 *     [T, 2·d_ff_shared] for the shared expert; 4-byte aligned. With preact
 *     the gate/up GEMM runs on its grouped tiles at every row count.
 *   p_out, l_aux, z_loss, entropy: nullable, as in moe_layer_fused.
 * y and every output equal moe_layer_fused's on the same inputs (at decode
 * sizes with preact, within rounding: another tile shape). */
moe_status moe_layer_forward_train(const moe_shape* s, const void* h,
                                   const void* w_router, const float* b_router,
                                   const float* b_select, const void* w_gate,
                                   const void* w_up, const void* w_down,
                                   const void* sh_gate, const void* sh_up,
                                   const void* sh_down, void* y,
                                   int32_t* topk_ids, float* topk_gates,
                                   int32_t* counts, int32_t* offsets,
                                   int32_t* perm_src, int32_t* row_of,
                                   float* preact, float* p_out, float* l_aux,
                                   float* z_loss, float* entropy, void* ws,
                                   size_t ws_bytes, void* stream);

/* Host, pure: workspace bytes for moe_layer_backward with this shape (0 for
 * an invalid shape). It holds the recomputed router logits and gate/up
 * pre-activations, the intermediate row gradients, zero-padded transposed
 * activations for the weight gradients, the GEMMs' split-K partials, a
 * transposed copy of the router weights and, only where an expert (or the
 * shared expert) has at most 64 rows or the dtype is fp32, transposed
 * copies of its weights: of the order of 10 (T·k + 32·N) max(d, 2 d_ff)
 * elements (plus 3x the expert weights in those cases). No initialisation
 * needed; one call at a time per workspace. */
size_t moe_backward_workspace_bytes(const moe_shape* s);

/* Backward pass of the layer for the selection and dispatch of a forward
 * call: the gradients of  <dy, y> + d_laux·L_aux + d_zloss·L_z  with the
 * discrete selection held fixed [cooking-agi, "top-k 不可导，router 怎么学" and
 * "怎么知道实现没把梯度弄丢？"; wuhy-notes, "Top-k 不可导，为什么 Router 还能学"
 * and the total-loss paragraph].
 * The router receives gradient only through the gate values of the selected
 * experts (mode A: the softmax of the selected logits; mode B: the full
 * softmax, so every logit; mode C: the renormalised sigmoids of the
 * selected; b_select is not differentiated), plus the L_aux term (f_i are
 * counts and carry no gradient; p_i = mean_t P_ti does) and the z-loss
 * term. A slot dropped by the capacity contributes nothing. Experts get
 * gradient only from their kept rows.
 * Inputs: the forward's inputs (b_select is not needed) and its outputs
 *   topk_ids, topk_gates [T, k], counts [N] (routed, before capacity),
 *   offsets [N+1], perm_src [T·k], row_of [T·k] exactly as moe_route /
 *   moe_dispatch (or moe_layer_forward_train) wrote them for this shape;
 *   preact fp32, nullable: moe_layer_forward_train's pre-activations (the
 *   backward then skips their recompute; the gradients are the same bits);
 *   dy [T, d] dtype; d_laux and
 *   d_zloss are host scalars (the weights of L_aux and L_z in the loss;
 *   0 leaves them out).
 * Outputs (overwritten, not accumulated):
 *   dh [T, d] dtype; dw_gate, dw_up [N, d_ff, d], dw_down [N, d, d_ff]
 *   dtype (zero for experts without kept rows); dsh_gate, dsh_up [d_ff_shared,
 *   d], dsh_down [d, d_ff_shared] dtype, required iff d_ff_shared > 0;
 *   dw_router [N, d] fp32; db_router [N] fp32, nullable; dgates [T, k]
 *   fp32, nullable: dL/dg per slot (0 for dropped slots).
 * Arithmetic: fp32 accumulation; on the bf16 path the recomputed
 * pre-activations, the row gradients and the router-logit gradient fed to
 * the weight-gradient GEMMs are rounded to bf16. Deterministic (no float
 * atomics). Errors as for the other calls (MOE_ERR_UNSUPPORTED also when a
 * padded transposed activation exceeds 2^31 bytes). */
moe_status moe_layer_backward(const moe_shape* s, const void* h,
                              const void* w_router, const float* b_router,
                              const void* w_gate, const void* w_up,
                              const void* w_down, const void* sh_gate,
                              const void* sh_up, const void* sh_down,
                              const int32_t* topk_ids, const float* topk_gates,
                              const int32_t* counts, const int32_t* offsets,
                              const int32_t* perm_src, const int32_t* row_of,
                              const float* preact, const void* dy, float d_laux,
                              float d_zloss,
                              void* dh, float* dw_router, float* db_router,
                              void* dw_gate, void* dw_up, void* dw_down,
                              void* dsh_gate, void* dsh_up, void* dsh_down,
                              float* dgates, void* ws, size_t ws_bytes,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
