// C ABI of the MoE layer: argument validation, workspace layout and the
// launch sequence route -> dispatch -> expert GEMMs -> combine. Every check
// runs before the first HIP call, so invalid arguments never reach the GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <optional>
#include <string>

#include "../../include/moe.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_err;

moe_status fail(moe_status st, const std::string& msg) {
  g_err = msg;
  return st;
}

constexpr int64_t kI32Max = 2147483647LL;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

size_t esize(const moe_shape* s) { return s->dtype == MOE_BF16 ? 2 : 4; }

// ------------------------------------------------------------ validation
moe_status check_shape(const moe_shape* s) {
  if (!s) return fail(MOE_ERR_INVALID_ARG, "shape is NULL");
  if (s->T < 0) return fail(MOE_ERR_INVALID_ARG, "T < 0");
  if (s->d < 1 || s->N < 1 || s->k < 1 || s->d_ff < 1)
    return fail(MOE_ERR_INVALID_ARG, "d, N, k and d_ff must be >= 1");
  if (s->d_ff_shared < 0) return fail(MOE_ERR_INVALID_ARG, "d_ff_shared < 0");
  if (s->dtype != MOE_F32 && s->dtype != MOE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "unknown dtype");
  if (s->mode < MOE_GATE_SOFTMAX_RENORM || s->mode > MOE_GATE_SIGMOID_BIAS_RENORM)
    return fail(MOE_ERR_INVALID_ARG, "unknown gate mode");
  if (!std::isfinite(s->aux_alpha)) return fail(MOE_ERR_INVALID_ARG, "aux_alpha is not finite");
  if (!std::isfinite(s->capacity_factor) || s->capacity_factor < 0.0f ||
      s->capacity_factor > (float)s->N)
    return fail(MOE_ERR_INVALID_ARG, "capacity_factor must be finite and in [0, N]");
  if (s->k > s->N) return fail(MOE_ERR_INVALID_ARG, "k > N: not enough candidate experts");
  if (s->N > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "N > 512");
  if (s->k > MOE_MAX_TOPK) return fail(MOE_ERR_UNSUPPORTED, "k > 16");
  if (s->n_groups == 0) {
    if (s->topk_groups != 0 || s->group_topm != 0)
      return fail(MOE_ERR_INVALID_ARG, "topk_groups and group_topm need n_groups > 0");
  } else {
    if (s->n_groups < 0 || s->N % s->n_groups)
      return fail(MOE_ERR_INVALID_ARG, "n_groups must divide N");
    if (s->n_groups > MOE_MAX_GROUPS) return fail(MOE_ERR_UNSUPPORTED, "n_groups > 64");
    const int gs = s->N / s->n_groups;
    if (s->topk_groups < 1 || s->topk_groups > s->n_groups)
      return fail(MOE_ERR_INVALID_ARG, "need 1 <= topk_groups <= n_groups");
    if (s->group_topm < 1 || s->group_topm > gs)
      return fail(MOE_ERR_INVALID_ARG, "need 1 <= group_topm <= N / n_groups");
    if (s->group_topm > MOE_MAX_GROUP_TOPM) return fail(MOE_ERR_UNSUPPORTED, "group_topm > 8");
    if ((int64_t)s->topk_groups * gs < s->k)
      return fail(MOE_ERR_INVALID_ARG, "the kept groups hold fewer than k experts");
  }
  if (s->dtype == MOE_BF16 &&
      (s->d % 64 || s->d_ff % 64 || s->d_ff_shared % 64))
    return fail(MOE_ERR_UNSUPPORTED, "bf16 needs d, d_ff and d_ff_shared multiples of 64");
  const int64_t T = s->T, R = T * s->k, Rt = R + (s->d_ff_shared ? T : 0);
  const int64_t lim[] = {R, Rt * s->d, R * s->d_ff, T * s->d_ff_shared, T * s->d,
                         (int64_t)s->d_ff * s->d, (int64_t)s->d_ff_shared * s->d,
                         (int64_t)s->N * s->d, T * s->N * moe::kRouterMaxSplits};
  for (int64_t v : lim)
    if (v > kI32Max) return fail(MOE_ERR_UNSUPPORTED, "a tensor exceeds 2^31-1 elements");
  return MOE_OK;
}

// Expert capacity C = ceil(capacity_factor * T * k / N) in double precision,
// 0 for dropless [wuhy-notes §六 Expert Capacity]. capacity_factor <= N keeps
// C <= T * k.
int expert_capacity(const moe_shape* s) {
  if (s->capacity_factor == 0.0f) return 0;
  const double c = std::ceil((double)s->capacity_factor * (double)((int64_t)s->T * s->k) /
                             (double)s->N);
  return (int)c;
}

moe_status need(const void* p, const char* name) {
  if (!p) return fail(MOE_ERR_INVALID_ARG, std::string(name) + " is NULL");
  return MOE_OK;
}
moe_status need16(const void* p, const char* name) {
  if (!p) return fail(MOE_ERR_INVALID_ARG, std::string(name) + " is NULL");
  if (!aligned16(p)) return fail(MOE_ERR_INVALID_ARG, std::string(name) + " is not 16-byte aligned");
  return MOE_OK;
}
moe_status need4(const void* p, const char* name) {
  if (!p) return fail(MOE_ERR_INVALID_ARG, std::string(name) + " is NULL");
  if (!aligned4(p)) return fail(MOE_ERR_INVALID_ARG, std::string(name) + " is not 4-byte aligned");
  return MOE_OK;
}
moe_status opt4(const void* p, const char* name) {
  if (p && !aligned4(p)) return fail(MOE_ERR_INVALID_ARG, std::string(name) + " is not 4-byte aligned");
  return MOE_OK;
}

#define TRY(x)                      \
  do {                              \
    const moe_status _st = (x);     \
    if (_st != MOE_OK) return _st;  \
  } while (0)

moe_status check_bias(const moe_shape* s, const float* b_router, const float* b_select) {
  TRY(opt4(b_router, "b_router"));
  if (s->mode == MOE_GATE_SIGMOID_BIAS_RENORM) {
    TRY(need4(b_select, "b_select (mode C)"));
  } else if (b_select) {
    return fail(MOE_ERR_INVALID_ARG, "b_select must be NULL in the softmax gate modes");
  }
  return MOE_OK;
}

moe_status check_shared(const moe_shape* s, const void* sg, const void* su, const void* sd) {
  if (s->d_ff_shared) {
    TRY(need16(sg, "sh_gate"));
    TRY(need16(su, "sh_up"));
    TRY(need16(sd, "sh_down"));
  } else if (sg || su || sd) {
    return fail(MOE_ERR_INVALID_ARG, "shared-expert weights given but d_ff_shared = 0");
  }
  return MOE_OK;
}

// ------------------------------------------------------- workspace layout
struct RouteWs {
  size_t z, p_part, zl_part, end;
};
RouteWs route_ws(const moe_shape* s, size_t base) {
  RouteWs w;
  const size_t blocks = (size_t)moe::route_select_blocks(s->T, s->N);
  w.z = base;
  w.p_part = align_up(w.z + sizeof(float) * (size_t)moe::kRouterMaxSplits * s->T * s->N);
  w.zl_part = align_up(w.p_part + sizeof(float) * blocks * s->N);
  w.end = align_up(w.zl_part + sizeof(float) * blocks * 2);
  return w;
}
size_t act_bytes(const moe_shape* s) {
  const size_t R = (size_t)s->T * s->k;
  return esize(s) * (R * s->d_ff + (size_t)s->T * s->d_ff_shared);
}
// Expert stage: SwiGLU activations, then (bf16) the split-K partial sums
// and arrival counters of the grouped GEMMs.
int64_t split_floats(const moe_shape* s) {
  if (s->dtype != MOE_BF16) return 0;
  const int64_t R = (int64_t)s->T * s->k;
  int64_t f = std::max(moe::split_part_floats(R, s->N, s->d_ff, true),
                       moe::split_part_floats(R, s->N, s->d, false));
  if (s->d_ff_shared)
    f = std::max(f, std::max(moe::split_part_floats(s->T, 1, s->d_ff_shared, true),
                             moe::split_part_floats(s->T, 1, s->d, false)));
  return f;
}
struct FfnWs {
  size_t act, part, cnt, end;
};
// Whether the forward launches a grouped (tiled) GEMM, whose split-K tail
// uses the partial-sum region: bf16 with more than 64 rows per expert, or a
// shared expert over more than 64 tokens (at most 64 rows, the weight-
// streaming kernels run, which need no partials).
bool grouped_gemm_used(const moe_shape* s) {
  if (s->dtype != MOE_BF16) return false;
  const int C = expert_capacity(s);
  const int rows_max = C ? std::min(s->T, C) : s->T;
  return rows_max > 64 || (s->d_ff_shared && s->T > 64);
}
// trim: no partial-sum region when no grouped GEMM runs (the layout of the
// allocation-free forward; the caller-workspace calls keep the full one,
// which the training forward also uses at every row count).
FfnWs ffn_ws(const moe_shape* s, size_t base, bool trim = false) {
  FfnWs w;
  w.act = base;
  w.part = align_up(w.act + act_bytes(s));
  const int64_t f = (trim && !grouped_gemm_used(s)) ? 0 : split_floats(s);
  w.cnt = align_up(w.part + sizeof(float) * (size_t)f);
  w.end = f ? align_up(w.cnt + sizeof(int32_t) * moe::kSplitCounters) : w.cnt;
  return w;
}
// dispatch scratch: per-chunk expert counts
size_t dispatch_ws_bytes(const moe_shape* s) {
  return align_up(sizeof(int32_t) * (size_t)moe::dispatch_hist_ints(s->T, s->k, s->N));
}

struct FusedWs {
  RouteWs r;
  FfnWs x;
  size_t p_mean, ids, gates, counts, offsets, perm, row_of, f, dhist, cmb, rows, end;
};
FusedWs fused_ws(const moe_shape* s, bool trim = false) {
  FusedWs w;
  w.r = route_ws(s, 0);
  const size_t T = s->T, N = s->N, R = T * s->k;
  w.p_mean = w.r.end;
  w.ids = align_up(w.p_mean + 4 * N);
  w.gates = align_up(w.ids + 4 * R);
  w.counts = align_up(w.gates + 4 * R);
  w.offsets = align_up(w.counts + 4 * N);
  w.perm = align_up(w.offsets + 4 * (N + 1));
  w.row_of = align_up(w.perm + 4 * R);
  w.f = align_up(w.row_of + 4 * R);
  w.dhist = align_up(w.f + 4 * N + 4);
  w.cmb = w.dhist + dispatch_ws_bytes(s);
  w.x = ffn_ws(s, align_up(w.cmb + 4 * (size_t)moe::combine_counters(s->d)), trim);
  w.rows = w.x.end;
  w.end = align_up(w.rows + esize(s) * (R + (s->d_ff_shared ? T : 0)) * s->d);
  return w;
}

moe_status check_ws(void* ws, size_t ws_bytes, size_t need_bytes) {
  if (need_bytes == 0) return MOE_OK;
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned16(ws)) return fail(MOE_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  if (ws_bytes < need_bytes)
    return fail(MOE_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need_bytes) +
                                       " bytes, got " + std::to_string(ws_bytes));
  return MOE_OK;
}

// ------------------------------------------------------------- device info
int num_cu() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (dev < 64 && cache[dev]) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) cache[dev] = n;
  return n;
}

moe_status hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(MOE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return MOE_OK;
}

// ----------------------------------------------- allocation-free scratch
// The workspace of moe_layer_fused_noalloc: a file-scope device array, of
// which every GPU the library runs on holds its own copy until the process
// ends. In host code the array's name is a host-side stand-in, never a
// device address: the address of the current device's copy comes from
// hipGetSymbolAddress, taken once per device (with that device current) and
// kept; only that address reaches kernels.
constexpr size_t kNoAllocScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char g_noalloc_scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;

moe_status noalloc_scratch(void** out) {
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {nullptr};
  int dev = -1;
  TRY(hip_check(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "device index beyond 63 for the static scratch");
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    TRY(hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(g_noalloc_scratch)),
                  "hipGetSymbolAddress(scratch)"));
    if (!p || !aligned16(p)) return fail(MOE_ERR_HIP, "scratch address is not usable");
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return MOE_OK;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// ------------------------------------------------------------ stage impls
// Router logits as split-K slices z_part[splits][T][N] (bf16: a GEMV for a
// few tokens, else the split-K GEMM; fp32: one slice).
moe_status router_logits(const moe_shape* s, const void* h, const void* w_router, float* z_part,
                         int& splits, hipStream_t st) {
  splits = 1;
  if (s->dtype == MOE_BF16) {
    if (moe::router_use_gemv(s->T, s->N))
      return hip_check(moe::launch_router_gemv_bf16(h, w_router, z_part, s->T, s->d, s->N, st),
                       "router GEMV");
    splits = moe::router_splits(s->T, s->d, s->N);
    return hip_check(moe::launch_router_gemm_bf16(h, w_router, z_part, s->T, s->d, s->N, splits,
                                                  st),
                     "router GEMM");
  }
  return hip_check(moe::launch_router_logits_f32(static_cast<const float*>(h),
                                                 static_cast<const float*>(w_router), z_part,
                                                 s->T, s->d, s->N, st),
                   "router logits");
}

// A batch that fits one selection block and one dispatch chunk.
bool route_dispatch_fits(const moe_shape* s) {
  return moe::route_select_blocks(s->T, s->N) == 1 && moe::dispatch_chunks(s->T, s->k) == 1;
}

// dq (only when route_dispatch_fits): the selection kernel also dispatches.
moe_status route_impl(const moe_shape* s, const void* h, const void* w_router,
                      const float* b_router, const float* b_select, int32_t* ids,
                      float* gates, float* p_mean, float* z_loss, float* entropy,
                      const RouteWs& W, void* ws, hipStream_t st,
                      const std::optional<moe::DispatchOut>& dq = std::nullopt) {
  float* z_part = at<float>(ws, W.z);
  float* p_part = at<float>(ws, W.p_part);
  float* zl_part = (z_loss || entropy) ? at<float>(ws, W.zl_part) : nullptr;
  int splits = 1;
  TRY(router_logits(s, h, w_router, z_part, splits, st));
  // a group limit that keeps every group changes nothing
  const bool grouped = s->n_groups > 1 && s->topk_groups < s->n_groups;
  const moe::GroupLimit gl{grouped ? s->n_groups : 0, s->topk_groups, s->group_topm};
  // a single selection block writes the final statistics itself
  const bool single = moe::route_select_blocks(s->T, s->N) == 1;
  const moe::RouteFinal fin{p_mean, z_loss, entropy, single ? 1 : 0};
  TRY(hip_check(moe::launch_route_select(z_part, splits, b_router, b_select, ids, gates,
                                         p_mean ? p_part : nullptr, zl_part, s->T, s->N, s->k,
                                         s->mode, gl, fin, st, dq ? &*dq : nullptr),
                dq ? "route select + dispatch" : "route select"));
  if (!single && (p_mean || zl_part))
    TRY(hip_check(moe::launch_p_reduce(p_part, p_mean, zl_part, z_loss, entropy,
                                       moe::route_select_blocks(s->T, s->N), s->T, s->N, st),
                  "p reduce"));
  return MOE_OK;
}

moe_status dispatch_impl(const moe_shape* s, const int32_t* ids, int32_t* counts,
                         int32_t* offsets, int32_t* perm_src, int32_t* row_of,
                         const float* p_mean, float* f_out, float* l_aux, float* cap_stats,
                         int32_t* hist, hipStream_t st, int32_t* zero = nullptr,
                         int zero_n = 0) {
  return hip_check(moe::launch_dispatch(ids, s->T, s->k, s->N, counts, offsets, perm_src, row_of,
                                        p_mean, f_out, l_aux, s->aux_alpha, expert_capacity(s),
                                        cap_stats, hist, st, zero, zero_n),
                   "dispatch");
}

// bf16 with a shared expert as wide as the routed ones: the grouped
// launchers run it as one more group of the routed experts' launch (or on
// its own where the routed experts take the weight-streaming kernels).
bool shared_in_routed(const moe_shape* s) {
  return s->dtype == MOE_BF16 && s->d_ff_shared > 0 && s->d_ff_shared == s->d_ff;
}

moe_status ffn_stage(const moe_shape* s, bool gateup, const void* h, const int32_t* perm_src,
                     const int32_t* offsets, const void* w_gate, const void* w_up,
                     const void* w_down, const void* sh_gate, const void* sh_up,
                     const void* sh_down, void* out_rows, void* ws, const FfnWs& W,
                     hipStream_t st, float* preact = nullptr,
                     const moe::CombineFuse* fuse = nullptr, bool* combined = nullptr) {
  const int T = s->T, d = s->d, dff = s->d_ff, dfs = s->d_ff_shared;
  void* act = at<char>(ws, W.act);
  float* part = W.cnt > W.part ? at<float>(ws, W.part) : nullptr;
  int32_t* part_cnt = part ? at<int32_t>(ws, W.cnt) : nullptr;
  const int64_t part_floats = part ? (int64_t)((W.cnt - W.part) / sizeof(float)) : 0;
  const int R = T * s->k;
  // bounds on the routed rows: all of them and T per expert, or what the
  // capacity keeps
  const int C = expert_capacity(s);
  const int rows_all = C ? (int)std::min<int64_t>(R, (int64_t)s->N * C) : R;
  const int rows_max = C ? std::min(T, C) : T;
  const bool bf16 = s->dtype == MOE_BF16;
  const int ncu = bf16 ? num_cu() : 0;
  const size_t esz = esize(s);
  void* act_sh = static_cast<char*>(act) + esize(s) * (size_t)R * dff;
  auto run = [&](const moe::GroupedProblem& p, bool gu) -> hipError_t {
    if (bf16) return gu ? moe::launch_gateup_bf16(p, ncu, st) : moe::launch_down_bf16(p, ncu, st);
    return gu ? moe::launch_gateup_f32(p, st) : moe::launch_down_f32(p, st);
  };
  // the shared expert as one more group of the routed launches (same
  // d_ff): its rows h[t] in order, its outputs at rows R + t
  const bool merge = shared_in_routed(s);
  moe::GroupedProblem p{};
  if (gateup) {
    p = moe::GroupedProblem{h, d, perm_src, s->k, offsets, s->N, rows_all, rows_max, w_gate,
                            w_up, (int64_t)dff * d, d, dff, d, act, dff, 0, (uint32_t)(esz * T * d),
                            part, part_cnt, part_floats, preact, 2 * (int64_t)dff};
    if (merge) {
      p.X0 = sh_gate;
      p.X1 = sh_up;
      p.x_rows = T;
      p.x_a_row0 = 0;
      p.x_c_row0 = R;
    }
    TRY(hip_check(run(p, true), merge ? "gate/up GEMM (routed and shared)" : "gate/up GEMM"));
    if (dfs && !merge) {
      p = moe::GroupedProblem{h, d, nullptr, 1, nullptr, 1, T, T, sh_gate, sh_up, 0, d, dfs, d,
                              act_sh, dfs, 0, (uint32_t)(esz * T * d),
                              part, part_cnt, part_floats,
                              preact ? preact + (int64_t)R * 2 * dff : nullptr, 2 * (int64_t)dfs};
      TRY(hip_check(run(p, true), "shared gate/up GEMM"));
    }
  } else {
    const moe::GroupedProblem pr{act, dff, nullptr, 1, offsets, s->N, rows_all, rows_max, w_down,
                                 nullptr, (int64_t)d * dff, dff, d, dff, out_rows, d, 0,
                                 (uint32_t)(esz * R * dff), part, part_cnt, part_floats};
    const moe::GroupedProblem ps{act_sh, dfs, nullptr, 1, nullptr, 1, T, T, sh_down, nullptr, 0,
                                 dfs, d, dfs, out_rows, d, (int64_t)R, (uint32_t)(esz * T * dfs),
                                 part, part_cnt, part_floats};
    // the combine fused into the weight-streaming down GEMM: the shared
    // expert's rows first, then the routed rows and the combine
    const bool fused = fuse && bf16 && moe::down_combine_ok(pr, *fuse);
    if (combined) *combined = fused;
    if (fused) {
      if (dfs) TRY(hip_check(run(ps, false), "shared down GEMM"));
      return hip_check(moe::launch_down_combine_bf16(pr, *fuse, ncu, st), "down GEMM + combine");
    }
    if (merge) {
      moe::GroupedProblem pm = pr;
      pm.a_bytes = (uint32_t)(esz * ((size_t)R + T) * dff);
      pm.X0 = sh_down;
      pm.x_rows = T;
      pm.x_a_row0 = R;
      pm.x_c_row0 = R;
      return hip_check(run(pm, false), "down GEMM (routed and shared)");
    }
    TRY(hip_check(run(pr, false), "down GEMM"));
    if (dfs) TRY(hip_check(run(ps, false), "shared down GEMM"));
  }
  return MOE_OK;
}

moe_status combine_impl(const moe_shape* s, const void* out_rows, const int32_t* row_of,
                        const float* gates, void* y, hipStream_t st) {
  return hip_check(moe::launch_combine(out_rows, row_of, gates, y, s->T, s->k, s->d,
                                       s->d_ff_shared ? 1 : 0, s->dtype == MOE_BF16, st),
                   "combine");
}

moe_status mark(void* const* events, int i, hipStream_t st) {
  if (!events || !events[i]) return MOE_OK;
  return hip_check(hipEventRecord(static_cast<hipEvent_t>(events[i]), st), "event record");
}

// What the training forward returns besides the fused call's outputs.
struct TrainOut {
  int32_t* offsets;
  int32_t* perm;
  int32_t* row_of;
  float* preact;
};

moe_status layer_impl(const moe_shape* s, const void* h, const void* w_router,
                      const float* b_router, const float* b_select, const void* w_gate,
                      const void* w_up, const void* w_down, const void* sh_gate,
                      const void* sh_up, const void* sh_down, void* y, int32_t* topk_ids,
                      float* topk_gates, int32_t* counts, float* f_out, float* p_out,
                      float* l_aux, float* z_loss, float* entropy, float* cap_stats, void* ws,
                      size_t ws_bytes, void* stream, void* const* events,
                      const TrainOut& train = TrainOut{nullptr, nullptr, nullptr, nullptr},
                      bool noalloc = false) {
  TRY(check_shape(s));
  TRY(need16(h, "h"));
  TRY(need16(w_router, "w_router"));
  TRY(check_bias(s, b_router, b_select));
  TRY(need16(w_gate, "w_gate"));
  TRY(need16(w_up, "w_up"));
  TRY(need16(w_down, "w_down"));
  TRY(check_shared(s, sh_gate, sh_up, sh_down));
  TRY(need16(y, "y"));
  TRY(opt4(topk_ids, "topk_ids"));
  TRY(opt4(topk_gates, "topk_gates"));
  TRY(opt4(counts, "counts"));
  TRY(opt4(f_out, "f_out"));
  TRY(opt4(p_out, "p_out"));
  TRY(opt4(l_aux, "l_aux"));
  TRY(opt4(z_loss, "z_loss"));
  TRY(opt4(entropy, "entropy"));
  TRY(opt4(cap_stats, "cap_stats"));
  TRY(opt4(train.offsets, "offsets"));
  TRY(opt4(train.perm, "perm_src"));
  TRY(opt4(train.row_of, "row_of"));
  TRY(opt4(train.preact, "preact"));
  const FusedWs L = fused_ws(s, noalloc);
  if (noalloc) {
    if (L.end > kNoAllocScratchBytes)
      return fail(MOE_ERR_WORKSPACE,
                  "this shape needs " + std::to_string(L.end) + " bytes of scratch, more than "
                  "the " + std::to_string(kNoAllocScratchBytes) + " the allocation-free call "
                  "holds; use moe_layer_fused with a workspace");
    if (s->T == 0) return MOE_OK;
    TRY(noalloc_scratch(&ws));
    ws_bytes = L.end;
  } else {
    TRY(check_ws(ws, ws_bytes, L.end));
    if (s->T == 0) return MOE_OK;
  }

  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* ids = topk_ids ? topk_ids : at<int32_t>(ws, L.ids);
  float* gates = topk_gates ? topk_gates : at<float>(ws, L.gates);
  int32_t* cnt = counts ? counts : at<int32_t>(ws, L.counts);
  const bool want_p = p_out || l_aux;
  float* p_mean = want_p ? (p_out ? p_out : at<float>(ws, L.p_mean)) : nullptr;
  int32_t* offsets = train.offsets ? train.offsets : at<int32_t>(ws, L.offsets);
  int32_t* perm = train.perm ? train.perm : at<int32_t>(ws, L.perm);
  int32_t* row_of = train.row_of ? train.row_of : at<int32_t>(ws, L.row_of);
  void* rows = at<char>(ws, L.rows);

  int32_t* cmb_cnt = at<int32_t>(ws, L.cmb);
  const int cmb_n = moe::combine_counters(s->d);

  TRY(mark(events, 0, st));
  if (route_dispatch_fits(s)) {
    // one selection block and one dispatch chunk: a single kernel selects
    // and dispatches (same bits as the separate kernels)
    TRY(route_impl(s, h, w_router, b_router, b_select, ids, gates, p_mean, z_loss, entropy, L.r,
                   ws, st,
                   moe::DispatchOut{cnt, offsets, perm, row_of, f_out, l_aux, s->aux_alpha,
                                    expert_capacity(s), cap_stats, cmb_cnt, cmb_n}));
    TRY(mark(events, 1, st));
  } else {
    TRY(route_impl(s, h, w_router, b_router, b_select, ids, gates, p_mean, z_loss, entropy, L.r,
                   ws, st));
    TRY(mark(events, 1, st));
    TRY(dispatch_impl(s, ids, cnt, offsets, perm, row_of, p_mean, f_out, l_aux, cap_stats,
                      at<int32_t>(ws, L.dhist), st, cmb_cnt, cmb_n));
  }
  TRY(mark(events, 2, st));
  TRY(ffn_stage(s, true, h, perm, offsets, w_gate, w_up, w_down, sh_gate, sh_up, sh_down, rows,
                ws, L.x, st, train.preact));
  TRY(mark(events, 3, st));
  const moe::CombineFuse fuse{row_of, gates, y, s->T, s->k, s->d_ff_shared ? 1 : 0, cmb_cnt};
  bool combined = false;
  TRY(ffn_stage(s, false, h, perm, offsets, w_gate, w_up, w_down, sh_gate, sh_up, sh_down, rows,
                ws, L.x, st, nullptr, &fuse, &combined));
  TRY(mark(events, 4, st));
  if (!combined) TRY(combine_impl(s, rows, row_of, gates, y, st));
  TRY(mark(events, 5, st));
  return MOE_OK;
}

// ------------------------------------------------------------- backward
int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Workspace of the backward pass (offsets in bytes; sizes in elements of the
// layer dtype unless noted).
struct BwdWs {
  RouteWs r;                 // router logits (split-K slices)
  int64_t Rp, Tp, Np;        // padded K spaces: routed rows, tokens, experts
  int64_t ta_rows, tb_rows;  // rows of the transposed-activation buffers
  size_t kofs, kofs_t, dg, dz, dzb, colpart;
  size_t gu, v, dgu, dgpart, gus, vs, dgus, acts;
  size_t wdT, wguT, sdT, sguT, wrT;
  size_t dhr, dhs, dhrt;
  size_t ta, tb, tc, part, cnt, end;
  int64_t part_floats;
};
// Rows per expert at most (all routed rows of a token set, or the capacity).
int bwd_rows_max(const moe_shape* s) {
  const int C = expert_capacity(s);
  return C ? std::min(s->T, C) : s->T;
}
// bf16 with more than 64 rows per expert (per shared-expert call: T): v and
// the h-row gradients read the weights in their own [K, N] layout (no
// transposed copies); fewer rows take the weight-streaming kernels, which
// read K-contiguous (transposed) weights.
bool bwd_nn(const moe_shape* s) { return s->dtype == MOE_BF16 && bwd_rows_max(s) > 64; }
bool bwd_nn_shared(const moe_shape* s) { return s->dtype == MOE_BF16 && s->T > 64; }

BwdWs bwd_ws(const moe_shape* s) {
  BwdWs w;
  const int64_t T = s->T, N = s->N, k = s->k, d = s->d, dff = s->d_ff, dfs = s->d_ff_shared;
  const int64_t R = T * k;
  const size_t es = esize(s);
  w.Rp = round_up(R + 64 * N, 64);
  w.Tp = round_up(T, 64);
  w.Np = round_up(N, 64);
  w.ta_rows = std::max(std::max(d, 2 * dff), std::max(2 * dfs, w.Np));
  w.tb_rows = std::max(std::max(d, dff), dfs);
  w.r = route_ws(s, 0);
  size_t o = w.r.end;
  auto take = [&](size_t bytes) {
    const size_t at_ = o;
    o = align_up(o + bytes);
    return at_;
  };
  w.kofs = take(4 * (N + 1));
  w.kofs_t = take(4 * 2);
  w.dg = take(4 * R);
  w.dz = take(4 * T * N);
  w.colpart = take(4 * (size_t)moe::colsum_chunks((int)T) * N);
  w.dzb = take(es * T * w.Np);
  // fp32 pre-activations (the shared expert's right after the routed rows
  // when one launch computes both) and v
  const bool merge = shared_in_routed(s);
  w.gu = take(4 * (R + (merge ? T : 0)) * 2 * dff);
  w.v = take(4 * R * dff);
  w.dgu = take(es * R * 2 * dff);
  w.dgpart = take(4 * R * (size_t)moe::swiglu_bwd_t_tiles((int)dff));
  w.gus = merge ? w.gu + 4 * R * 2 * dff : take(4 * T * 2 * dfs);
  w.vs = take(4 * T * dfs);
  w.dgus = take(es * T * 2 * dfs);
  w.acts = take(es * T * dfs);
  const bool nn = bwd_nn(s), nn_sh = bwd_nn_shared(s);
  w.wdT = take(nn ? 0 : es * N * dff * d);
  w.wguT = take(nn ? 0 : es * N * d * 2 * dff);
  w.sdT = take(nn_sh ? 0 : es * dfs * d);
  w.sguT = take(nn_sh ? 0 : es * d * 2 * dfs);
  w.wrT = take(es * d * w.Np);
  w.dhr = take(es * R * d);
  w.dhs = take(es * T * d);
  w.dhrt = take(es * T * d);
  w.ta = take(es * w.ta_rows * w.Rp);
  w.tb = take(es * w.tb_rows * w.Rp);
  w.tc = take(es * d * w.Rp);
  w.part_floats = 0;
  if (s->dtype == MOE_BF16) {
    int64_t f = std::max(moe::split_part_floats(R, s->N, s->d_ff, true),
                         moe::split_part_floats(R, s->N, s->d, false));
    f = std::max(f, moe::split_part_floats(R, s->N, s->d_ff, false));
    f = std::max(f, moe::split_part_floats(T, 1, s->d, false));
    if (dfs)
      f = std::max(f, std::max(moe::split_part_floats(T, 1, s->d_ff_shared, true),
                               moe::split_part_floats(T, 1, s->d_ff_shared, false)));
    w.part_floats = f;
  }
  w.part = take(sizeof(float) * (size_t)w.part_floats);
  w.cnt = take(w.part_floats ? sizeof(int32_t) * moe::kSplitCounters : 0);
  w.end = o;
  return w;
}

moe_status check_bwd_limits(const moe_shape* s) {
  const BwdWs w = bwd_ws(s);
  const int64_t es = (int64_t)esize(s);
  const int64_t lim2g = 2147483647LL;
  if (w.ta_rows * w.Rp * es > lim2g || w.tb_rows * w.Rp * es > lim2g ||
      (int64_t)s->T * s->k * 2 * s->d_ff * es > lim2g ||
      (int64_t)s->d * 2 * std::max(s->d_ff, s->d_ff_shared) * es > lim2g)
    return fail(MOE_ERR_UNSUPPORTED, "a backward operand exceeds 2^31 bytes");
  return MOE_OK;
}

moe_status backward_impl(const moe_shape* s, const void* h, const void* w_router,
                         const float* b_router, const void* w_gate, const void* w_up,
                         const void* w_down, const void* sh_gate, const void* sh_up,
                         const void* sh_down, const int32_t* ids, const float* gates,
                         const int32_t* counts, const int32_t* offsets, const int32_t* perm,
                         const int32_t* row_of, const float* preact, const void* dy,
                         float d_laux, float d_zloss, void* dh, float* dw_router,
                         float* db_router, void* dw_gate, void* dw_up, void* dw_down,
                         void* dsh_gate, void* dsh_up, void* dsh_down, float* dgates, void* ws,
                         const BwdWs& W, hipStream_t st) {
  const int T = s->T, N = s->N, k = s->k, d = s->d, dff = s->d_ff, dfs = s->d_ff_shared;
  const int R = T * k;
  const bool bf16 = s->dtype == MOE_BF16;
  const int b = bf16 ? 1 : 0;
  const size_t es = esize(s);
  const int ncu = bf16 ? num_cu() : 0;
  const int C = expert_capacity(s);
  const int rows_all = C ? (int)std::min<int64_t>(R, (int64_t)N * C) : R;
  const int rows_max = bwd_rows_max(s);
  const bool nn = bwd_nn(s), nn_sh = bwd_nn_shared(s);
  const int Rp = (int)W.Rp, Tp = (int)W.Tp, Np = (int)W.Np;
  float* part = W.part_floats ? at<float>(ws, W.part) : nullptr;
  int32_t* cnt = W.part_floats ? at<int32_t>(ws, W.cnt) : nullptr;
  // the forward's pre-activations when it kept them, else recomputed here
  float* gu = preact ? const_cast<float*>(preact) : at<float>(ws, W.gu);
  float* v = at<float>(ws, W.v);
  char* dgu = at<char>(ws, W.dgu);
  float* dgpart = at<float>(ws, W.dgpart);
  float* gus = preact ? const_cast<float*>(preact) + (int64_t)R * 2 * dff : at<float>(ws, W.gus);
  float* vs = at<float>(ws, W.vs);
  char* dgus = at<char>(ws, W.dgus);
  char* acts = at<char>(ws, W.acts);
  char* wdT = at<char>(ws, W.wdT);
  char* wguT = at<char>(ws, W.wguT);
  char* sdT = at<char>(ws, W.sdT);
  char* sguT = at<char>(ws, W.sguT);
  char* wrT = at<char>(ws, W.wrT);
  char* dhr = at<char>(ws, W.dhr);
  char* dhs = at<char>(ws, W.dhs);
  char* dhrt = at<char>(ws, W.dhrt);
  char* ta = at<char>(ws, W.ta);
  char* tb = at<char>(ws, W.tb);
  char* tc = at<char>(ws, W.tc);
  int32_t* kofs = at<int32_t>(ws, W.kofs);
  int32_t* kofs_t = at<int32_t>(ws, W.kofs_t);
  float* dg = at<float>(ws, W.dg);
  float* dz = at<float>(ws, W.dz);
  char* dzb = at<char>(ws, W.dzb);
  // kind 0: gate/up pre-activations (fp32 out); 1: plain product, fp32 out;
  // 2: plain product in the layer dtype
  auto grouped = [&](const moe::GroupedProblem& p, int kind, const char* what) -> moe_status {
    hipError_t e;
    if (bf16)
      e = kind == 0 ? moe::launch_gateup_preact_bf16(p, ncu, st)
          : kind == 1 ? moe::launch_down_f32out_bf16(p, ncu, st)
                      : moe::launch_down_bf16(p, ncu, st);
    else
      e = kind == 0 ? moe::launch_gateup_preact_f32(p, st) : moe::launch_down_f32(p, st);
    return hip_check(e, what);
  };
  // B in its own [K, N] layout (bf16, more than 64 rows per group)
  auto grouped_nn = [&](const moe::GroupedProblem& p, bool f32out,
                        const char* what) -> moe_status {
    return hip_check(f32out ? moe::launch_down_nn_f32out_bf16(p, ncu, st)
                            : moe::launch_down_nn_bf16(p, ncu, st),
                     what);
  };
  auto kgroup = [&](const void* A, int lda, int64_t a_rows, const void* B, int ldb,
                    int64_t b_rows, const int32_t* ko, int G, int M, int Ncols, void* Cout,
                    int64_t gstride, int ldc, bool f32out, const char* what) -> moe_status {
    if (bf16)
      return hip_check(moe::launch_kgroup_bf16(A, lda, a_rows, B, ldb, b_rows, ko, G, M, Ncols,
                                               Cout, gstride, ldc, f32out, ncu, st), what);
    return hip_check(moe::launch_kgroup_f32(static_cast<const float*>(A), lda,
                                            static_cast<const float*>(B), ldb, ko, G, M, Ncols,
                                            static_cast<float*>(Cout), gstride, ldc, st), what);
  };
  auto pack = [&](const void* src, int ld_src, int ncols, const int32_t* pm, int kdiv,
                  const float* scale, const int32_t* offs, const int32_t* ko, int G,
                  int n_single, int64_t p_limit, void* dst, int64_t ld_dst, int batch,
                  int64_t sb, int64_t db, const char* what) -> moe_status {
    return hip_check(moe::launch_pack_t(src, ld_src, ncols, pm, kdiv, scale, offs, ko, G,
                                        n_single, p_limit, dst, ld_dst, b, st, batch, sb, db),
                     what);
  };

  // 1. router logits again (split-K slices, as in the forward)
  float* z_part = at<float>(ws, W.r.z);
  int splits = 1;
  TRY(router_logits(s, h, w_router, z_part, splits, st));
  // 2. gate/up pre-activations of the kept rows (and the shared expert),
  //    unless the forward kept them
  if (!preact) {
    // the forward's launches: the shared expert's rows (at R + t, gus) in
    // the routed launch when it ran there
    moe::GroupedProblem pg{h, d, perm, k, offsets, N, rows_all, rows_max, w_gate, w_up,
                           (int64_t)dff * d, d, dff, d, gu, 2 * dff, 0,
                           (uint32_t)(es * T * d), part, cnt, W.part_floats};
    const bool merge = shared_in_routed(s);
    if (merge) {
      pg.X0 = sh_gate;
      pg.X1 = sh_up;
      pg.x_rows = T;
      pg.x_a_row0 = 0;
      pg.x_c_row0 = R;
    }
    TRY(grouped(pg, 0, "gate/up recompute"));
    if (dfs && !merge)
      TRY(grouped(moe::GroupedProblem{h, d, nullptr, 1, nullptr, 1, T, T, sh_gate, sh_up, 0, d,
                                      dfs, d, gus, 2 * dfs, 0, (uint32_t)(es * T * d), part,
                                      cnt, W.part_floats},
                  0, "shared gate/up recompute"));
  }
  // 3. v = W_down^T dy per kept row: W_down as it is ([d, d_ff] per expert,
  //    K = d), or transposed to [d_ff, d] for the weight-streaming kernels
  if (nn) {
    TRY(grouped_nn(moe::GroupedProblem{dy, d, perm, k, offsets, N, rows_all, rows_max, w_down,
                                       nullptr, (int64_t)d * dff, dff, dff, d, v, dff, 0,
                                       (uint32_t)(es * T * d), part, cnt, W.part_floats, nullptr,
                                       0, 0},
                   true, "v GEMM"));
  } else {
    TRY(pack(w_down, dff, dff, nullptr, 1, nullptr, nullptr, nullptr, 0, d, d, wdT, d, N,
             (int64_t)d * dff, (int64_t)dff * d, "W_down transpose"));
    TRY(grouped(moe::GroupedProblem{dy, d, perm, k, offsets, N, rows_all, rows_max, wdT, nullptr,
                                    (int64_t)dff * d, d, dff, d, v, dff, 0,
                                    (uint32_t)(es * T * d), part, cnt, W.part_floats},
                1, "v GEMM"));
  }
  if (dfs && nn_sh) {
    TRY(grouped_nn(moe::GroupedProblem{dy, d, nullptr, 1, nullptr, 1, T, T, sh_down, nullptr, 0,
                                       dfs, dfs, d, vs, dfs, 0, (uint32_t)(es * T * d), part, cnt,
                                       W.part_floats, nullptr, 0, 0},
                   true, "shared v GEMM"));
  } else if (dfs) {
    TRY(pack(sh_down, dfs, dfs, nullptr, 1, nullptr, nullptr, nullptr, 0, d, d, sdT, d, 1, 0, 0,
             "shared W_down transpose"));
    TRY(grouped(moe::GroupedProblem{dy, d, nullptr, 1, nullptr, 1, T, T, sdT, nullptr, 0, d, dfs,
                                    d, vs, dfs, 0, (uint32_t)(es * T * d), part, cnt,
                                    W.part_floats},
                1, "shared v GEMM"));
  }
  // 4. SwiGLU backward: [dgp | du] row-major for the h-row GEMM, act^T and
  //    [dgp | du]^T in the weight-gradient GEMMs' padded K ranges (kofs),
  //    dg per slot
  TRY(hip_check(moe::launch_kofs(offsets, N, 0, kofs, st), "K ranges"));
  TRY(hip_check(moe::launch_swiglu_bwd_t(gu, v, dgu, tb, ta, Rp, perm, gates, offsets, kofs, N,
                                         Rp, rows_all, dff, dgpart, dg, b, st),
                "SwiGLU backward"));
  if (dfs)
    TRY(hip_check(moe::launch_swiglu_bwd(gus, vs, acts, dgus, nullptr, nullptr, nullptr, nullptr,
                                         0, T, dfs, b, st), "shared SwiGLU backward"));
  // 5. router-logit gradient, b_r gradient
  TRY(hip_check(moe::launch_route_bwd(z_part, splits, b_router, ids, gates, dg, row_of, counts, T,
                                      N, k, s->mode, s->aux_alpha, d_laux, d_zloss, dz, dzb, Np,
                                      b, dgates, st), "router backward"));
  if (db_router)
    TRY(hip_check(moe::launch_colsum(dz, T, N, at<float>(ws, W.colpart), db_router, st),
                  "b_r gradient"));
  // 6. row gradients of h: [W_gate; W_up]^T [dgp | du] per kept row (K =
  //    2 d_ff: W_gate's rows, then W_up's), the shared expert's, and the
  //    router's dz W_r
  if (nn) {
    TRY(grouped_nn(moe::GroupedProblem{dgu, 2 * dff, nullptr, 1, offsets, N, rows_all, rows_max,
                                       w_gate, w_up, (int64_t)dff * d, d, d, 2 * dff, dhr, d, 0,
                                       (uint32_t)(es * R * 2 * dff), part, cnt, W.part_floats,
                                       nullptr, 0, dff},
                   false, "dh rows GEMM"));
  } else {
    TRY(pack(w_gate, d, d, nullptr, 1, nullptr, nullptr, nullptr, 0, dff, dff, wguT, 2 * dff, N,
             (int64_t)dff * d, (int64_t)d * 2 * dff, "W_gate transpose"));
    TRY(pack(w_up, d, d, nullptr, 1, nullptr, nullptr, nullptr, 0, dff, dff, wguT + es * dff,
             2 * dff, N, (int64_t)dff * d, (int64_t)d * 2 * dff, "W_up transpose"));
    TRY(grouped(moe::GroupedProblem{dgu, 2 * dff, nullptr, 1, offsets, N, rows_all, rows_max,
                                    wguT, nullptr, (int64_t)d * 2 * dff, 2 * dff, d, 2 * dff, dhr,
                                    d, 0, (uint32_t)(es * R * 2 * dff), part, cnt,
                                    W.part_floats},
                2, "dh rows GEMM"));
  }
  if (dfs && nn_sh) {
    TRY(grouped_nn(moe::GroupedProblem{dgus, 2 * dfs, nullptr, 1, nullptr, 1, T, T, sh_gate, sh_up,
                                       0, d, d, 2 * dfs, dhs, d, 0, (uint32_t)(es * T * 2 * dfs),
                                       part, cnt, W.part_floats, nullptr, 0, dfs},
                   false, "shared dh GEMM"));
  } else if (dfs) {
    TRY(pack(sh_gate, d, d, nullptr, 1, nullptr, nullptr, nullptr, 0, dfs, dfs, sguT, 2 * dfs, 1,
             0, 0, "shared W_gate transpose"));
    TRY(pack(sh_up, d, d, nullptr, 1, nullptr, nullptr, nullptr, 0, dfs, dfs, sguT + es * dfs,
             2 * dfs, 1, 0, 0, "shared W_up transpose"));
    TRY(grouped(moe::GroupedProblem{dgus, 2 * dfs, nullptr, 1, nullptr, 1, T, T, sguT, nullptr, 0,
                                    2 * dfs, d, 2 * dfs, dhs, d, 0, (uint32_t)(es * T * 2 * dfs),
                                    part, cnt, W.part_floats},
                2, "shared dh GEMM"));
  }
  // the router's term dz W_r: for a few experts inside the combine (N fp32
  // products per element), else a GEMM over the padded dz
  const bool router_in_combine = N <= moe::kMaxRouterFused;
  if (!router_in_combine) {
    TRY(pack(w_router, d, d, nullptr, 1, nullptr, nullptr, nullptr, 0, N, Np, wrT, Np, 1, 0, 0,
             "W_r transpose"));
    TRY(grouped(moe::GroupedProblem{dzb, Np, nullptr, 1, nullptr, 1, T, T, wrT, nullptr, 0, Np,
                                    d, Np, dhrt, d, 0, (uint32_t)(es * T * Np), part, cnt,
                                    W.part_floats},
                2, "router dh GEMM"));
  }
  TRY(hip_check(moe::launch_dh_combine(dhr, row_of, dfs ? dhs : nullptr,
                                       router_in_combine ? nullptr : dhrt,
                                       router_in_combine ? dz : nullptr, w_router, N, dh, T, k,
                                       d, b, st),
                "dh combine"));
  // 7. expert weight gradients over each expert's kept rows (padded K
  //    ranges): act^T (tb) and [dgp | du]^T (ta) from step 4
  TRY(pack(dy, d, d, perm, k, gates, offsets, kofs, N, 0, Rp, tc, Rp, 1, 0, 0, "dOut transpose"));
  TRY(kgroup(tc, Rp, d, tb, Rp, dff, kofs, N, d, dff, dw_down, (int64_t)d * dff, dff, false,
             "W_down gradient"));
  TRY(pack(h, d, d, perm, k, nullptr, offsets, kofs, N, 0, Rp, tb, Rp, 1, 0, 0, "h transpose"));
  TRY(kgroup(ta, Rp, 2 * dff, tb, Rp, d, kofs, N, dff, d, dw_gate, (int64_t)dff * d, d, false,
             "W_gate gradient"));
  TRY(kgroup(ta + es * (size_t)dff * Rp, Rp, dff, tb, Rp, d, kofs, N, dff, d, dw_up,
             (int64_t)dff * d, d, false, "W_up gradient"));
  // 8. shared-expert and router weight gradients over all tokens
  TRY(hip_check(moe::launch_kofs(nullptr, 1, T, kofs_t, st), "token K range"));
  if (dfs) {
    TRY(pack(dy, d, d, nullptr, 1, nullptr, nullptr, nullptr, 0, T, Tp, ta, Tp, 1, 0, 0,
             "shared dOut transpose"));
    TRY(pack(acts, dfs, dfs, nullptr, 1, nullptr, nullptr, nullptr, 0, T, Tp, tb, Tp, 1, 0, 0,
             "shared act transpose"));
    TRY(kgroup(ta, Tp, d, tb, Tp, dfs, kofs_t, 1, d, dfs, dsh_down, 0, dfs, false,
               "shared W_down gradient"));
    TRY(pack(dgus, 2 * dfs, 2 * dfs, nullptr, 1, nullptr, nullptr, nullptr, 0, T, Tp, ta, Tp, 1,
             0, 0, "shared dgu transpose"));
  }
  TRY(pack(h, d, d, nullptr, 1, nullptr, nullptr, nullptr, 0, T, Tp, tb, Tp, 1, 0, 0,
           "h transpose (all tokens)"));
  if (dfs) {
    TRY(kgroup(ta, Tp, 2 * dfs, tb, Tp, d, kofs_t, 1, dfs, d, dsh_gate, 0, d, false,
               "shared W_gate gradient"));
    TRY(kgroup(ta + es * (size_t)dfs * Tp, Tp, dfs, tb, Tp, d, kofs_t, 1, dfs, d, dsh_up, 0, d,
               false, "shared W_up gradient"));
  }
  TRY(pack(dzb, Np, N, nullptr, 1, nullptr, nullptr, nullptr, 0, T, Tp, ta, Tp, 1, 0, 0,
           "dz transpose"));
  TRY(kgroup(ta, Tp, N, tb, Tp, d, kofs_t, 1, N, d, dw_router, 0, d, true, "W_r gradient"));
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_err.c_str(); }

size_t moe_workspace_bytes(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return 0;
  return fused_ws(s).end;
}

moe_status moe_route(const moe_shape* s, const void* h, const void* w_router,
                     const float* b_router, const float* b_select, int32_t* topk_ids,
                     float* topk_gates, float* p_mean, float* z_loss, float* entropy, void* ws,
                     size_t ws_bytes, void* stream) {
  g_err.clear();
  TRY(check_shape(s));
  TRY(need16(h, "h"));
  TRY(need16(w_router, "w_router"));
  TRY(check_bias(s, b_router, b_select));
  TRY(need4(topk_ids, "topk_ids"));
  TRY(need4(topk_gates, "topk_gates"));
  TRY(opt4(p_mean, "p_mean"));
  TRY(opt4(z_loss, "z_loss"));
  TRY(opt4(entropy, "entropy"));
  const RouteWs L = route_ws(s, 0);
  TRY(check_ws(ws, ws_bytes, L.end));
  if (s->T == 0) return MOE_OK;
  return route_impl(s, h, w_router, b_router, b_select, topk_ids, topk_gates, p_mean, z_loss,
                    entropy, L, ws, static_cast<hipStream_t>(stream));
}

moe_status moe_dispatch(const moe_shape* s, const int32_t* topk_ids, int32_t* counts,
                        int32_t* offsets, int32_t* perm_src, int32_t* row_of,
                        const float* p_mean, float* f_out, float* l_aux, float* cap_stats,
                        void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  TRY(check_shape(s));
  TRY(need4(topk_ids, "topk_ids"));
  TRY(need4(counts, "counts"));
  TRY(need4(offsets, "offsets"));
  TRY(need4(perm_src, "perm_src"));
  TRY(need4(row_of, "row_of"));
  TRY(opt4(p_mean, "p_mean"));
  TRY(opt4(f_out, "f_out"));
  TRY(opt4(l_aux, "l_aux"));
  TRY(opt4(cap_stats, "cap_stats"));
  if (l_aux && !p_mean) return fail(MOE_ERR_INVALID_ARG, "l_aux requested without p_mean");
  TRY(check_ws(ws, ws_bytes, dispatch_ws_bytes(s)));
  if (s->T == 0) return MOE_OK;
  return dispatch_impl(s, topk_ids, counts, offsets, perm_src, row_of, p_mean, f_out, l_aux,
                       cap_stats, static_cast<int32_t*>(ws), static_cast<hipStream_t>(stream));
}

moe_status moe_expert_ffn(const moe_shape* s, const void* h, const int32_t* perm_src,
                          const int32_t* offsets, const void* w_gate, const void* w_up,
                          const void* w_down, const void* sh_gate, const void* sh_up,
                          const void* sh_down, void* out_rows, void* ws, size_t ws_bytes,
                          void* stream) {
  g_err.clear();
  TRY(check_shape(s));
  TRY(need16(h, "h"));
  TRY(need4(perm_src, "perm_src"));
  TRY(need4(offsets, "offsets"));
  TRY(need16(w_gate, "w_gate"));
  TRY(need16(w_up, "w_up"));
  TRY(need16(w_down, "w_down"));
  TRY(check_shared(s, sh_gate, sh_up, sh_down));
  TRY(need16(out_rows, "out_rows"));
  const FfnWs W = ffn_ws(s, 0);
  TRY(check_ws(ws, ws_bytes, W.end));
  if (s->T == 0) return MOE_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  TRY(ffn_stage(s, true, h, perm_src, offsets, w_gate, w_up, w_down, sh_gate, sh_up, sh_down,
                out_rows, ws, W, st));
  return ffn_stage(s, false, h, perm_src, offsets, w_gate, w_up, w_down, sh_gate, sh_up, sh_down,
                   out_rows, ws, W, st);
}

moe_status moe_combine(const moe_shape* s, const void* out_rows, const int32_t* row_of,
                       const float* topk_gates, void* y, void* stream) {
  g_err.clear();
  TRY(check_shape(s));
  TRY(need16(out_rows, "out_rows"));
  TRY(need4(row_of, "row_of"));
  TRY(need4(topk_gates, "topk_gates"));
  TRY(need16(y, "y"));
  if (s->T == 0) return MOE_OK;
  return combine_impl(s, out_rows, row_of, topk_gates, y, static_cast<hipStream_t>(stream));
}

size_t moe_backward_workspace_bytes(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return 0;
  return bwd_ws(s).end;
}

moe_status moe_layer_backward(const moe_shape* s, const void* h, const void* w_router,
                              const float* b_router, const void* w_gate, const void* w_up,
                              const void* w_down, const void* sh_gate, const void* sh_up,
                              const void* sh_down, const int32_t* topk_ids,
                              const float* topk_gates, const int32_t* counts,
                              const int32_t* offsets, const int32_t* perm_src,
                              const int32_t* row_of, const float* preact, const void* dy,
                              float d_laux, float d_zloss, void* dh, float* dw_router,
                              float* db_router,
                              void* dw_gate, void* dw_up, void* dw_down, void* dsh_gate,
                              void* dsh_up, void* dsh_down, float* dgates, void* ws,
                              size_t ws_bytes, void* stream) {
  g_err.clear();
  TRY(check_shape(s));
  TRY(need16(h, "h"));
  TRY(need16(w_router, "w_router"));
  TRY(opt4(b_router, "b_router"));
  TRY(need16(w_gate, "w_gate"));
  TRY(need16(w_up, "w_up"));
  TRY(need16(w_down, "w_down"));
  TRY(check_shared(s, sh_gate, sh_up, sh_down));
  TRY(need4(topk_ids, "topk_ids"));
  TRY(need4(topk_gates, "topk_gates"));
  TRY(need4(counts, "counts"));
  TRY(need4(offsets, "offsets"));
  TRY(need4(perm_src, "perm_src"));
  TRY(need4(row_of, "row_of"));
  TRY(opt4(preact, "preact"));
  TRY(need16(dy, "dy"));
  TRY(need16(dh, "dh"));
  TRY(need4(dw_router, "dw_router"));
  TRY(opt4(db_router, "db_router"));
  TRY(need16(dw_gate, "dw_gate"));
  TRY(need16(dw_up, "dw_up"));
  TRY(need16(dw_down, "dw_down"));
  if (s->d_ff_shared) {
    TRY(need16(dsh_gate, "dsh_gate"));
    TRY(need16(dsh_up, "dsh_up"));
    TRY(need16(dsh_down, "dsh_down"));
  } else if (dsh_gate || dsh_up || dsh_down) {
    return fail(MOE_ERR_INVALID_ARG, "shared-expert gradients given but d_ff_shared = 0");
  }
  TRY(opt4(dgates, "dgates"));
  if (!std::isfinite(d_laux) || !std::isfinite(d_zloss))
    return fail(MOE_ERR_INVALID_ARG, "d_laux and d_zloss must be finite");
  TRY(check_bwd_limits(s));
  const BwdWs W = bwd_ws(s);
  TRY(check_ws(ws, ws_bytes, W.end));
  if (s->T == 0) return MOE_OK;
  return backward_impl(s, h, w_router, b_router, w_gate, w_up, w_down, sh_gate, sh_up, sh_down,
                       topk_ids, topk_gates, counts, offsets, perm_src, row_of, preact, dy, d_laux,
                       d_zloss, dh, dw_router, db_router, dw_gate, dw_up, dw_down, dsh_gate,
                       dsh_up, dsh_down, dgates, ws, W, static_cast<hipStream_t>(stream));
}

moe_status moe_layer_fused(const moe_shape* s, const void* h, const void* w_router,
                           const float* b_router, const float* b_select, const void* w_gate,
                           const void* w_up, const void* w_down, const void* sh_gate,
                           const void* sh_up, const void* sh_down, void* y, int32_t* topk_ids,
                           float* topk_gates, int32_t* counts, float* f_out, float* p_out,
                           float* l_aux, float* z_loss, float* entropy, float* cap_stats,
                           void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  return layer_impl(s, h, w_router, b_router, b_select, w_gate, w_up, w_down, sh_gate, sh_up,
                    sh_down, y, topk_ids, topk_gates, counts, f_out, p_out, l_aux, z_loss,
                    entropy, cap_stats, ws, ws_bytes, stream, nullptr);
}

moe_status moe_layer_fused_noalloc(const moe_shape* s, const void* h, const void* w_router,
                                   const float* b_router, const float* b_select,
                                   const void* w_gate, const void* w_up, const void* w_down,
                                   const void* sh_gate, const void* sh_up, const void* sh_down,
                                   void* y, int32_t* topk_ids, float* topk_gates,
                                   int32_t* counts, float* f_out, float* p_out, float* l_aux,
                                   float* z_loss, float* entropy, float* cap_stats,
                                   void* stream) {
  g_err.clear();
  return layer_impl(s, h, w_router, b_router, b_select, w_gate, w_up, w_down, sh_gate, sh_up,
                    sh_down, y, topk_ids, topk_gates, counts, f_out, p_out, l_aux, z_loss,
                    entropy, cap_stats, nullptr, 0, stream, nullptr,
                    TrainOut{nullptr, nullptr, nullptr, nullptr}, true);
}

moe_status moe_layer_forward_train(const moe_shape* s, const void* h, const void* w_router,
                                   const float* b_router, const float* b_select,
                                   const void* w_gate, const void* w_up, const void* w_down,
                                   const void* sh_gate, const void* sh_up, const void* sh_down,
                                   void* y, int32_t* topk_ids, float* topk_gates,
                                   int32_t* counts, int32_t* offsets, int32_t* perm_src,
                                   int32_t* row_of, float* preact, float* p_out, float* l_aux,
                                   float* z_loss, float* entropy, void* ws, size_t ws_bytes,
                                   void* stream) {
  g_err.clear();
  TRY(need4(topk_ids, "topk_ids"));
  TRY(need4(topk_gates, "topk_gates"));
  TRY(need4(counts, "counts"));
  TRY(need4(offsets, "offsets"));
  TRY(need4(perm_src, "perm_src"));
  TRY(need4(row_of, "row_of"));
  return layer_impl(s, h, w_router, b_router, b_select, w_gate, w_up, w_down, sh_gate, sh_up,
                    sh_down, y, topk_ids, topk_gates, counts, nullptr, p_out, l_aux, z_loss,
                    entropy, nullptr, ws, ws_bytes, stream, nullptr,
                    TrainOut{offsets, perm_src, row_of, preact});
}

moe_status moe_layer_fused_marked(const moe_shape* s, const void* h, const void* w_router,
                                  const float* b_router, const float* b_select,
                                  const void* w_gate, const void* w_up, const void* w_down,
                                  const void* sh_gate, const void* sh_up, const void* sh_down,
                                  void* y, int32_t* topk_ids, float* topk_gates,
                                  int32_t* counts, float* f_out, float* p_out, float* l_aux,
                                  float* z_loss, float* entropy, float* cap_stats, void* ws,
                                  size_t ws_bytes, void* stream, void* const* events) {
  g_err.clear();
  if (!events) return fail(MOE_ERR_INVALID_ARG, "events is NULL");
  return layer_impl(s, h, w_router, b_router, b_select, w_gate, w_up, w_down, sh_gate, sh_up,
                    sh_down, y, topk_ids, topk_gates, counts, f_out, p_out, l_aux, z_loss,
                    entropy, cap_stats, ws, ws_bytes, stream, events);
}

}  // extern "C"
