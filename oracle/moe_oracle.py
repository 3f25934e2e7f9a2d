"""Plain float64 CPU oracle for the forward pass of one sparse MoE FFN layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the tests, the smoke check of the graft entry point
and the benchmark's CPU-baseline leg use it. It shares no code with the HIP
library (no kernels, headers, tables or helpers) and imports nothing from it.

Every step is the plain definition the pages give, in their order and
notation, with numpy as the only primitive (matrix products, exp, a sort):

  1. router logits  z_t = W_r h_t + b_r
     [page "MOE 专家选择与路由机制" (wuhy-notes), §二 第一步;
      page "MoE：router 怎样选 expert" (cooking-agi), first section]
  2. scores: softmax p_t = exp(z_t) / sum_j exp(z_tj)            [§二 第二步]
     or sigmoid s_t = 1/(1+exp(-z_t)) (DeepSeek-V3 style)
     [cooking-agi, first section, the remark after the gate formula]
  3. top-k selection S_t = TopK(score_t, k)                      [§二 第三步]
     optionally over group-limited candidates: the best groups of experts
     by the sum of their top-m scores first, the rest masked to -inf
     [cooking-agi, section on choosing groups first across devices]
  4. gates, three modes
     A  g_i = p_i / sum_{j in S} p_j  (= softmax over the selected logits)
        [wuhy-notes §二 第三步 gate formula; cooking-agi first section]
     B  g_i = p_i, the full-softmax probability, no renormalisation
        (Switch top-1; the route() snippet keeps top_probs for any k)
        [cooking-agi first section, Switch remark; page pwwt.cn §2.1]
     C  select on s + b_sel, g_i = s_i / sum_{j in S} s_j with the unbiased s
        [cooking-agi first section; page "拆解 MoE：单个 Token 如何经过专家层"
         (feinterview), load-balance section: where the bias acts is left to
         the implementation; read here as selection only]
  5. dispatch: stable regroup of the (token, slot) pairs by expert
     [wuhy-notes §三 "Token Dispatch" table and bucket listing;
      page "【大模型】MoE（专家混合模型）简介" (horizon.auto) §3 ② Dispatch]
     optionally with an expert capacity C = ceil(factor * T k / N): each
     expert keeps its first C slots in token order, later ones are dropped
     [wuhy-notes §六 Expert Capacity]; usage and drop fraction are reported
  6. experts: E_i(h) = W_down^(i) (SiLU(W_gate^(i) h) * W_up^(i) h)
     [wuhy-notes §一, SwiGLU FFN and expert formulas]
     shared expert: added to every token with weight 1  [wuhy-notes §八]
  7. combine: y_t = sum_{i in S_t} g_ti E_i(h_t) (+ shared) -- a sum, never
     an overwrite [cooking-agi "选好以后，token 怎么过去，输出怎么回来？";
     horizon.auto §3 ④ Gather]
  8. load statistics f_i, p_i and L_aux = alpha * N * sum_i f_i p_i
     [feinterview, load-balance section; wuhy-notes §五 (garbled print)];
     router z-loss (mean squared log-sum-exp of the logits) and the mean
     routing entropy [wuhy-notes §五 and its monitoring list]
  9. dense brute force: every expert on every token, unselected gates zero
     [cooking-agi "怎么知道实现没把梯度弄丢？"]
 10. backward: gradients of <dy, y> (+ weighted L_aux and z-loss) for the
     forward pass's fixed selection; the router learns through the selected
     gate values (and the full-softmax denominator in mode B)
     [cooking-agi "top-k 不可导，router 怎么学"; wuhy-notes "Top-k 不可导，
      为什么 Router 还能学" and the total-loss paragraph]

Readings where the pages are silent or garbled (each is listed in the design
notes): ties in top-k go to the lower expert index; f_i = count_i / (T k);
p_i in mode C averages s_ti / sum_j s_tj; the shared expert is ungated; the
router bias is optional; SiLU(x) = x * sigmoid(x); expert linears have no
bias; the layer output excludes the residual; with a capacity, slots past C
are dropped in token order (latest first), contribute nothing to y and still
count in f_i (f_i is the routing decision, not what was computed).

Parity pins: every function here is pinned in tests/test_oracle_pins.py
against the pages' worked examples, closed forms, brute force or library
routines; tests/test_oracle_mutations.py plants plausible mistakes and shows
a pin catches each.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Callable, Optional, Sequence

import numpy as np

MODE_SOFTMAX_RENORM = 0
MODE_SOFTMAX_FULL = 1
MODE_SIGMOID_BIAS_RENORM = 2

F64 = np.float64


def _f64(a):
    return None if a is None else np.asarray(a, dtype=F64)


# ----------------------------------------------------------- 1. router logits
def router_logits(h, w_router, b_router=None):
    """z[t, i] = sum_c W_r[i, c] h[t, c] + b_r[i]; W_r is [N, d] (one row per
    expert), h is [T, d]. The bias is optional (two of the pages omit it)."""
    z = _f64(h) @ _f64(w_router).T
    if b_router is not None:
        z = z + _f64(b_router)[None, :]
    return z


# ------------------------------------------------------------------ 2. scores
def softmax(z):
    """p[t, i] = exp(z[t, i]) / sum_j exp(z[t, j]), evaluated as
    exp(z - max) / sum exp(z - max) (same value, no overflow)."""
    z = _f64(z)
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def sigmoid(z):
    """s = 1 / (1 + exp(-z))."""
    return 1.0 / (1.0 + np.exp(-_f64(z)))


# ------------------------------------------------------------------- 3. top-k
def topk(sel, k):
    """Top-k of each row of ``sel`` [T, N].

    Experts are ordered by selection score descending, ties broken by the
    lower expert index; the first k are the slots 0..k-1. Also returns the
    gap between the k-th and (k+1)-th scores (+inf when k == N), used to
    flag near-ties.
    """
    sel = _f64(sel)
    T, N = sel.shape
    if not 1 <= k <= N:
        raise ValueError(f"need 1 <= k <= N, got k={k}, N={N}")
    idx = np.broadcast_to(np.arange(N), sel.shape)
    order = np.lexsort((idx, -sel), axis=-1)          # primary key: -score
    ids = order[:, :k].astype(np.int64)
    srt = np.take_along_axis(sel, order, axis=-1)
    gap = srt[:, k - 1] - srt[:, k] if k < N else np.full(T, np.inf)
    return ids, gap


# ------------------------------------------------- 3b. group-limited top-k
def group_limit(sel, n_groups, topk_groups, topm):
    """Group-limited candidates [cooking-agi, section on choosing groups
    first across devices]: the N experts form n_groups contiguous groups of
    N / n_groups; a group's score is the sum of its topm largest selection
    scores (topm = 1: the group's maximum); the topk_groups best groups (ties
    to the lower group index) keep their experts as candidates and every
    other expert gets -inf, not 0, so that a negative score cannot lose to a
    masked expert. Returns the masked scores and the gap between the
    topk_groups-th and the next group score (+inf when every group is kept)."""
    sel = _f64(sel)
    T, N = sel.shape
    if n_groups < 1 or N % n_groups:
        raise ValueError(f"{N} experts do not split into {n_groups} equal groups")
    gs = N // n_groups
    if not 1 <= topk_groups <= n_groups:
        raise ValueError(f"need 1 <= topk_groups <= n_groups, got {topk_groups}")
    if not 1 <= topm <= gs:
        raise ValueError(f"need 1 <= topm <= group size {gs}, got {topm}")
    per_group = sel.reshape(T, n_groups, gs)
    best_m = -np.sort(-per_group, axis=-1)[:, :, :topm]
    gscore = best_m.sum(axis=-1)                                   # [T, G]
    gids, ggap = topk(gscore, topk_groups)
    keep = np.zeros((T, n_groups), dtype=bool)
    np.put_along_axis(keep, gids, True, axis=-1)
    masked = np.where(np.repeat(keep, gs, axis=1), sel, -np.inf)
    return masked, ggap


@dataclasses.dataclass
class Routing:
    ids: np.ndarray        # [T, k] int64, slot order = descending selection score
    gates: np.ndarray      # [T, k] float64
    z: np.ndarray          # [T, N] logits
    sel: np.ndarray        # [T, N] selection score
    gap: np.ndarray        # [T] k-th minus (k+1)-th selection score
    stat_prob: np.ndarray  # [T, N] per-token probabilities averaged into p_i


# ------------------------------------------------------------------- 4. gates
def _select(sel, k, groups):
    """Top-k of sel, over the group-limited candidates when ``groups`` is
    (n_groups, topk_groups, topm); the near-tie gap is then the smaller of
    the expert and the group gaps."""
    if not groups:
        return topk(sel, k)
    n_groups, topk_groups, topm = groups
    if topk_groups * (sel.shape[1] // n_groups) < k:
        raise ValueError("fewer candidate experts than k in the kept groups")
    masked, ggap = group_limit(sel, n_groups, topk_groups, topm)
    ids, gap = topk(masked, k)
    return ids, np.minimum(gap, ggap)


def route(h, w_router, k, mode, b_router=None, b_select=None, groups=None,
          ids=None) -> Routing:
    """Router logits, scores, top-k selection and gate values (steps 1-4).
    ``groups`` = (n_groups, topk_groups, topm) limits the candidates to the
    best groups first (group_limit); None selects over all experts. ``ids``
    [T, k], when given, replaces the selection (gates and statistics are then
    those of that selection; gap is +inf): the backward pass of another
    implementation's forward is checked for the selection it made."""
    z = router_logits(h, w_router, b_router)
    fixed = ids is not None
    if fixed:
        ids = np.asarray(ids, dtype=np.int64)
        gap = np.full(ids.shape[0], np.inf)
    if mode in (MODE_SOFTMAX_RENORM, MODE_SOFTMAX_FULL):
        p = softmax(z)
        sel = p                       # TopK(p_t, k)
        if not fixed:
            ids, gap = _select(sel, k, groups)
        p_sel = np.take_along_axis(p, ids, axis=-1)
        if mode == MODE_SOFTMAX_RENORM:
            gates = p_sel / p_sel.sum(axis=-1, keepdims=True)
        else:
            gates = p_sel
        stat_prob = p
    elif mode == MODE_SIGMOID_BIAS_RENORM:
        if b_select is None:
            raise ValueError("mode C needs the selection bias")
        s = sigmoid(z)
        sel = s + _f64(b_select)[None, :]
        if not fixed:
            ids, gap = _select(sel, k, groups)
        s_sel = np.take_along_axis(s, ids, axis=-1)   # unbiased scores
        gates = s_sel / s_sel.sum(axis=-1, keepdims=True)
        stat_prob = s / s.sum(axis=-1, keepdims=True)
    else:
        raise ValueError(f"unknown gate mode {mode}")
    return Routing(ids, gates, z, sel, gap, stat_prob)


# ---------------------------------------------------------------- 5. dispatch
@dataclasses.dataclass
class Dispatch:
    counts: np.ndarray    # [N] slots routed to each expert
    offsets: np.ndarray   # [N+1] exclusive prefix of the kept counts
    perm_src: np.ndarray  # [sum kept] bucket row -> flat slot t*k + j
    row_of: np.ndarray    # [T*k] flat slot -> bucket row, -1 if dropped
    kept: np.ndarray      # [N] slots each expert keeps (= counts without a capacity)


def expert_capacity(capacity_factor, T, k, N):
    """C = ceil(capacity_factor * T * k / N) [wuhy-notes §六 Expert Capacity],
    evaluated in double precision on the float32 factor the library gets."""
    return int(math.ceil(float(np.float32(capacity_factor)) * (T * k) / N))


def dispatch(ids, N, capacity=None) -> Dispatch:
    """Group the flat slots f = t*k + j by expert: expert 0's slots first,
    then expert 1's, ...; within one expert in ascending f (token order).
    With a capacity C each expert keeps its first C slots in that order and
    the later ones are dropped (row_of = -1) [wuhy-notes §六: what happens to
    overflow depends on the implementation; here it is dropped]."""
    flat = np.asarray(ids).reshape(-1)
    buckets = [np.nonzero(flat == e)[0] for e in range(N)]
    counts = np.array([len(b) for b in buckets], dtype=np.int64)
    if capacity is not None:
        buckets = [b[:capacity] for b in buckets]
    kept = np.array([len(b) for b in buckets], dtype=np.int64)
    offsets = np.zeros(N + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept)
    perm_src = (np.concatenate(buckets) if buckets else np.zeros(0)).astype(np.int64)
    row_of = np.full(flat.size, -1, dtype=np.int64)
    row_of[perm_src] = np.arange(perm_src.size)
    return Dispatch(counts, offsets, perm_src, row_of, kept)


def capacity_stats(disp: Dispatch, capacity):
    """Capacity usage sum_e kept_e / (N C) and the fraction of routed slots
    dropped [wuhy-notes, monitoring list: expert capacity usage and dropped
    token ratio]."""
    N = disp.counts.size
    routed = int(disp.counts.sum())
    kept = int(disp.kept.sum())
    usage = kept / (N * capacity) if capacity else 0.0
    return usage, ((routed - kept) / routed if routed else 0.0)


# ----------------------------------------------------------------- 6. experts
def silu(x):
    """SiLU(x) = x * sigmoid(x) = x / (1 + exp(-x))."""
    x = _f64(x)
    return x / (1.0 + np.exp(-x))


def expert_ffn(x, w_gate, w_up, w_down):
    """SwiGLU expert on rows x [n, d]: W_down (SiLU(W_gate x) * (W_up x)).
    w_gate, w_up are [d_ff, d]; w_down is [d, d_ff] (out x in)."""
    x = _f64(x)
    g = x @ _f64(w_gate).T
    u = x @ _f64(w_up).T
    return (silu(g) * u) @ _f64(w_down).T


WeightsOf = Callable[[int], Sequence[np.ndarray]]


def weights_getter(w_gate, w_up, w_down) -> WeightsOf:
    """Expert-weight provider over stacked [N, ...] arrays."""
    return lambda e: (w_gate[e], w_up[e], w_down[e])


def expert_rows(h, disp: Dispatch, k, weights_of: WeightsOf,
                shared: Optional[Sequence[np.ndarray]] = None):
    """Rows of expert outputs in bucket order: out[r] = E_e(h[perm_src[r] // k])
    for the expert e whose bucket holds row r; then, with a shared expert,
    out[T*k + t] = E_shared(h[t]). Streams one expert's weights at a time."""
    h = _f64(h)
    T = h.shape[0]
    R = disp.row_of.size                     # T*k: shared rows follow at T*k + t
    out = np.zeros((R + (T if shared is not None else 0), h.shape[1]))
    for e in range(disp.counts.size):
        lo, hi = disp.offsets[e], disp.offsets[e + 1]
        if hi == lo:
            continue
        tok = disp.perm_src[lo:hi] // k
        out[lo:hi] = expert_ffn(h[tok], *weights_of(e))
    if shared is not None:
        out[R:] = expert_ffn(h, *shared)
    return out


# ----------------------------------------------------------------- 7. combine
def combine(out_rows, row_of, gates, has_shared=False):
    """y[t] = out_rows[T*k + t] (shared, weight 1) + sum_j g[t, j] *
    out_rows[row_of[t*k + j]]: every routed contribution is added; a dropped
    slot (row_of = -1) adds nothing."""
    gates = _f64(gates)
    T, k = gates.shape
    out_rows = _f64(out_rows)
    y = np.zeros((T, out_rows.shape[1]))
    if has_shared:
        y += out_rows[T * k:T * k + T]
    rows = np.asarray(row_of).reshape(T, k)
    for j in range(k):
        keep = rows[:, j] >= 0
        y[keep] += gates[keep, j:j + 1] * out_rows[rows[keep, j]]
    return y


# ------------------------------------------------------------------- 8. stats
def load_stats(counts, stat_prob, k, alpha):
    """f_i = count_i / (T k); p_i = mean over tokens of the routing
    probability; L_aux = alpha * N * sum_i f_i p_i."""
    stat_prob = _f64(stat_prob)
    T, N = stat_prob.shape
    f = np.asarray(counts, dtype=F64) / (T * k) if T else np.zeros(N)
    p = stat_prob.mean(axis=0) if T else np.zeros(N)
    l_aux = alpha * N * float(np.sum(f * p))
    return f, p, l_aux


# ------------------------------------------------- router z-loss, entropy
def router_z_loss(z):
    """L_z = (1/T) sum_t (log sum_i exp z_ti)^2: the mean squared
    log-sum-exp of the router logits [wuhy-notes §五 Router z-loss (the
    extracted formula is garbled; this is its plain reading)]."""
    z = _f64(z)
    if z.shape[0] == 0:
        return 0.0
    m = z.max(axis=-1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(z - m).sum(axis=-1))
    return float(np.mean(lse ** 2))


def routing_entropy(stat_prob):
    """Mean over tokens of the entropy -sum_i q_ti log q_ti of the routing
    distribution q_t (the rows that p_i averages: the softmax in modes A/B,
    the normalised sigmoid scores in mode C) [wuhy-notes, monitoring list:
    router probability distribution and routing entropy]."""
    q = _f64(stat_prob)
    if q.shape[0] == 0:
        return 0.0
    with np.errstate(divide="ignore", invalid="ignore"):
        terms = np.where(q > 0, -q * np.log(q), 0.0)
    return float(np.mean(terms.sum(axis=-1)))


# --------------------------------------------------------------- whole layer
@dataclasses.dataclass
class LayerResult:
    routing: Routing
    disp: Dispatch
    out_rows: np.ndarray
    y: np.ndarray
    f: np.ndarray
    p: np.ndarray
    l_aux: float


def layer(h, w_router, k, mode, weights_of: WeightsOf, b_router=None,
          b_select=None, shared=None, alpha=0.01, groups=None,
          capacity_factor=None) -> LayerResult:
    """The whole forward pass, steps 1-8, on all tokens (dropless, or with
    the expert capacity of ``capacity_factor``)."""
    N = np.asarray(w_router).shape[0]
    T = np.asarray(h).shape[0]
    r = route(h, w_router, k, mode, b_router, b_select, groups)
    cap = expert_capacity(capacity_factor, T, k, N) if capacity_factor else None
    disp = dispatch(r.ids, N, cap)
    out_rows = expert_rows(h, disp, k, weights_of, shared)
    y = combine(out_rows, disp.row_of, r.gates, shared is not None)
    f, p, l_aux = load_stats(disp.counts, r.stat_prob, k, alpha)
    return LayerResult(r, disp, out_rows, y, f, p, l_aux)


def layer_tokens(h, routing: Routing, tokens, weights_of: WeightsOf,
                 shared=None, row_of=None):
    """y for a subset of tokens only (without a capacity no step couples two
    tokens), computed one token at a time: for each token, run each of its
    selected experts on its row and add the gated outputs (+ shared). With a
    capacity, pass the dispatch's row_of: dropped slots are skipped."""
    h = _f64(h)
    tokens = np.asarray(tokens, dtype=np.int64)
    y = np.zeros((tokens.size, h.shape[1]))
    k = routing.ids.shape[1]
    need = {}
    for n, t in enumerate(tokens):
        for j, e in enumerate(routing.ids[t]):
            if row_of is not None and row_of[t * k + j] < 0:
                continue
            need.setdefault(int(e), []).append((n, t, j))
    for e, items in sorted(need.items()):
        wg, wu, wd = weights_of(e)
        rows = np.array([t for _, t, _ in items])
        o = expert_ffn(h[rows], wg, wu, wd)
        for m, (n, t, j) in enumerate(items):
            y[n] += routing.gates[t, j] * o[m]
    if shared is not None:
        y += expert_ffn(h[tokens], *shared)
    return y


def dense_layer(h, w_router, k, mode, weights_of: WeightsOf, b_router=None,
                b_select=None, shared=None, groups=None, capacity_factor=None):
    """Brute force: run every expert on every token, build the dense gate
    matrix G (g on the selected experts, 0 elsewhere) and sum G[t,i] E_i(h_t),
    plus the shared expert. With a capacity C, walking the tokens in order,
    an expert's (C+1)-th and later slots get gate 0."""
    h = _f64(h)
    T = h.shape[0]
    N = np.asarray(w_router).shape[0]
    r = route(h, w_router, k, mode, b_router, b_select, groups)
    G = np.zeros((T, N))
    np.put_along_axis(G, r.ids, r.gates, axis=-1)
    if capacity_factor:
        cap = expert_capacity(capacity_factor, T, k, N)
        seen = np.zeros(N, dtype=np.int64)
        for t in range(T):
            for j in range(k):
                e = int(r.ids[t, j])
                seen[e] += 1
                if seen[e] > cap:
                    G[t, e] = 0.0
    y = np.zeros_like(h)
    for e in range(N):
        y += G[:, e:e + 1] * expert_ffn(h, *weights_of(e))
    if shared is not None:
        y += expert_ffn(h, *shared)
    return y


# ------------------------------------------------------------- 10. backward
# Gradients of the layer for an upstream gradient dy of y (and optional
# weights d_laux, d_zloss of the two auxiliary losses added to the training
# objective [wuhy-notes, total-loss paragraph]). The discrete selection and
# the dispatch are held fixed; gradients reach the router only through the
# continuous gate values of the selected experts, and through every logit in
# a normalisation that involves them (the full softmax of mode B)
# [cooking-agi, "top-k 不可导，router 怎么学"; wuhy-notes "Top-k 不可导，为什么
# Router 还能学"]. Written from the chain rule of steps 1-8.

def silu_grad(x):
    """d/dx [x sigmoid(x)] = sigmoid(x) (1 + x (1 - sigmoid(x)))."""
    s = sigmoid(x)
    return s * (1.0 + _f64(x) * (1.0 - s))


def expert_ffn_backward(x, w_gate, w_up, w_down, dout):
    """Backward of E(x) = W_down (SiLU(W_gate x) * W_up x) on rows x [n, d]
    with output gradients dout [n, d]: returns dx [n, d], dW_gate [d_ff, d],
    dW_up [d_ff, d], dW_down [d, d_ff] (each summed over the rows)."""
    x, dout = _f64(x), _f64(dout)
    wg, wu, wd = _f64(w_gate), _f64(w_up), _f64(w_down)
    gp = x @ wg.T                     # gate pre-activation
    up = x @ wu.T                     # up projection
    act = silu(gp) * up
    dw_down = dout.T @ act
    dact = dout @ wd
    du = dact * silu(gp)
    dgp = dact * up * silu_grad(gp)
    dw_gate = dgp.T @ x
    dw_up = du.T @ x
    dx = dgp @ wg + du @ wu
    return dx, dw_gate, dw_up, dw_down


def gate_backward(routing: Routing, dg, mode):
    """Router-logit gradient [T, N] of the gate values, given dL/dg [T, k]
    (zero for slots that contributed nothing). Mode A: g is the softmax of
    the selected logits; mode B: g is the full-softmax probability, whose
    denominator holds every logit; mode C: g = s_i / sum of the selected s,
    s = sigmoid(z) (the selection bias is not differentiated: it only
    chooses)."""
    dg = _f64(dg)
    z = routing.z
    T, N = z.shape
    ids = routing.ids
    dz = np.zeros((T, N))
    g = routing.gates
    if mode == MODE_SOFTMAX_RENORM:
        inner = (g * dg).sum(axis=-1, keepdims=True)
        np.put_along_axis(dz, ids, g * (dg - inner), axis=-1)
    elif mode == MODE_SOFTMAX_FULL:
        P = softmax(z)
        a = np.zeros((T, N))
        np.put_along_axis(a, ids, dg, axis=-1)
        dz = P * (a - (P * a).sum(axis=-1, keepdims=True))
    elif mode == MODE_SIGMOID_BIAS_RENORM:
        s_sel = np.take_along_axis(sigmoid(z), ids, axis=-1)
        S = s_sel.sum(axis=-1, keepdims=True)
        ds = (dg - (g * dg).sum(axis=-1, keepdims=True)) / S
        np.put_along_axis(dz, ids, ds * s_sel * (1.0 - s_sel), axis=-1)
    else:
        raise ValueError(f"unknown gate mode {mode}")
    return dz


def stats_backward(routing: Routing, counts, k, mode, alpha, d_laux=0.0, d_zloss=0.0):
    """Router-logit gradient [T, N] of d_laux * L_aux + d_zloss * L_z. In
    L_aux = alpha N sum_i f_i p_i the fractions f_i are counts (piecewise
    constant: no gradient) and p_i = (1/T) sum_t P_ti; L_z is the mean squared
    log-sum-exp of the logits."""
    z = routing.z
    T, N = z.shape
    dz = np.zeros((T, N))
    if T == 0:
        return dz
    if d_laux:
        f = np.asarray(counts, dtype=F64) / (T * k)
        a = np.broadcast_to(d_laux * alpha * N * f / T, (T, N))   # dL/dP_ti
        if mode in (MODE_SOFTMAX_RENORM, MODE_SOFTMAX_FULL):
            P = softmax(z)
            dz += P * (a - (P * a).sum(axis=-1, keepdims=True))
        else:
            s = sigmoid(z)
            S = s.sum(axis=-1, keepdims=True)
            P = s / S
            ds = (a - (P * a).sum(axis=-1, keepdims=True)) / S
            dz += ds * s * (1.0 - s)
    if d_zloss:
        m = z.max(axis=-1, keepdims=True)
        lse = m + np.log(np.exp(z - m).sum(axis=-1, keepdims=True))
        dz += d_zloss * (2.0 / T) * lse * softmax(z)
    return dz


@dataclasses.dataclass
class LayerGrads:
    dh: np.ndarray         # [T, d]
    dw_router: np.ndarray  # [N, d]
    db_router: np.ndarray  # [N]
    dw_gate: np.ndarray    # [N, d_ff, d]
    dw_up: np.ndarray      # [N, d_ff, d]
    dw_down: np.ndarray    # [N, d, d_ff]
    dsh: Optional[tuple]   # (d sh_gate, d sh_up, d sh_down) or None
    dg: np.ndarray         # [T, k] gradient of the gate values
    dz: np.ndarray         # [T, N] gradient of the router logits


def layer_backward(h, w_router, k, mode, weights_of: WeightsOf, dy, b_router=None,
                   b_select=None, shared=None, alpha=0.01, groups=None,
                   capacity_factor=None, d_laux=0.0, d_zloss=0.0, ids=None) -> LayerGrads:
    """Gradients of <dy, y> + d_laux L_aux + d_zloss L_z with respect to h,
    W_r, b_r, every expert's weights and the shared expert's weights, for
    the selection and dispatch of the forward pass. Each kept slot (t, j) of
    expert e contributes dg[t, j] = <dy_t, E_e(h_t)> and back-propagates
    g[t, j] dy_t through E_e; a dropped slot contributes nothing. ``ids``
    fixes the selection (see route)."""
    h, dy = _f64(h), _f64(dy)
    T, d = h.shape
    wr = _f64(w_router)
    N = wr.shape[0]
    r = route(h, wr, k, mode, b_router, b_select, groups, ids)
    cap = expert_capacity(capacity_factor, T, k, N) if capacity_factor else None
    disp = dispatch(r.ids, N, cap)
    dh = np.zeros((T, d))
    dg = np.zeros((T, k))
    dwg, dwu, dwd = [], [], []
    for e in range(N):
        wg, wu, wd = weights_of(e)
        flats = disp.perm_src[disp.offsets[e]:disp.offsets[e + 1]]
        t, j = flats // k, flats % k
        x = h[t]
        dg[t, j] = np.sum(dy[t] * expert_ffn(x, wg, wu, wd), axis=-1)
        dout = r.gates[t, j][:, None] * dy[t]
        dx, g_g, g_u, g_d = expert_ffn_backward(x, wg, wu, wd, dout)
        np.add.at(dh, t, dx)
        dwg.append(g_g)
        dwu.append(g_u)
        dwd.append(g_d)
    dsh = None
    if shared is not None:
        dx, *dsh = expert_ffn_backward(h, *shared, dy)
        dh += dx
        dsh = tuple(dsh)
    dz = gate_backward(r, dg, mode) + stats_backward(r, disp.counts, k, mode, alpha, d_laux,
                                                     d_zloss)
    dh += dz @ wr
    return LayerGrads(dh, dz.T @ h, dz.sum(axis=0), np.stack(dwg), np.stack(dwu), np.stack(dwd),
                      dsh, dg, dz)


# ------------------------------------------------------ comparison helpers
def near_tie_tokens(gap, threshold=1e-4):
    """Tokens whose k-th and (k+1)-th selection scores are closer than the
    threshold: their selected set may legitimately differ between two
    correctly rounded implementations."""
    return np.asarray(gap) < threshold


def row_rel_err(y, y_ref):
    """max over elements of |y - y_ref| divided by max |y_ref|, per row."""
    y = _f64(y)
    y_ref = _f64(y_ref)
    num = np.abs(y - y_ref).max(axis=-1) if y.size else np.zeros(y.shape[0])
    den = np.abs(y_ref).max(axis=-1) if y.size else np.ones(y.shape[0])
    return num / np.where(den == 0, 1.0, den)
