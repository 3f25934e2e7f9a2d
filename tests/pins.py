"""Pins of the float64 oracle to facts that do not come from the oracle.

Each pin raises AssertionError when the oracle disagrees with what the pages
print for a worked example, a closed form, a library routine, brute force on
a tiny input, or an invariant of the mathematics. tests/test_oracle_pins.py
runs every pin; tests/test_oracle_mutations.py plants plausible mistakes in
the oracle and checks that at least one pin fails for each.
"""
import itertools
import json
import math
import os

import numpy as np
import scipy.special

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def _rand_inputs(rng, T, d, N, d_ff, shared=False):
    h = rng.standard_normal((T, d)) / math.sqrt(d)
    wr = rng.standard_normal((N, d))
    wg = rng.standard_normal((N, d_ff, d))
    wu = rng.standard_normal((N, d_ff, d))
    wd = rng.standard_normal((N, d, d_ff)) / math.sqrt(d_ff)
    sh = None
    if shared:
        sh = (rng.standard_normal((d_ff + 3, d)), rng.standard_normal((d_ff + 3, d)),
              rng.standard_normal((d, d_ff + 3)) / math.sqrt(d_ff))
    return h, wr, wg, wu, wd, sh


# --------------------------------------------------------- worked examples
def pin_softmax_worked_example():
    """Logits [2.2, 0.5, 1.8, -0.4] -> printed softmax (3 decimals); also
    scipy's softmax. [wuhy-notes §二 numeric example]"""
    g = golden("softmax_worked_example.json")
    p = O.softmax(np.array([g["logits"]]))[0]
    assert np.all(np.abs(p - g["softmax_printed"]) <= g["printed_tolerance"]), p
    assert np.allclose(p, scipy.special.softmax(g["logits"]), rtol=0, atol=1e-15)


def pin_top2_renorm_worked_example():
    """Same logits, top-2 renormalised -> experts {0, 2}, printed gates.
    Fed through the router with W_r = I and h = logits."""
    g = golden("softmax_worked_example.json")
    z = np.array([g["logits"]])
    r = O.route(z, np.eye(4), 2, O.MODE_SOFTMAX_RENORM)
    assert r.ids[0].tolist() == g["top2_experts"], r.ids
    assert np.all(np.abs(r.gates[0] - g["top2_gates_printed"]) <= g["printed_tolerance"])


def pin_top2_scores_example():
    """Scores [2, 1, 0]: top-2 renormalised -> [0.731, 0.269]; closed form
    sigmoid(1) = e/(1+e). Mode B keeps e^2/(e^2+e+1), e/(e^2+e+1).
    [cooking-agi, first section]"""
    g = golden("top2_renorm_example.json")
    z = np.array([g["scores"]])
    a = O.route(z, np.eye(3), 2, O.MODE_SOFTMAX_RENORM)
    assert a.ids[0].tolist() == [0, 1]
    assert np.all(np.abs(a.gates[0] - g["top2_gates_printed"]) <= g["printed_tolerance"])
    e = math.e
    assert abs(a.gates[0, 0] - e / (1 + e)) < 1e-15
    b = O.route(z, np.eye(3), 2, O.MODE_SOFTMAX_FULL)
    den = e * e + e + 1
    assert np.allclose(b.gates[0], [e * e / den, e / den], rtol=0, atol=1e-15)


def pin_dispatch_combine_example():
    """2 tokens / 3 experts: buckets E0<-{t0}, E1<-{t1}, E2<-{t0,t1};
    y0 = [1.5, 1], y1 = [2.6, 2.2] (a sum, not an overwrite).
    [cooking-agi, dispatch/combine section]"""
    g = golden("dispatch_combine_example.json")
    ids = np.array(g["ids"])
    disp = O.dispatch(ids, g["N"])
    for e, toks in g["buckets_printed"].items():
        lo, hi = disp.offsets[int(e)], disp.offsets[int(e) + 1]
        assert (disp.perm_src[lo:hi] // g["k"]).tolist() == toks
    eo = g["expert_outputs"]
    by_slot = {(0, 0): eo["t0_e0"], (0, 1): eo["t0_e2"], (1, 0): eo["t1_e1"], (1, 1): eo["t1_e2"]}
    out_rows = np.zeros((4, 2))
    for (t, j), v in by_slot.items():
        out_rows[disp.row_of[t * 2 + j]] = v
    y = O.combine(out_rows, disp.row_of, np.array(g["gates"]))
    assert np.allclose(y, g["y_printed"], rtol=0, atol=1e-12), y
    assert not np.allclose(y, g["y_if_overwritten_by_last_expert"])


def pin_dispatch_grouping_example():
    """4 tokens, top-2: E0<-T0,T2; E1<-T1,T3; E2<-T0,T1,T3; E3<-T2.
    [wuhy-notes §三 Token Dispatch]"""
    g = golden("dispatch_grouping_example.json")
    disp = O.dispatch(np.array(g["ids"]), g["N"])
    for e, toks in g["buckets_printed"].items():
        lo, hi = disp.offsets[int(e)], disp.offsets[int(e) + 1]
        assert (disp.perm_src[lo:hi] // g["k"]).tolist() == toks
    assert disp.counts.tolist() == [2, 2, 3, 1]
    assert disp.perm_src.tolist() == [0, 4, 2, 7, 1, 3, 6, 5]


# ------------------------------------------------------------ closed forms
def pin_router_logits_integer():
    """z = W_r h + b_r with W_r [N, d] = [[1,2,3],[4,5,6]], h = [1,1,1],
    b_r = [1,-1] -> [7, 14]; non-square so a transpose cannot pass."""
    z = O.router_logits(np.array([[1.0, 1.0, 1.0], [1.0, 0.0, 0.0]]),
                        np.array([[1.0, 2.0, 3.0], [4.0, 5.0, 6.0]]),
                        np.array([1.0, -1.0]))
    assert z.tolist() == [[7.0, 14.0], [2.0, 3.0]], z


def pin_sigmoid_silu_closed_forms():
    """sigmoid(ln a) = a/(1+a); SiLU(x) - SiLU(-x) = x; SiLU(0) = 0;
    scipy's expit."""
    for a in (0.25, 1.0, 3.0, 9.0):
        assert abs(O.sigmoid(np.log(a)) - a / (1 + a)) < 1e-15
        assert abs(O.silu(np.log(a)) - np.log(a) * a / (1 + a)) < 1e-15
    x = np.linspace(-8, 8, 33)
    assert np.allclose(O.silu(x) - O.silu(-x), x, rtol=0, atol=1e-13)
    assert O.silu(0.0) == 0.0
    assert np.allclose(O.sigmoid(x), scipy.special.expit(x), rtol=1e-15, atol=0)


def pin_expert_ffn_integer():
    """W_gate h = [40, 50, 60, -40] (SiLU ~ identity / ~0 there), W_up h =
    [1, 2, 3, 7], W_down [2 x 4] -> [220, -80] up to e^-40 terms.
    Non-square shapes: a transposed operand cannot pass."""
    h = np.array([[1.0, 2.0]])
    wg = np.array([[10.0, 15.0], [20.0, 15.0], [0.0, 30.0], [-40.0, 0.0]])
    wu = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [7.0, 0.0]])
    wd = np.array([[1.0, 0.0, 1.0, 1.0], [0.0, 1.0, -1.0, 1.0]])
    y = O.expert_ffn(h, wg, wu, wd)
    assert np.allclose(y, [[220.0, -80.0]], rtol=1e-12, atol=0), y


def pin_topk_brute_force():
    """Top-k equals the k-subset with the largest score sum (distinct
    scores), listed by descending score; ties go to the lower index."""
    rng = np.random.default_rng(7)
    for N, k in [(5, 2), (6, 3), (7, 1), (4, 4)]:
        s = rng.standard_normal((20, N))
        ids, gap = O.topk(s, k)
        for t in range(20):
            best = max(itertools.combinations(range(N), k), key=lambda c: s[t, list(c)].sum())
            assert sorted(ids[t].tolist()) == sorted(best)
            assert np.all(np.diff(s[t, ids[t]]) < 0)
            srt = np.sort(s[t])[::-1]
            want = srt[k - 1] - srt[k] if k < N else np.inf
            assert gap[t] == want
    ids, _ = O.topk(np.array([[1.0, 3.0, 3.0, 2.0], [5.0, 5.0, 5.0, 5.0]]), 2)
    assert ids.tolist() == [[1, 2], [0, 1]]
    ids, _ = O.topk(np.array([[1.0, 3.0, 3.0, 2.0]]), 1)
    assert ids.tolist() == [[1]]


def pin_dispatch_stable_sort():
    """perm_src is numpy's stable argsort of the flat expert ids; counts
    its bincount; row_of its inverse."""
    rng = np.random.default_rng(3)
    for T, N, k in [(0, 4, 2), (1, 4, 4), (37, 9, 3), (200, 16, 1)]:
        ids = np.stack([rng.permutation(N)[:k] for _ in range(T)]) if T else np.zeros((0, k), int)
        disp = O.dispatch(ids, N)
        flat = ids.reshape(-1)
        assert disp.perm_src.tolist() == np.argsort(flat, kind="stable").tolist()
        assert disp.counts.tolist() == np.bincount(flat, minlength=N).tolist()
        assert disp.offsets[-1] == T * k
        assert np.all(disp.perm_src[disp.row_of] == np.arange(T * k))


def pin_mode_a_equivalence():
    """Softmax over the selected logits equals the full softmax renormalised
    over the selected experts. [cooking-agi, first section]"""
    rng = np.random.default_rng(11)
    z = rng.standard_normal((50, 9)) * 3
    r = O.route(z, np.eye(9), 3, O.MODE_SOFTMAX_RENORM)
    zs = np.take_along_axis(z, r.ids, axis=-1)
    assert np.allclose(r.gates, scipy.special.softmax(zs, axis=-1), rtol=0, atol=1e-15)
    full = scipy.special.softmax(z, axis=-1)
    assert np.allclose(r.stat_prob, full, rtol=0, atol=1e-15)


def pin_mode_b_top1():
    """Mode B with k = 1: the gate is max_i p_ti and is below 1;
    mode A with k = 1 gives gate 1."""
    rng = np.random.default_rng(5)
    z = rng.standard_normal((30, 6))
    b = O.route(z, np.eye(6), 1, O.MODE_SOFTMAX_FULL)
    p = scipy.special.softmax(z, axis=-1)
    assert np.allclose(b.gates[:, 0], p.max(axis=-1), rtol=0, atol=1e-15)
    assert np.all(b.gates < 1)
    assert b.ids[:, 0].tolist() == p.argmax(axis=-1).tolist()
    a = O.route(z, np.eye(6), 1, O.MODE_SOFTMAX_RENORM)
    assert np.all(a.gates == 1.0)


def pin_mode_c_hand_case():
    """sigmoid(z) = [0.60, 0.55, 0.50], b_sel = [-0.1, 0, 0.1], k = 2:
    selection scores [0.50, 0.55, 0.60] -> experts [2, 1], gates from the
    unbiased scores [0.50, 0.55] / 1.05."""
    s = np.array([0.60, 0.55, 0.50])
    z = np.log(s / (1 - s))[None, :]
    r = O.route(z, np.eye(3), 2, O.MODE_SIGMOID_BIAS_RENORM,
                b_select=np.array([-0.1, 0.0, 0.1]))
    assert r.ids[0].tolist() == [2, 1]
    assert np.allclose(r.gates[0], [0.50 / 1.05, 0.55 / 1.05], rtol=0, atol=1e-15)
    assert np.allclose(r.stat_prob[0], s / s.sum(), rtol=0, atol=1e-15)


def pin_load_stats_hand_case():
    """T=2, N=2, k=1: logits [ln 3, 0] -> p = [0.75, 0.25]; logits [0, 0]
    -> [0.5, 0.5], a tie taken by expert 0. counts [2, 0], f = [1, 0],
    p = [0.625, 0.375], L_aux = alpha * 2 * 0.625."""
    z = np.array([[math.log(3.0), 0.0], [0.0, 0.0]])
    r = O.route(z, np.eye(2), 1, O.MODE_SOFTMAX_FULL)
    assert r.ids[:, 0].tolist() == [0, 0]
    d = O.dispatch(r.ids, 2)
    f, p, l_aux = O.load_stats(d.counts, r.stat_prob, 1, 0.01)
    assert d.counts.tolist() == [2, 0]
    assert np.allclose(f, [1.0, 0.0], rtol=0, atol=0)
    assert np.allclose(p, [0.625, 0.375], rtol=0, atol=1e-15)
    assert abs(l_aux - 0.01 * 2 * 0.625) < 1e-15
    # k = 2 normalisation: both experts always chosen -> f = [0.5, 0.5]
    d2 = O.dispatch(O.route(z, np.eye(2), 2, O.MODE_SOFTMAX_RENORM).ids, 2)
    f2, _, _ = O.load_stats(d2.counts, r.stat_prob, 2, 0.01)
    assert np.allclose(f2, [0.5, 0.5], rtol=0, atol=0)


def pin_balanced_cyclic_stats():
    """Exactly balanced routing by construction: token t's logits are a
    cyclic shift of one vector, T a multiple of N -> f_i = p_i = 1/N and
    L_aux = alpha (Switch loss at perfect balance)."""
    N, k, alpha = 8, 2, 0.05
    base = np.array([3.0, 2.0, 1.5, 0.5, 0.0, -1.0, -2.0, -3.0])
    z = np.stack([np.roll(base, t) for t in range(4 * N)])
    for mode, bsel in ((O.MODE_SOFTMAX_RENORM, None), (O.MODE_SIGMOID_BIAS_RENORM, np.zeros(N))):
        r = O.route(z, np.eye(N), k, mode, b_select=bsel)
        d = O.dispatch(r.ids, N)
        f, p, l_aux = O.load_stats(d.counts, r.stat_prob, k, alpha)
        assert np.allclose(f, 1.0 / N, rtol=0, atol=1e-15)
        assert np.allclose(p, 1.0 / N, rtol=0, atol=1e-15)
        assert abs(l_aux - alpha) < 1e-14


# ------------------------------------------------ whole-layer brute force
def pin_sparse_equals_dense():
    """Sparse dispatch + combine equals the dense brute force (all experts on
    all tokens, gates zero off the selection), all modes, with and without a
    shared expert. [cooking-agi, dense-oracle section]"""
    rng = np.random.default_rng(21)
    for mode in (O.MODE_SOFTMAX_RENORM, O.MODE_SOFTMAX_FULL, O.MODE_SIGMOID_BIAS_RENORM):
        for shared in (False, True):
            T, d, N, k, dff = 23, 6, 5, 2, 7
            h, wr, wg, wu, wd, sh = _rand_inputs(rng, T, d, N, dff, shared)
            br = rng.standard_normal(N)
            bs = rng.uniform(-0.1, 0.1, N) if mode == O.MODE_SIGMOID_BIAS_RENORM else None
            W = O.weights_getter(wg, wu, wd)
            res = O.layer(h, wr, k, mode, W, br, bs, sh)
            yd = O.dense_layer(h, wr, k, mode, W, br, bs, sh)
            assert np.allclose(res.y, yd, rtol=0, atol=1e-12)
            yt = O.layer_tokens(h, res.routing, [5, 0, 22], W, sh)
            assert np.allclose(yt, res.y[[5, 0, 22]], rtol=0, atol=1e-12)


def pin_identical_experts():
    """All experts equal and gates summing to 1 (modes A, C) -> y = E(h),
    a plain SwiGLU FFN evaluated directly here."""
    rng = np.random.default_rng(8)
    T, d, N, dff = 17, 5, 6, 4
    h = rng.standard_normal((T, d))
    wr = rng.standard_normal((N, d))
    wg, wu, wd = rng.standard_normal((dff, d)), rng.standard_normal((dff, d)), rng.standard_normal((d, dff))
    g = h @ wg.T
    direct = ((g * scipy.special.expit(g)) * (h @ wu.T)) @ wd.T
    for mode, bs in ((O.MODE_SOFTMAX_RENORM, None), (O.MODE_SIGMOID_BIAS_RENORM, rng.uniform(-.1, .1, N))):
        res = O.layer(h, wr, 3, mode, lambda e: (wg, wu, wd), b_select=bs)
        assert np.allclose(res.y, direct, rtol=0, atol=1e-12)


def pin_soft_mixture_k_equals_n():
    """Mode A with k = N: y_t = sum_i softmax(z_t)_i E_i(h_t)."""
    rng = np.random.default_rng(9)
    T, d, N, dff = 11, 4, 3, 5
    h, wr, wg, wu, wd, _ = _rand_inputs(rng, T, d, N, dff)
    P = scipy.special.softmax(h @ wr.T, axis=-1)
    want = np.zeros((T, d))
    for e in range(N):
        g = h @ wg[e].T
        want += P[:, e:e + 1] * (((g * scipy.special.expit(g)) * (h @ wu[e].T)) @ wd[e].T)
    res = O.layer(h, wr, N, O.MODE_SOFTMAX_RENORM, O.weights_getter(wg, wu, wd))
    assert np.allclose(res.y, want, rtol=0, atol=1e-12)


def pin_permutation_symmetry():
    """Permuting tokens permutes y; relabelling the experts (router rows,
    expert weights and selection bias together) leaves y and gates alone."""
    rng = np.random.default_rng(13)
    T, d, N, k, dff = 19, 6, 7, 3, 5
    h, wr, wg, wu, wd, sh = _rand_inputs(rng, T, d, N, dff, True)
    bs = rng.uniform(-0.1, 0.1, N)
    br = rng.standard_normal(N)
    for mode in (O.MODE_SOFTMAX_RENORM, O.MODE_SIGMOID_BIAS_RENORM):
        base = O.layer(h, wr, k, mode, O.weights_getter(wg, wu, wd), br, bs, sh)
        tp = rng.permutation(T)
        pt = O.layer(h[tp], wr, k, mode, O.weights_getter(wg, wu, wd), br, bs, sh)
        assert np.allclose(pt.y, base.y[tp], rtol=0, atol=1e-12)
        ep = rng.permutation(N)
        pe = O.layer(h, wr[ep], k, mode, O.weights_getter(wg[ep], wu[ep], wd[ep]), br[ep], bs[ep], sh)
        assert np.allclose(pe.y, base.y, rtol=0, atol=1e-12)
        assert np.allclose(pe.routing.gates, base.routing.gates, rtol=0, atol=1e-15)
        assert (ep[pe.routing.ids] == base.routing.ids).all()


# ------------------------------------------------- group-limited selection
def pin_group_limited_worked_example():
    """Groups A = [0.90, 0.10], B = [0.80, 0.79], k = 2: unrestricted ->
    {0, 2}; keep the group with the larger maximum -> {0, 1}; keep the group
    with the larger top-2 sum -> {2, 3}. Run as mode C selection scores
    (sigmoid(z) = score, no bias) and as mode A (softmax probabilities
    proportional to the scores). [cooking-agi, group-limited routing]"""
    g = golden("group_limited_example.json")
    sc = np.array(g["scores"])
    G, k = g["n_groups"], g["k"]
    for mode, z, b in ((O.MODE_SIGMOID_BIAS_RENORM, np.log(sc / (1 - sc)), np.zeros(4)),
                       (O.MODE_SOFTMAX_RENORM, np.log(sc), None)):
        z = z[None, :]
        for groups, want in ((None, g["unrestricted"]), ((G, 1, 1), g["keep_1_group_by_max"]),
                             ((G, 1, 2), g["keep_1_group_by_top2_sum"])):
            r = O.route(z, np.eye(4), k, mode, b_select=b, groups=groups)
            assert r.ids[0].tolist() == want, (mode, groups, r.ids)
            if mode == O.MODE_SIGMOID_BIAS_RENORM:
                assert np.allclose(r.gates[0], sc[want] / sc[want].sum(), rtol=0, atol=1e-15)
        _, ggap = O.group_limit(sc[None, :], G, 1, 2)
        assert abs(ggap[0] - (g["group_scores_by_top2_sum"][1] - g["group_scores_by_top2_sum"][0])) < 1e-12


def pin_group_limit_brute_force():
    """On tiny random inputs (distinct scores), the kept groups are a set K
    of topk_groups groups with no outside group scoring higher (ties to the
    lower index), a group's score being the largest sum over topm of its
    experts (enumerated); the picks are the best k-subset of K's experts."""
    rng = np.random.default_rng(11)
    for N, G in ((6, 2), (6, 3), (8, 4), (12, 3), (12, 6)):
        gs = N // G
        for gk in range(1, G + 1):
            for m in range(1, gs + 1):
                for k in range(1, min(gk * gs, 4) + 1):
                    sel = rng.permutation(N)[None, :].astype(float) / N + rng.random(N)[None, :] * 1e-3
                    score = [max(sum(c) for c in itertools.combinations(sel[0, g * gs:(g + 1) * gs], m))
                             for g in range(G)]
                    best = None
                    for K in itertools.combinations(range(G), gk):
                        out = [g for g in range(G) if g not in K]
                        if all(score[a] > score[b] or (score[a] == score[b] and a < b)
                               for a in K for b in out):
                            best = K
                    cand = [e for e in range(N) if e // gs in best]
                    pick = max(itertools.combinations(cand, k), key=lambda c: sum(sel[0, list(c)]))
                    masked, _ = O.group_limit(sel, G, gk, m)
                    ids, _ = O.topk(masked, k)
                    assert sorted(ids[0].tolist()) == sorted(pick), (N, G, gk, m, k)
                    assert all(sel[0, ids[0][i]] > sel[0, ids[0][i + 1]] for i in range(k - 1))


def pin_group_limit_trivial_cases():
    """One group, or keeping every group, selects exactly as without a
    group limit."""
    rng = np.random.default_rng(12)
    h, wr, *_ = _rand_inputs(rng, 30, 8, 8, 4)
    for mode in (O.MODE_SOFTMAX_RENORM, O.MODE_SOFTMAX_FULL, O.MODE_SIGMOID_BIAS_RENORM):
        b = rng.uniform(-0.1, 0.1, 8) if mode == O.MODE_SIGMOID_BIAS_RENORM else None
        ref = O.route(h, wr, 3, mode, b_select=b)
        for groups in ((1, 1, 1), (4, 4, 2), (2, 2, 1)):
            r = O.route(h, wr, 3, mode, b_select=b, groups=groups)
            assert np.array_equal(r.ids, ref.ids) and np.allclose(r.gates, ref.gates, rtol=0, atol=0)


def pin_group_mask_is_minus_infinity():
    """Mode C selection scores can be negative: with sel = [0.9, -0.05, 0.5,
    0.4] in groups {0, 1} and {2, 3}, keeping one group by its maximum keeps
    the first and must pick experts 0 and 1 (a zero mask would pick 2)."""
    s = np.array([0.8, 0.05, 0.45, 0.35])
    b = np.array([0.1, -0.1, 0.05, 0.05])
    r = O.route(np.log(s / (1 - s))[None, :], np.eye(4), 2, O.MODE_SIGMOID_BIAS_RENORM,
                b_select=b, groups=(2, 1, 1))
    assert r.ids[0].tolist() == [0, 1]
    assert np.allclose(r.gates[0], s[[0, 1]] / s[[0, 1]].sum(), rtol=0, atol=1e-15)


# ------------------------------------------------ z-loss and routing entropy
def pin_z_loss_closed_forms():
    """z-loss of the worked-example logits [2.2, 0.5, 1.8, -0.4] is
    (ln(e^2.2 + e^0.5 + e^1.8 + e^-0.4))^2 (scipy's logsumexp); all-zero
    logits over N experts give (ln N)^2; a shift by c adds c to every
    log-sum-exp; the mean is over tokens."""
    z = np.array([[2.2, 0.5, 1.8, -0.4]])
    want = math.log(math.exp(2.2) + math.exp(0.5) + math.exp(1.8) + math.exp(-0.4)) ** 2
    assert abs(O.router_z_loss(z) - want) < 1e-12
    assert abs(O.router_z_loss(z) - scipy.special.logsumexp(z[0]) ** 2) < 1e-12
    assert abs(O.router_z_loss(np.zeros((3, 8))) - math.log(8) ** 2) < 1e-12
    two = np.vstack([z, z + 1.5])
    l0 = scipy.special.logsumexp(z[0])
    assert abs(O.router_z_loss(two) - (l0 ** 2 + (l0 + 1.5) ** 2) / 2) < 1e-12


def pin_routing_entropy_closed_forms():
    """Uniform routing over N experts has entropy ln N; a one-hot row has 0;
    random rows match scipy.stats.entropy (natural log), averaged over
    tokens."""
    import scipy.stats
    assert abs(O.routing_entropy(np.full((2, 8), 1 / 8)) - math.log(8)) < 1e-12
    assert O.routing_entropy(np.eye(4)) == 0.0
    rng = np.random.default_rng(13)
    q = rng.random((5, 7))
    q /= q.sum(axis=1, keepdims=True)
    want = np.mean([scipy.stats.entropy(r) for r in q])
    assert abs(O.routing_entropy(q) - want) < 1e-12


# ------------------------------------------------------- expert capacity
def pin_capacity_closed_form():
    """C = ceil(capacity_factor * T * k / N) [wuhy-notes §六 Expert
    Capacity]: T = 4, k = 2, N = 4 gives T k / N = 2, so factor 1 -> 2,
    1.25 -> 3 (2.5 rounds up), 0.5 -> 1; T = 10, k = 2, N = 4, factor 1.25
    -> ceil(6.25) = 7."""
    assert O.expert_capacity(1.0, 4, 2, 4) == 2
    assert O.expert_capacity(1.25, 4, 2, 4) == 3
    assert O.expert_capacity(0.5, 4, 2, 4) == 1
    assert O.expert_capacity(1.25, 10, 2, 4) == 7


def pin_capacity_grouping_example():
    """The 4-token top-2 grouping example (E0<-T0,T2; E1<-T1,T3;
    E2<-T0,T1,T3; E3<-T2) with capacity factor 1 (C = 2): E2's third slot,
    the latest token T3, is dropped; every other slot is kept. Worked by
    hand from the page's listing and the capacity formula."""
    g = golden("dispatch_grouping_example.json")
    ids = np.array(g["ids"])
    d = O.dispatch(ids, 4, O.expert_capacity(1.0, 4, 2, 4))
    assert d.counts.tolist() == [2, 2, 3, 1]
    assert d.kept.tolist() == [2, 2, 2, 1]
    assert d.offsets.tolist() == [0, 2, 4, 6, 7]
    dropped = [f for f in range(8) if d.row_of[f] < 0]
    assert dropped == [6] and ids.reshape(-1)[6] == 2 and 6 // 2 == 3
    assert d.perm_src.tolist() == [0, 4, 2, 7, 1, 3, 5]
    for e, toks in g["buckets_printed"].items():     # kept tokens: the printed ones, C at most
        kept = [int(f) // 2 for f in d.perm_src[d.offsets[int(e)]:d.offsets[int(e) + 1]]]
        assert kept == toks[:2]
    usage, drop = O.capacity_stats(d, 2)
    assert usage == 7 / 8 and drop == 1 / 8
    y = O.combine(np.arange(7.0)[:, None] + 1.0, d.row_of, np.ones((4, 2)))
    assert y[:, 0].tolist() == [1 + 5, 3 + 6, 2 + 7, 4]   # token 3 keeps only its E1 row


def pin_capacity_dense_equivalence():
    """With a capacity, the sparse layer equals the dense brute force whose
    gates are zeroed on each expert's slots past C (in token order), for all
    gate modes, with and without a shared expert; a capacity that no expert
    reaches changes nothing."""
    rng = np.random.default_rng(14)
    for mode, shared, cf in ((O.MODE_SOFTMAX_RENORM, False, 0.75), (O.MODE_SOFTMAX_FULL, True, 1.0),
                             (O.MODE_SIGMOID_BIAS_RENORM, True, 0.5)):
        h, wr, wg, wu, wd, sh = _rand_inputs(rng, 24, 6, 5, 7, shared)
        b = rng.uniform(-0.1, 0.1, 5) if mode == O.MODE_SIGMOID_BIAS_RENORM else None
        W_ = O.weights_getter(wg, wu, wd)
        sparse = O.layer(h, wr, 2, mode, W_, b_select=b, shared=sh, capacity_factor=cf)
        dense = O.dense_layer(h, wr, 2, mode, W_, b_select=b, shared=sh, capacity_factor=cf)
        assert np.allclose(sparse.y, dense, rtol=0, atol=1e-12)
        assert (sparse.disp.row_of < 0).any()
        free = O.layer(h, wr, 2, mode, W_, b_select=b, shared=sh)
        big = O.layer(h, wr, 2, mode, W_, b_select=b, shared=sh, capacity_factor=5.0)
        assert np.array_equal(big.y, free.y)


# --------------------------------------------------------------- backward
def _dense_loss_torch(h, wr, br, wg, wu, wd, sh, ids, keep, counts, k, mode, alpha, dy,
                      d_laux, d_zloss):
    """The dense brute force of the loss <dy, y> + d_laux L_aux + d_zloss L_z
    in float64 torch ops, for a fixed selection ids [T, k] and kept-slot mask
    keep [T, k]: every expert runs on every token, the gates (a softmax of
    the selected logits in mode A, the full-softmax probability in mode B,
    the renormalised selected sigmoids in mode C) sit in a dense [T, N]
    matrix that is zero elsewhere [cooking-agi "怎么知道实现没把梯度弄丢？"]."""
    import torch
    T, N = h.shape[0], wr.shape[0]
    z = h @ wr.T + (br if br is not None else 0.0)
    if mode == O.MODE_SOFTMAX_RENORM:
        P = torch.softmax(z, -1)
        g = torch.softmax(z.gather(1, ids), -1)
    elif mode == O.MODE_SOFTMAX_FULL:
        P = torch.softmax(z, -1)
        g = P.gather(1, ids)
    else:
        s = torch.sigmoid(z)
        ss = s.gather(1, ids)
        g = ss / ss.sum(-1, keepdim=True)
        P = s / s.sum(-1, keepdim=True)
    G = torch.zeros(T, N, dtype=torch.float64).scatter(1, ids, g * keep)
    y = torch.zeros_like(h)
    for e in range(N):
        a = torch.nn.functional.silu(h @ wg[e].T) * (h @ wu[e].T)
        y = y + G[:, e:e + 1] * (a @ wd[e].T)
    if sh is not None:
        y = y + (torch.nn.functional.silu(h @ sh[0].T) * (h @ sh[1].T)) @ sh[2].T
    f = torch.as_tensor(counts, dtype=torch.float64) / (T * k)
    l_aux = alpha * N * (f * P.mean(0)).sum()
    l_z = (torch.logsumexp(z, -1) ** 2).mean()
    return (dy * y).sum() + d_laux * l_aux + d_zloss * l_z


def _kept_mask(ids, N, cap):
    """Slots kept under capacity cap, walking tokens in order (all without)."""
    keep = np.ones(ids.shape)
    if cap is None:
        return keep
    seen = np.zeros(N, dtype=int)
    for t in range(ids.shape[0]):
        for j in range(ids.shape[1]):
            seen[ids[t, j]] += 1
            keep[t, j] = 1.0 if seen[ids[t, j]] <= cap else 0.0
    return keep


def pin_backward_matches_dense_autograd():
    """The oracle's gradients of h, W_r, b_r, every expert's and the shared
    expert's weights equal torch autograd through the dense brute force
    (float64), in all three gate modes, with and without a shared expert,
    a capacity, a group limit and the auxiliary-loss terms."""
    import torch
    rng = np.random.default_rng(21)
    cases = [(O.MODE_SOFTMAX_RENORM, False, None, None, 0.0, 0.0),
             (O.MODE_SOFTMAX_RENORM, True, 0.75, None, 0.7, 0.3),
             (O.MODE_SOFTMAX_FULL, False, None, None, 0.0, 0.0),
             (O.MODE_SOFTMAX_FULL, True, 1.0, (3, 2, 1), 1.3, 0.0),
             (O.MODE_SIGMOID_BIAS_RENORM, False, None, None, 0.0, 0.0),
             (O.MODE_SIGMOID_BIAS_RENORM, True, 0.5, (3, 2, 2), 0.9, 0.4)]
    T, d, N, k, d_ff = 20, 6, 6, 2, 5
    for mode, shared, cf, groups, d_laux, d_zloss in cases:
        h, wr, wg, wu, wd, sh = _rand_inputs(rng, T, d, N, d_ff, shared)
        br = rng.uniform(-0.3, 0.3, N)
        bs = rng.uniform(-0.1, 0.1, N) if mode == O.MODE_SIGMOID_BIAS_RENORM else None
        dy = rng.standard_normal((T, d))
        W_ = O.weights_getter(wg, wu, wd)
        gr = O.layer_backward(h, wr, k, mode, W_, dy, br, bs, sh, 0.02, groups, cf, d_laux, d_zloss)
        r = O.route(h, wr, k, mode, br, bs, groups)
        cap = O.expert_capacity(cf, T, k, N) if cf else None
        counts = np.bincount(r.ids.reshape(-1), minlength=N)
        keep = _kept_mask(r.ids, N, cap)
        if cap is not None:
            assert keep.min() == 0.0
        tt = {n: torch.tensor(v, dtype=torch.float64, requires_grad=True)
              for n, v in (("h", h), ("wr", wr), ("br", br), ("wg", wg), ("wu", wu), ("wd", wd))}
        tsh = None if sh is None else [torch.tensor(v, requires_grad=True) for v in sh]
        loss = _dense_loss_torch(tt["h"], tt["wr"], tt["br"], tt["wg"], tt["wu"], tt["wd"], tsh,
                                 torch.as_tensor(r.ids), torch.as_tensor(keep), counts, k, mode,
                                 0.02, torch.as_tensor(dy), d_laux, d_zloss)
        loss.backward()
        for mine, ref in ((gr.dh, tt["h"]), (gr.dw_router, tt["wr"]), (gr.db_router, tt["br"]),
                          (gr.dw_gate, tt["wg"]), (gr.dw_up, tt["wu"]), (gr.dw_down, tt["wd"])):
            assert np.allclose(mine, ref.grad.numpy(), rtol=1e-10, atol=1e-12), (mode, cf)
        if sh is not None:
            for mine, ref in zip(gr.dsh, tsh):
                assert np.allclose(mine, ref.grad.numpy(), rtol=1e-10, atol=1e-12)


def _loss_of(h, wr, br, bs, wg, wu, wd, sh, k, mode, alpha, groups, cf, dy, d_laux, d_zloss):
    res = O.layer(h, wr, k, mode, O.weights_getter(wg, wu, wd), br, bs, sh, alpha, groups,
                  capacity_factor=cf)
    r = O.route(h, wr, k, mode, br, bs, groups)
    return (float(np.sum(dy * res.y)) + d_laux * res.l_aux + d_zloss * O.router_z_loss(r.z),
            r.ids)


def pin_backward_finite_differences():
    """Central differences of the oracle's own forward loss (step 1e-5, the
    selection checked unchanged at both points, inputs far from top-k ties)
    agree with the oracle's gradients on sampled coordinates of every
    parameter, for each gate mode."""
    rng = np.random.default_rng(22)
    T, d, N, k, d_ff = 12, 5, 5, 2, 4
    eps = 1e-5
    for mode, cf, d_laux, d_zloss in ((O.MODE_SOFTMAX_RENORM, None, 0.5, 0.2),
                                      (O.MODE_SOFTMAX_FULL, 1.0, 0.0, 0.7),
                                      (O.MODE_SIGMOID_BIAS_RENORM, 0.75, 1.1, 0.0)):
        for _ in range(20):
            h, wr, wg, wu, wd, sh = _rand_inputs(rng, T, d, N, d_ff, True)
            wr = wr * 2.0
            br = rng.uniform(-0.3, 0.3, N)
            bs = rng.uniform(-0.1, 0.1, N) if mode == O.MODE_SIGMOID_BIAS_RENORM else None
            if O.route(h, wr, k, mode, br, bs).gap.min() > 1e-3:
                break
        dy = rng.standard_normal((T, d))
        gr = O.layer_backward(h, wr, k, mode, O.weights_getter(wg, wu, wd), dy, br, bs, sh, 0.02,
                              None, cf, d_laux, d_zloss)
        params = {"h": (h, gr.dh), "wr": (wr, gr.dw_router), "br": (br, gr.db_router),
                  "wg": (wg, gr.dw_gate), "wu": (wu, gr.dw_up), "wd": (wd, gr.dw_down),
                  "sg": (sh[0], gr.dsh[0]), "sd": (sh[2], gr.dsh[2])}
        for name, (arr, grad) in params.items():
            for flat in rng.choice(arr.size, size=4, replace=False):
                idx = np.unravel_index(flat, arr.shape)
                vals = []
                for sgn in (1.0, -1.0):
                    a2 = {n: v[0].copy() for n, v in params.items()}
                    a2[name][idx] += sgn * eps
                    shp = (a2["sg"], sh[1], a2["sd"])
                    lv, ids = _loss_of(a2["h"], a2["wr"], a2["br"], bs, a2["wg"], a2["wu"],
                                       a2["wd"], shp, k, mode, 0.02, None, cf, dy, d_laux, d_zloss)
                    assert np.array_equal(ids, O.route(h, wr, k, mode, br, bs).ids)
                    vals.append(lv)
                fd = (vals[0] - vals[1]) / (2 * eps)
                assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (mode, name, idx, fd, grad[idx])


def pin_backward_zero_structure():
    """An expert never selected gets exactly zero weight gradients; without
    auxiliary losses the unselected logits get no gradient in modes A and C
    but do in mode B (its full-softmax denominator holds them); with top-1
    in mode A the gate is identically 1, so the router gets no task
    gradient [cooking-agi "top-k 不可导，router 怎么学"]."""
    rng = np.random.default_rng(23)
    T, d, N, d_ff = 16, 6, 5, 4
    h, wr, wg, wu, wd, _ = _rand_inputs(rng, T, d, N, d_ff)
    br = np.zeros(N)
    br[4] = -50.0                            # expert 4 is never chosen
    dy = rng.standard_normal((T, d))
    W_ = O.weights_getter(wg, wu, wd)
    for mode in (O.MODE_SOFTMAX_RENORM, O.MODE_SOFTMAX_FULL, O.MODE_SIGMOID_BIAS_RENORM):
        bs = np.zeros(N) if mode == O.MODE_SIGMOID_BIAS_RENORM else None
        gr = O.layer_backward(h, wr, 2, mode, W_, dy, br, bs)
        assert not np.any(gr.dw_gate[4]) and not np.any(gr.dw_up[4]) and not np.any(gr.dw_down[4])
        r = O.route(h, wr, 2, mode, br, bs)
        unsel = np.ones((T, N), dtype=bool)
        np.put_along_axis(unsel, r.ids, False, axis=-1)
        if mode == O.MODE_SOFTMAX_FULL:
            assert np.all(np.abs(gr.dz[unsel]) > 0)
        else:
            assert not np.any(gr.dz[unsel])
    gr = O.layer_backward(h, wr, 1, O.MODE_SOFTMAX_RENORM, W_, dy, br)
    assert not np.any(gr.dz) and not np.any(gr.dw_router) and not np.any(gr.db_router)


def pin_route_given_selection():
    """Routing with a given selection reproduces the oracle's own gates and
    statistics when that selection is its own; for another selection the
    gates follow the mode's formula on those experts (mode A: softmax of
    their logits; B: their full-softmax probabilities; C: their renormalised
    sigmoids)."""
    rng = np.random.default_rng(24)
    h, wr, *_ = _rand_inputs(rng, 9, 6, 7, 4)
    for mode in (O.MODE_SOFTMAX_RENORM, O.MODE_SOFTMAX_FULL, O.MODE_SIGMOID_BIAS_RENORM):
        bs = rng.uniform(-0.1, 0.1, 7) if mode == O.MODE_SIGMOID_BIAS_RENORM else None
        r = O.route(h, wr, 3, mode, b_select=bs)
        r2 = O.route(h, wr, 3, mode, b_select=bs, ids=r.ids)
        assert np.array_equal(r2.gates, r.gates) and np.array_equal(r2.stat_prob, r.stat_prob)
        other = np.tile(np.array([[6, 0, 3]]), (9, 1))
        g = O.route(h, wr, 3, mode, b_select=bs, ids=other).gates
        z = h @ wr.T
        zs = np.take_along_axis(z, other, axis=-1)
        if mode == O.MODE_SOFTMAX_RENORM:
            want = scipy.special.softmax(zs, axis=-1)
        elif mode == O.MODE_SOFTMAX_FULL:
            want = np.take_along_axis(scipy.special.softmax(z, axis=-1), other, axis=-1)
        else:
            sg = scipy.special.expit(zs)
            want = sg / sg.sum(axis=-1, keepdims=True)
        assert np.allclose(g, want, rtol=1e-13, atol=0)



# ------------------------------------------------------ comparison helpers
def pin_row_rel_err_hand_cases():
    """Per-row max |y - y_ref| over max |y_ref|, worked by hand: [1, 2] vs
    [1, 4] -> 2/4; [-3, 0] vs [-1, 2] -> 2/2 (magnitudes, not signed
    values); [0.5, -0.25, 7] vs [1, -0.5, 7] -> 0.5/7 (the row's largest
    reference entry, not the entry where the error is); stacked rows are
    independent (no tensor-wide scale); a zero reference row gives the
    absolute difference; no rows, no errors."""
    a = O.row_rel_err(np.array([[1.0, 2.0]]), np.array([[1.0, 4.0]]))
    assert a.shape == (1,) and a[0] == 0.5, a
    b = O.row_rel_err(np.array([[-3.0, 0.0]]), np.array([[-1.0, 2.0]]))
    assert b[0] == 1.0, b
    c = O.row_rel_err(np.array([[0.5, -0.25, 7.0]]), np.array([[1.0, -0.5, 7.0]]))
    assert abs(c[0] - 0.5 / 7.0) < 1e-16, c
    both = O.row_rel_err(np.array([[1.0, 2.0], [-3.0, 0.0], [10.0, 10.0]]),
                         np.array([[1.0, 4.0], [-1.0, 2.0], [10.0, 10.0]]))
    assert both.tolist() == [0.5, 1.0, 0.0], both
    z = O.row_rel_err(np.array([[0.0, 3e-3], [0.0, 0.0]]), np.zeros((2, 2)))
    assert z.tolist() == [3e-3, 0.0], z
    assert O.row_rel_err(np.zeros((0, 4)), np.zeros((0, 4))).shape == (0,)


def pin_near_tie_tokens_hand_cases():
    """A token is near a tie when its gap is strictly below the threshold
    (1e-4 by default): gaps just below, at and just above it, zero, and
    +inf (k = N)."""
    gaps = np.array([0.0, 5e-5, 9.99e-5, 1e-4, 1.0001e-4, 0.3, np.inf])
    assert O.near_tie_tokens(gaps).tolist() == [True, True, True, False, False, False, False]
    assert O.near_tie_tokens(np.array([0.5, 1.5]), 1.0).tolist() == [True, False]
    assert O.near_tie_tokens(np.array([2e-8]), 1e-8).tolist() == [False]
    # the gap the oracle's own routing reports: a planted tie is near, a
    # clear winner is not
    z = np.array([[1.0, 1.0 + 5e-5, -2.0], [3.0, 0.0, -1.0]])
    r = O.route(z, np.eye(3), 1, O.MODE_SOFTMAX_FULL)
    assert O.near_tie_tokens(r.gap).tolist() == [True, False], r.gap


ALL_PINS = [v for k_, v in sorted(globals().items()) if k_.startswith("pin_")]
