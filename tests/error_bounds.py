"""Rounding-error scales for the GPU parity checks (test infrastructure).

A computed gradient element is a sum of products that the GPU evaluates
with fp32 accumulation and, on the bf16 path, a few intermediates rounded to
bf16. Its error is bounded by a small multiple of the unit roundoff times the
sum of the MAGNITUDES of the terms along the whole chain, not times the
element's own value, which can cancel to nothing. `grad_scales` returns that
magnitude for every gradient element: the oracle's backward (steps of
oracle.moe_oracle.layer_backward, same selection and dispatch) evaluated with
every product taken on absolute values, and with the first-order propagation
of each intermediate's error through the nonlinear steps:

    y = sum_i a_i b_i               M_y = sum_i M_a,i |b_i| + |a_i| M_b,i
    act = SiLU(gp) up               M_act = |SiLU(gp)| M_up + |SiLU'(gp) up| M_gp
    dgp = v up SiLU'(gp)            M_dgp = M_v |up SiLU'| + |v SiLU'| M_up
                                            + |v up SiLU''| M_gp
    du = v SiLU(gp)                 M_du = M_v |SiLU| + |v SiLU'| M_gp

(inputs and weights are exact, so their M is their magnitude). A correct
implementation whose every rounding is at most u relative to the quantity
rounded then satisfies |error| <= c u M element by element, c the number of
roundings on the longest path, with no assumption on how the errors
correlate.

That bound is exact but loose where terms cancel: a sum of n random-sign
terms is about sqrt(n) smaller than its magnitude, and so is its rounding
error, so a systematic 5% error on such an element hides under it. The same
pass therefore also propagates a NOISE scale, the standard deviation of the
error when every rounding is an independent error uniform in +-u of the
rounded value (variance (u |q|)^2 / 3), at the library's rounding points,
with fp32 accumulation noise u_f32 sqrt(n) M for a sum of n terms:

    var(sum_i a_i x_i) = sum_i a_i^2 var(x_i) + x_i^2 var(a_i) + accumulation
    var(f(x)) = f'(x)^2 var(x);   stored q: + (u |q|)^2 / 3

The checks hold each element's error to a dozen of these standard deviations
and each tensor's root-mean-square error to a few.

The router logits z are themselves fp32 sums of d products, and the gates
and the router-logit gradient are nonlinear in them. Their error reaches
the gradients by first-order propagation (`logit_propagation`): the
Jacobians of the gates and of dL/dz in each logit column, by central
differences of the oracle's own gate and statistics backward (the
selection, dL/dg and the counts held fixed). It matters where a gradient is
proportional to a logit that cancels: the z-loss term of a token is
lse(z) P, and a logit near zero carries a large relative error.

`comparison_scores` gives the same kind of bound for the scores the router
orders its slots by.
"""
import math

import numpy as np

from oracle import moe_oracle as O

U_F32 = 2.0 ** -24
U_BF16 = 2.0 ** -8
SQRT3 = math.sqrt(3.0)


def _a(x):
    return np.abs(np.asarray(x, np.float64))


def silu_grad2(x):
    """d^2/dx^2 [x sigmoid(x)] = s (1 - s) (2 + x (1 - 2 s)), s = sigmoid(x)."""
    x = np.asarray(x, np.float64)
    s = O.sigmoid(x)
    return s * (1.0 - s) * (2.0 + x * (1.0 - 2.0 * s))


def expert_scales(x, wg, wu, wd, dout, dy_rows, g=None, u_store=0.0, m_gz=None, v_g=None):
    """Magnitudes and noise for one expert's rows x [n, d] with output
    gradients dout (= gate * dy; ``g`` the gates, 1 for the shared expert):
    returns two dicts, M (magnitudes) and S (noise standard deviations), with
    keys dx [n, d], dw_gate, dw_up, dw_down (the weights' shapes) and dg [n]
    (the slot's dL/dg = <dy, E(x)>). ``u_store`` is the unit roundoff of the
    stored intermediates and outputs (bf16, or fp32). ``m_gz`` and ``v_g``
    [n] are the magnitude the gates take from their logits and the gates'
    error variance (logit_propagation); None for exact gates."""
    x = np.asarray(x, np.float64)
    wg, wu, wd = (np.asarray(w, np.float64) for w in (wg, wu, wd))
    dout = np.asarray(dout, np.float64)
    dy_rows = np.asarray(dy_rows, np.float64)
    n, d = x.shape
    dff = wg.shape[0]
    g = np.ones(n) if g is None else np.asarray(g, np.float64)
    ax, awg, awu, awd = _a(x), _a(wg), _a(wu), _a(wd)
    x2, wg2, wu2, wd2 = ax ** 2, awg ** 2, awu ** 2, awd ** 2
    rnd = lambda q: (u_store / SQRT3 * np.abs(q)) ** 2        # variance of one rounding
    acc = lambda m, nterms: (U_F32 * math.sqrt(nterms) * m) ** 2
    # forward recompute (fp32)
    gp, up = x @ wg.T, x @ wu.T
    m_gp, m_up = ax @ awg.T, ax @ awu.T
    v_gp, v_up = acc(m_gp, d), acc(m_up, d)
    s, s1, s2 = O.silu(gp), O.silu_grad(gp), silu_grad2(gp)
    act = s * up
    m_act = _a(s) * m_up + _a(s1 * up) * m_gp
    v_actf = (s1 * up) ** 2 * v_gp + s ** 2 * v_up
    v_act = v_actf + rnd(act)                                    # stored
    m_out = m_act @ awd.T                                        # E(x) = act W_down^T
    # v = W_down^T dy (fp32), dg = <v, act> (fp32 operands)
    vn = dy_rows @ wd
    m_vn = _a(dy_rows) @ awd
    v_vn = acc(m_vn, d)
    m_dg = (_a(dy_rows) * m_out).sum(axis=-1)
    v_dg = (act ** 2 * v_vn + vn ** 2 * v_actf).sum(axis=-1) + acc(m_dg, dff)
    # SwiGLU backward; the gate's own error enters through g dy and g v
    m_gz = np.zeros(n) if m_gz is None else np.asarray(m_gz, np.float64)
    v_g = np.zeros(n) if v_g is None else np.asarray(v_g, np.float64)
    v_ = g[:, None] * vn
    adout = _a(dout) + m_gz[:, None] * _a(dy_rows)
    m_v = adout @ awd
    v_v = g[:, None] ** 2 * v_vn
    du = v_ * s
    dgp = v_ * up * s1
    m_du = m_v * _a(s) + _a(v_ * s1) * m_gp
    m_dgp = m_v * _a(up * s1) + _a(v_ * s1) * m_up + _a(v_ * up * s2) * m_gp
    v_du0 = s ** 2 * v_v + (v_ * s1) ** 2 * v_gp + rnd(du)
    v_dgp0 = (up * s1) ** 2 * v_v + (v_ * s1) ** 2 * v_up + (v_ * up * s2) ** 2 * v_gp + rnd(dgp)
    # a gate's error scales its whole row of du and dgp: independent between
    # rows (the weight gradients), one common factor within a row (dx)
    du_g, dgp_g = vn * s, vn * up * s1                 # d du / dg, d dgp / dg
    v_du = v_du0 + du_g ** 2 * v_g[:, None]
    v_dgp = v_dgp0 + dgp_g ** 2 * v_g[:, None]
    # weight gradients over the rows (dout packed in the stored dtype)
    v_dout = rnd(dout) + dy_rows ** 2 * v_g[:, None]
    dwd = dout.T @ act
    m_dwd = adout.T @ m_act
    v_dwd = v_dout.T @ act ** 2 + (dout ** 2).T @ v_act + acc(m_dwd, n) + rnd(dwd)
    dwg, dwu = dgp.T @ x, du.T @ x
    m_dwg, m_dwu = m_dgp.T @ ax, m_du.T @ ax
    v_dwg = v_dgp.T @ x2 + acc(m_dwg, n) + rnd(dwg)
    v_dwu = v_du.T @ x2 + acc(m_dwu, n) + rnd(dwu)
    # row gradients of h (each row stored)
    dx = dgp @ wg + du @ wu
    m_dx = m_dgp @ awg + m_du @ awu
    v_dx = (v_dgp0 @ wg2 + v_du0 @ wu2 + (dgp_g @ wg + du_g @ wu) ** 2 * v_g[:, None]
            + acc(m_dx, 2 * dff) + rnd(dx))
    M = dict(dx=m_dx, dw_gate=m_dwg, dw_up=m_dwu, dw_down=m_dwd, dg=m_dg)
    S = dict(dx=v_dx, dw_gate=v_dwg, dw_up=v_dwu, dw_down=v_dwd, dg=v_dg)
    return M, S


class GradScales:
    """Per-element magnitudes (or noise standard deviations), shaped as
    oracle.LayerGrads' fields."""

    def __init__(self, dh, dw_router, db_router, dw_gate, dw_up, dw_down, dsh, dg):
        self.dh, self.dw_router, self.db_router = dh, dw_router, db_router
        self.dw_gate, self.dw_up, self.dw_down = dw_gate, dw_up, dw_down
        self.dsh, self.dg = dsh, dg


def _gate_jacobian(r, mode):
    """d dz[t, ids[t, i]] / d dg[t, j] (modes A, C; [T, k, k]) or
    d dz[t, :] / d dg[t, j] (mode B; [T, N, k])."""
    z, ids, g = r.z, r.ids, r.gates
    T, k = ids.shape
    if mode == O.MODE_SOFTMAX_RENORM:
        return g[:, :, None] * (np.eye(k)[None] - g[:, None, :])
    if mode == O.MODE_SOFTMAX_FULL:
        P = O.softmax(z)
        N = z.shape[1]
        oh = np.zeros((T, N, k))
        for j in range(k):
            oh[np.arange(T), ids[:, j], j] = 1.0
        Pl = np.take_along_axis(P, ids, axis=-1)                 # [T, k]
        return P[:, :, None] * (oh - Pl[:, None, :])
    s_sel = np.take_along_axis(O.sigmoid(z), ids, axis=-1)
    S = s_sel.sum(axis=-1, keepdims=True)
    return ((np.eye(k)[None] - g[:, None, :]) / S[:, :, None]) * (s_sel * (1 - s_sel))[:, :, None]


def router_scales(r, m_dg, counts, k, mode, alpha, d_laux, d_zloss, v_dg=None):
    """Magnitude of the router-logit gradient [T, N]: the gate Jacobian of
    the mode (oracle.gate_backward) applied to magnitudes, plus the
    auxiliary terms' (oracle.stats_backward) magnitudes. With v_dg (the
    variance of dL/dg), also the variance of dz: the Jacobian's squares
    applied to it, plus fp32 evaluation noise."""
    z = r.z
    T, N = z.shape
    ids, g = r.ids, _a(r.gates)
    m = np.zeros((T, N))
    if mode == O.MODE_SOFTMAX_RENORM:
        inner = (g * m_dg).sum(axis=-1, keepdims=True)
        np.put_along_axis(m, ids, g * (m_dg + inner), axis=-1)
    elif mode == O.MODE_SOFTMAX_FULL:
        P = O.softmax(z)
        a = np.zeros((T, N))
        np.put_along_axis(a, ids, m_dg, axis=-1)
        m = P * (a + (P * a).sum(axis=-1, keepdims=True))
    else:
        s = O.sigmoid(z)
        s_sel = np.take_along_axis(s, ids, axis=-1)
        S = s_sel.sum(axis=-1, keepdims=True)
        ds = (m_dg + (g * m_dg).sum(axis=-1, keepdims=True)) / S
        np.put_along_axis(m, ids, ds * s_sel * (1.0 - s_sel), axis=-1)
    if T and d_laux:
        f = np.asarray(counts, np.float64) / (T * k)
        a = np.broadcast_to(abs(d_laux * alpha * N) * f / T, (T, N))
        if mode in (O.MODE_SOFTMAX_RENORM, O.MODE_SOFTMAX_FULL):
            P = O.softmax(z)
            m = m + P * (a + (P * a).sum(axis=-1, keepdims=True))
        else:
            s = O.sigmoid(z)
            S = s.sum(axis=-1, keepdims=True)
            P = s / S
            m = m + (a + (P * a).sum(axis=-1, keepdims=True)) / S * s * (1.0 - s)
    if T and d_zloss:
        mx = z.max(axis=-1, keepdims=True)
        lse = mx + np.log(np.exp(z - mx).sum(axis=-1, keepdims=True))
        m = m + abs(d_zloss) * (2.0 / T) * np.abs(lse) * O.softmax(z)
    if v_dg is None:
        return m
    J2 = _gate_jacobian(r, mode) ** 2
    var = np.zeros((T, N))
    if mode == O.MODE_SOFTMAX_FULL:
        var = (J2 * v_dg[:, None, :]).sum(axis=-1)
    else:
        np.put_along_axis(var, ids, (J2 * v_dg[:, None, :]).sum(axis=-1), axis=-1)
    # fp32 evaluation of the logit gradient: a few roundings of its terms
    var = var + (8.0 * U_F32 * m) ** 2
    return m, var


def logit_scales(h, w_router, b_router=None):
    """Magnitude M_z [T, N] of each router logit's terms (|h| |W_r|^T + |b|)
    and the variance of its fp32 evaluation: d products (exact for bf16
    operands, fused into the adds for fp32 ones) accumulated in fp32, the
    bias added, the result rounded once."""
    h, wr = np.asarray(h, np.float64), np.asarray(w_router, np.float64)
    nterms = h.shape[1]
    m_z, z = _a(h) @ _a(wr).T, h @ wr.T
    if b_router is not None:
        m_z = m_z + _a(b_router)[None, :]
        z = z + np.asarray(b_router, np.float64)[None, :]
        nterms += 1
    return m_z, (U_F32 * math.sqrt(max(nterms, 1)) * m_z) ** 2 + (U_F32 / SQRT3 * z) ** 2


def gates_of(z, ids, mode):
    """Gate values of the slots ids [T, k] for the logits z [T, N]: the gate
    step of oracle.route for a fixed selection."""
    if mode == O.MODE_SIGMOID_BIAS_RENORM:
        s = np.take_along_axis(O.sigmoid(z), ids, axis=-1)
        return s / s.sum(axis=-1, keepdims=True)
    p = np.take_along_axis(O.softmax(z), ids, axis=-1)
    return p / p.sum(axis=-1, keepdims=True) if mode == O.MODE_SOFTMAX_RENORM else p


def logit_propagation(r, dg, counts, k, mode, alpha, d_laux, d_zloss, w_router, m_z, v_z,
                      step=1e-6):
    """First-order propagation of the logits' error (magnitude m_z, variance
    v_z, both [T, N]) into the gates and the router-logit gradient dL/dz =
    oracle.gate_backward + oracle.stats_backward (dL/dg, the selection and
    the counts held fixed). Each row of either depends only on its token's
    logits, so the Jacobian column d / dz[:, i] of every token comes from two
    evaluations with column i moved by +-step. An entry below the rounding
    noise of that difference is no dependence and counts as zero. Returns
    (m_g, v_g) [T, k], (m_dz, v_dz) [T, N] and v_dhr [T, d], the variance of
    dL/dz W_r with the errors of one token's logits shared by its d entries."""
    z = np.asarray(r.z, np.float64)
    T, N = z.shape
    k_ = r.ids.shape[1]
    wr = np.asarray(w_router, np.float64)
    m_g, v_g = np.zeros((T, k_)), np.zeros((T, k_))
    m_dz, v_dz = np.zeros((T, N)), np.zeros((T, N))
    v_dhr = np.zeros((T, wr.shape[1]))
    if T == 0:
        return m_g, v_g, m_dz, v_dz, v_dhr

    def at(zz):
        g = gates_of(zz, r.ids, mode)
        rr = O.Routing(r.ids, g, zz, r.sel, r.gap, r.stat_prob)
        return g, (O.gate_backward(rr, dg, mode)
                   + O.stats_backward(rr, counts, k, mode, alpha, d_laux, d_zloss))

    eps = 64.0 * np.finfo(np.float64).eps / (2.0 * step)

    def jac(fp, fm):
        j = (fp - fm) / (2.0 * step)
        return np.where(np.abs(j) > eps * (np.abs(fp) + np.abs(fm)), j, 0.0)

    for i in range(N):
        zp, zm = z.copy(), z.copy()
        zp[:, i] += step
        zm[:, i] -= step
        (gp, dzp), (gm, dzm) = at(zp), at(zm)
        jg, jd = jac(gp, gm), jac(dzp, dzm)
        mi, vi = m_z[:, i:i + 1], v_z[:, i:i + 1]
        m_g += np.abs(jg) * mi
        v_g += jg ** 2 * vi
        m_dz += np.abs(jd) * mi
        v_dz += jd ** 2 * vi
        v_dhr += (jd @ wr) ** 2 * vi
    return m_g, v_g, m_dz, v_dz, v_dhr


def grad_scales(h, w_router, k, mode, weights_of, dy, b_router=None, b_select=None,
                shared=None, alpha=0.01, capacity_factor=None, d_laux=0.0, d_zloss=0.0,
                ids=None, u_store=None, ref=None):
    """Magnitudes of every gradient oracle.layer_backward returns, for the
    same arguments (the selection fixed by ``ids``). With ``u_store`` (the
    unit roundoff of the stored intermediates: U_BF16 or U_F32) returns the
    pair (magnitudes, noise standard deviations) instead; ``ref`` is that
    call's oracle.layer_backward result when the caller has it."""
    h, dy = np.asarray(h, np.float64), np.asarray(dy, np.float64)
    T, d = h.shape
    wr = np.asarray(w_router, np.float64)
    N = wr.shape[0]
    us = U_F32 if u_store is None else u_store
    rnd = lambda q: (us / SQRT3 * np.abs(q)) ** 2
    r = O.route(h, wr, k, mode, b_router, b_select, None, ids)
    cap = O.expert_capacity(capacity_factor, T, k, N) if capacity_factor else None
    disp = O.dispatch(r.ids, N, cap)
    if ref is None:
        ref = O.layer_backward(h, wr, k, mode, weights_of, dy, b_router, b_select, shared,
                               alpha, None, capacity_factor, d_laux, d_zloss, ids=r.ids)
    # the logits' own fp32 error, through the gates and dL/dz; each gate
    # also takes a few roundings of its own (exp, sum, quotient)
    m_z, v_z = logit_scales(h, wr, b_router)
    m_gz, v_g, m_dzz, v_dzz, v_dhz = logit_propagation(r, ref.dg, disp.counts, k, mode, alpha,
                                                       d_laux, d_zloss, wr, m_z, v_z)
    v_g = v_g + 4.0 * (U_F32 / SQRT3 * r.gates) ** 2
    m_dh, v_dh = np.zeros((T, d)), np.zeros((T, d))
    m_dg, v_dg = np.zeros((T, k)), np.zeros((T, k))
    M_w = {key: [] for key in ("dw_gate", "dw_up", "dw_down")}
    V_w = {key: [] for key in ("dw_gate", "dw_up", "dw_down")}
    for e in range(N):
        wg, wu, wd = weights_of(e)
        flats = disp.perm_src[disp.offsets[e]:disp.offsets[e + 1]]
        t, j = flats // k, flats % k
        gt = r.gates[t, j]
        Me, Ve = expert_scales(h[t], wg, wu, wd, gt[:, None] * dy[t], dy[t], gt, us,
                               m_gz[t, j], v_g[t, j])
        np.add.at(m_dh, t, Me["dx"])
        np.add.at(v_dh, t, Ve["dx"])
        m_dg[t, j] = Me["dg"]
        v_dg[t, j] = Ve["dg"]
        for key in M_w:
            M_w[key].append(Me[key])
            V_w[key].append(Ve[key])
    msh = vsh = None
    if shared is not None:
        Ms, Vs = expert_scales(h, *shared, dy, dy, None, us)
        m_dh += Ms["dx"]
        v_dh += Vs["dx"]
        msh = (Ms["dw_gate"], Ms["dw_up"], Ms["dw_down"])
        vsh = (Vs["dw_gate"], Vs["dw_up"], Vs["dw_down"])
    m_dz, v_dz = router_scales(r, m_dg, disp.counts, k, mode, alpha, d_laux, d_zloss, v_dg)
    m_dz = m_dz + m_dzz
    ah, awr = _a(h), _a(wr)
    m_dhr = m_dz @ awr
    m_dh += m_dhr
    M = GradScales(m_dh, m_dz.T @ ah, m_dz.sum(axis=0), np.stack(M_w["dw_gate"]),
                   np.stack(M_w["dw_up"]), np.stack(M_w["dw_down"]), msh, m_dg)
    if u_store is None:
        return M
    # the router's contributions: dz rounded to the stored dtype before it
    # meets W_r and h; its dh rows stored; dh rounded once more. A logit's
    # error moves every entry of its token's dz row together, so its share
    # of dz W_r is v_dhz, not the entry-wise sum.
    v_dzb = v_dz + rnd(ref.dz)
    dhr = ref.dz @ wr
    v_dh = (v_dh + v_dzb @ wr ** 2 + v_dhz + (U_F32 * math.sqrt(N) * m_dhr) ** 2 + rnd(dhr)
            + rnd(ref.dh))
    v_dzb = v_dzb + v_dzz
    acc_t = lambda m: (U_F32 * math.sqrt(max(T, 1)) * m) ** 2
    Vv = GradScales(v_dh, v_dzb.T @ ah ** 2 + acc_t(M.dw_router),
                    (v_dz + v_dzz).sum(axis=0) + acc_t(M.db_router), np.stack(V_w["dw_gate"]),
                    np.stack(V_w["dw_up"]), np.stack(V_w["dw_down"]), vsh, v_dg)
    S = GradScales(*(None if f is None else (tuple(np.sqrt(x) for x in f) if isinstance(f, tuple)
                                              else np.sqrt(f))
                     for f in (Vv.dh, Vv.dw_router, Vv.db_router, Vv.dw_gate, Vv.dw_up,
                               Vv.dw_down, Vv.dsh, Vv.dg)))
    return M, S


# ------------------------------------------------------- selection scores
# Logit error model: z is a sum of d products accumulated in fp32 (bf16 x
# bf16 products are exact in fp32; fp32 products are fused into the adds).
# Higham & Mary's probabilistic bound for such a sum (SIAM J. Sci. Comput.
# 41(5), 2019, Theorem 3.1) is lambda sqrt(d) u sum_c |w_c h_c| with a
# failure probability below 2 exp(-lambda^2 / 2) per sum: lambda = 6 gives
# 3e-8. The worst-case bound (d u instead of sqrt(d) u) would allow slot
# swaps sqrt(d) times wider.
LAMBDA = 6.0


def ulp32(x):
    """Spacing of float32 numbers at |x| (the smallest normal's below it)."""
    x = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -126)))
    return np.exp2(e - 23)


def logit_error(h, w_router, b_router=None):
    """Bound on the fp32 error of each logit z[t, i] [T, N]."""
    h, wr = np.asarray(h, np.float64), np.asarray(w_router, np.float64)
    d = h.shape[1]
    mz = _a(h) @ _a(wr).T
    z = h @ wr.T
    if b_router is not None:
        mz = mz + _a(b_router)[None, :]
        z = z + np.asarray(b_router, np.float64)[None, :]
    return LAMBDA * math.sqrt(d) * U_F32 * mz + 2.0 * ulp32(z)


def comparison_scores(routing, mode, h, w_router, b_router=None, b_select=None):
    """The scores the GPU orders its slots by, computed exactly (the logits
    z in the softmax modes, which order the experts as the probabilities
    do; sigma(z) + b_select in mode C), and a bound on the GPU's fp32 error
    of each: the logit error, through sigma' in mode C, plus a few ulps for
    evaluating sigma and adding the bias."""
    dz = logit_error(h, w_router, b_router)
    z = routing.z
    if mode != O.MODE_SIGMOID_BIAS_RENORM:
        return z, dz
    s = O.sigmoid(z)
    sel = s + np.asarray(b_select, np.float64)[None, :]
    return sel, s * (1.0 - s) * dz + 4.0 * ulp32(s) + 2.0 * ulp32(sel)
