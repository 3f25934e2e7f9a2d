"""The rounding-error scales behind the GPU parity checks, on the CPU.

error_bounds.grad_scales must (1) bound every gradient's exact value (a sum's
magnitude is at least its value), (2) cover the error a bf16 implementation
with the library's rounding points makes (an emulation of those roundings in
numpy passes the bound), and (3) still fail a gradient that is wrong: a row
that is small because its inputs are small (not because it cancels) is held
to its own size, which the previous per-row check with a tensor-wide floor
did not do. The slot-order allowance of check_ids is checked against hand
cases of the fp32 score bound."""
import math

import numpy as np
import pytest

import error_bounds as EB
import workloads as W
from helpers import GRAD_TOL, check_grad, check_grad_elems, check_grad_noise, check_ids
from oracle import moe_oracle as O


def _rb(x):
    """Round to bf16 (round to nearest even), back in float64."""
    return W.round_to_bf16(np.asarray(x, np.float32)).astype(np.float64)


def _inputs(seed, T, d, N, k, dff, dfs, mode):
    inp = W.random_small(T, d, N, k, dff, dfs, W.DTYPE_BF16, mode, seed=seed, router_bias=True)
    rng = np.random.default_rng(seed + 100)
    dy = _rb(rng.standard_normal((T, d)))
    return inp, dy


def _args(inp, dy, k, mode):
    sh = None if inp.get("sh_gate") is None else (inp["sh_gate"], inp["sh_up"], inp["sh_down"])
    return (inp["h"], inp["w_router"], k, mode,
            O.weights_getter(inp["w_gate"], inp["w_up"], inp["w_down"]), dy, inp["b_router"],
            inp["b_select"], sh, 0.01)


def _emulated_bf16_backward(inp, dy, k, mode, cf, d_laux, d_zloss):
    """The oracle's chain of the backward with the bf16 path's rounding
    points: the SwiGLU output, the gate/up gradients [dgp | du] and g dy
    stored as bf16; each kept row's dh contribution, the shared expert's and
    the router's stored as bf16, then summed and rounded again; the router-
    logit gradient rounded to bf16 before it meets W_r and h; every gradient
    but dW_r / db_r rounded to bf16 at the end."""
    h = np.asarray(inp["h"], np.float64)
    wr = np.asarray(inp["w_router"], np.float64)
    T, d = h.shape
    N = wr.shape[0]
    r = O.route(h, wr, k, mode, inp["b_router"], inp["b_select"])
    cap = O.expert_capacity(cf, T, k, N) if cf else None
    disp = O.dispatch(r.ids, N, cap)
    dh = np.zeros((T, d))
    dg = np.zeros((T, k))
    dwg, dwu, dwd = [], [], []

    def expert(x, wg, wu, wd, g, dyr):
        gp, up = x @ wg.T, x @ wu.T
        act = _rb(O.silu(gp) * up)
        vn = dyr @ wd                       # W_down^T dy, before the gate
        v = g[:, None] * vn
        du = _rb(v * O.silu(gp))
        dgp = _rb(v * up * O.silu_grad(gp))
        dgate = np.sum(vn * O.silu(gp) * up, axis=-1)
        dout = _rb(g[:, None] * dyr)
        return (_rb(dgp @ wg + du @ wu), _rb(dgp.T @ x), _rb(du.T @ x), _rb(dout.T @ act), dgate)

    for e in range(N):
        flats = disp.perm_src[disp.offsets[e]:disp.offsets[e + 1]]
        t, j = flats // k, flats % k
        wg, wu, wd = (np.asarray(inp[key][e], np.float64) for key in ("w_gate", "w_up", "w_down"))
        dx, a, b, c, dgate = expert(h[t], wg, wu, wd, r.gates[t, j], dy[t])
        np.add.at(dh, t, dx)
        dg[t, j] = dgate
        dwg.append(a)
        dwu.append(b)
        dwd.append(c)
    dsh = None
    if inp.get("sh_gate") is not None:
        sg, su, sd = (np.asarray(inp[key], np.float64) for key in ("sh_gate", "sh_up", "sh_down"))
        dx, a, b, c, _ = expert(h, sg, su, sd, np.ones(T), dy)
        dh += dx
        dsh = (a, b, c)
    dz = O.gate_backward(r, dg, mode) + O.stats_backward(r, disp.counts, k, mode, 0.01, d_laux,
                                                         d_zloss)
    dh = _rb(dh + _rb(_rb(dz) @ wr))
    return O.LayerGrads(dh, _rb(dz).T @ h, dz.sum(axis=0), np.stack(dwg), np.stack(dwu),
                        np.stack(dwd), dsh, dg, dz)


CASES = [
    # seed, T, d, N, k, d_ff, d_ff_shared, mode, capacity, d_laux, d_zloss
    (1, 40, 32, 6, 2, 48, 0, O.MODE_SOFTMAX_RENORM, None, 0.0, 0.0),
    (2, 37, 48, 9, 3, 40, 24, O.MODE_SIGMOID_BIAS_RENORM, 0.75, 0.7, 0.2),
    (3, 50, 32, 5, 2, 32, 16, O.MODE_SOFTMAX_FULL, None, 0.5, 0.3),
    (4, 30, 64, 3, 1, 32, 0, O.MODE_SOFTMAX_RENORM, None, 1.0, 0.0),
]


def _fields(g):
    out = dict(dh=g.dh, dw_router=g.dw_router, db_router=g.db_router, dw_gate=g.dw_gate,
               dw_up=g.dw_up, dw_down=g.dw_down, dg=g.dg)
    if g.dsh is not None:
        out.update(dsh_gate=g.dsh[0], dsh_up=g.dsh[1], dsh_down=g.dsh[2])
    return out


def test_silu_second_derivative():
    x = np.linspace(-8.0, 8.0, 101)
    eps = 1e-5
    fd = (O.silu_grad(x + eps) - O.silu_grad(x - eps)) / (2 * eps)
    assert np.allclose(EB.silu_grad2(x), fd, rtol=0, atol=1e-8)


@pytest.mark.parametrize("case", CASES, ids=[str(c[0]) for c in CASES])
def test_scales_bound_values_and_bf16_emulation(case):
    seed, T, d, N, k, dff, dfs, mode, cf, d_laux, d_zloss = case
    inp, dy = _inputs(seed, T, d, N, k, dff, dfs, mode)
    args = _args(inp, dy, k, mode)
    ref = O.layer_backward(*args, None, cf, d_laux, d_zloss)
    sc, nz = EB.grad_scales(*args, cf, d_laux, d_zloss, ids=ref_ids(inp, k, mode),
                            u_store=EB.U_BF16, ref=ref)
    assert np.array_equal(EB.grad_scales(*args, cf, d_laux, d_zloss,
                                         ids=ref_ids(inp, k, mode)).dh, sc.dh)
    emu = _emulated_bf16_backward(inp, dy, k, mode, cf, d_laux, d_zloss)
    R, S, Z, E = _fields(ref), _fields(sc), _fields(nz), _fields(emu)
    assert R.keys() == S.keys() == E.keys() == Z.keys()
    worst, nmax, nrms = 0.0, 0.0, 0.0
    for key in R:
        # (1) the magnitude of the terms bounds the value
        assert np.all(S[key] >= np.abs(R[key]) * (1 - 1e-12)), key
        # (2) bf16 rounding at the library's points stays inside the bound
        worst = max(worst, check_grad_elems(E[key], R[key], S[key], GRAD_TOL[W.DTYPE_BF16], key))
        # (3) and inside the noise gate
        a, b = check_grad_noise(E[key], R[key], Z[key], key)
        nmax, nrms = max(nmax, a), max(nrms, b)
    assert worst > 0.0
    print(f"case {seed}: bf16 emulation max |error| / scale {worst:.2e} "
          f"(bound {GRAD_TOL[W.DTYPE_BF16]:.2e}); noise max {nmax:.2f}, worst rms {nrms:.2f}")


def ref_ids(inp, k, mode):
    return O.route(inp["h"], inp["w_router"], k, mode, inp["b_router"], inp["b_select"]).ids


def test_small_row_held_to_its_own_size():
    """A token whose upstream gradient is 1e-3 of the others' has a dh row at
    that scale. Its row made 20% wrong passes a per-row check whose scale is
    floored at 1e-2 of the tensor's largest value, and fails the checks: the
    noise of that row is at the row's own scale. (The exact magnitude bound
    alone passes it here: with unit-variance test weights the router term's
    magnitude exceeds its value a hundredfold.)"""
    inp, dy = _inputs(5, 40, 32, 6, 2, 48, 0, O.MODE_SOFTMAX_RENORM)
    dy[7] *= 1e-3
    args = _args(inp, dy, 2, O.MODE_SOFTMAX_RENORM)
    ref = O.layer_backward(*args)
    sc, nz = EB.grad_scales(*args, ids=ref_ids(inp, 2, O.MODE_SOFTMAX_RENORM),
                            u_store=EB.U_BF16, ref=ref)
    check_grad(_rb(ref.dh), ref.dh, sc.dh, nz.dh, GRAD_TOL[W.DTYPE_BF16], "dh")
    bad = ref.dh.copy()
    bad[7] *= 1.2
    floor = np.maximum(np.abs(ref.dh).max(axis=1), 1e-2 * np.abs(ref.dh).max())
    assert (np.abs(bad - ref.dh).max(axis=1) / floor).max() <= 2e-2      # the old check passes
    with pytest.raises(AssertionError):
        check_grad(bad, ref.dh, sc.dh, nz.dh, GRAD_TOL[W.DTYPE_BF16], "dh")


@pytest.mark.parametrize("what", ["dw_down_missing_row", "dw_gate_sign", "dz_mode_b_selected_only",
                                  "dg_scaled", "shared_missing"])
def test_planted_gradient_errors_fail(what):
    mode = O.MODE_SOFTMAX_FULL if what == "dz_mode_b_selected_only" else O.MODE_SOFTMAX_RENORM
    dfs = 16 if what == "shared_missing" else 0
    inp, dy = _inputs(6, 24, 32, 8, 2, 32, dfs, mode)
    args = _args(inp, dy, 2, mode)
    ref = O.layer_backward(*args)
    ids = ref_ids(inp, 2, mode)
    m, nz = EB.grad_scales(*args, ids=ids, u_store=EB.U_BF16, ref=ref)
    tol = GRAD_TOL[W.DTYPE_BF16]
    disp = O.dispatch(ids, 8)
    counts = disp.counts

    def check_grad_elems(y, y_ref, scale, tol_, what_):
        return check_grad(y, y_ref, scale, getattr(nz, what_), tol_, what_)

    sc = m
    with pytest.raises(AssertionError):
        if what == "dw_down_missing_row":
            # an expert with two rows, one of them left out of its weight gradient
            e = int(np.argmin(np.where(counts > 1, counts, 1 << 30)))
            f = disp.perm_src[disp.offsets[e]]
            t, j = f // 2, f % 2
            x = np.asarray(inp["h"], np.float64)[t:t + 1]
            wg, wu, wd = (np.asarray(inp[key][e], np.float64) for key in ("w_gate", "w_up", "w_down"))
            _, _, _, one = O.expert_ffn_backward(x, wg, wu, wd, ref_gate(inp, mode, t, j) * dy[t:t + 1])
            bad = ref.dw_down.copy()
            bad[e] -= one
            check_grad_elems(bad, ref.dw_down, sc.dw_down, tol, "dw_down")
        elif what == "dw_gate_sign":
            bad = ref.dw_gate.copy()
            e = int(np.argmax(counts))
            bad[e, 3] = -bad[e, 3]
            check_grad_elems(bad, ref.dw_gate, sc.dw_gate, tol, "dw_gate")
        elif what == "dz_mode_b_selected_only":
            r = O.route(inp["h"], inp["w_router"], 2, mode, inp["b_router"])
            dz = O.gate_backward(r, ref.dg, mode)
            sel = np.zeros_like(dz, bool)
            np.put_along_axis(sel, r.ids, True, axis=-1)
            dz_bad = np.where(sel, dz, 0.0) + (ref.dz - dz)
            check_grad_elems(dz_bad.T @ np.asarray(inp["h"], np.float64), ref.dw_router,
                             sc.dw_router, tol, "dw_router")
        elif what == "dg_scaled":
            check_grad_elems(ref.dg * 1.05, ref.dg, sc.dg, tol, "dg")
        else:
            sh = (inp["sh_gate"], inp["sh_up"], inp["sh_down"])
            dx = O.expert_ffn_backward(np.asarray(inp["h"], np.float64), *sh, dy)[0]
            check_grad_elems(ref.dh - dx, ref.dh, sc.dh, tol, "dh")


def ref_gate(inp, mode, t, j):
    return O.route(inp["h"], inp["w_router"], 2, mode, inp["b_router"]).gates[t, j]


# ------------------------------------------------------------ slot order
def test_ulp32():
    assert EB.ulp32(1.0) == 2.0 ** -23
    assert EB.ulp32(0.97) == 2.0 ** -24
    assert EB.ulp32(-3.0) == 2.0 ** -22
    assert EB.ulp32(0.0) == 2.0 ** -149


def test_logit_error_bound_covers_fp32_sums():
    """The bound holds for the fp32 dot products numpy forms in several
    orders (sequential, pairwise) on random rows of the shapes the library
    routes (d up to 7168)."""
    rng = np.random.default_rng(8)
    for d in (32, 1024, 7168):
        h = _rb(rng.standard_normal((16, d)) / math.sqrt(d))
        w = _rb(rng.standard_normal((8, d)))
        bound = EB.logit_error(h, w)
        exact = h @ w.T
        seq = np.zeros((16, 8), np.float32)
        h32, w32 = h.astype(np.float32), w.astype(np.float32)
        for c in range(d):
            seq += h32[:, c:c + 1] * w32[None, :, c]
        pair = h32 @ w32.T
        for got in (seq, pair):
            assert np.all(np.abs(got.astype(np.float64) - exact) <= bound)


def test_check_ids_slot_order():
    """Two selected experts whose sigmoid scores are 2.4e-8 apart (below
    one fp32 ulp at 0.97) may come in either order; 1e-4 apart they may not,
    although that is within the previous NEAR_TIE allowance."""
    d, N, k = 4, 4, 2
    b_sel = np.zeros(N)
    for gap, ok in ((2.4e-8, True), (1e-4, False)):
        s_hi = 0.97
        z = np.array([-2.0, math.log(s_hi / (1 - s_hi)),
                      math.log((s_hi + gap) / (1 - s_hi - gap)), -3.0])
        w = np.diag(z)                           # z = w h with h = (1, 1, 1, 1)
        hh = np.ones((1, d))
        r = O.route(hh, w, k, O.MODE_SIGMOID_BIAS_RENORM, None, b_sel)
        assert sorted(r.ids[0].tolist()) == [1, 2]
        swapped = np.array([[1, 2]])              # the lower score first
        if ok:
            check_ids(swapped, r, k, O.MODE_SIGMOID_BIAS_RENORM, hh, w, None, b_sel)
        else:
            with pytest.raises(AssertionError):
                check_ids(swapped, r, k, O.MODE_SIGMOID_BIAS_RENORM, hh, w, None, b_sel)
        check_ids(r.ids, r, k, O.MODE_SIGMOID_BIAS_RENORM, hh, w, None, b_sel)


def test_gates_of_matches_route():
    """The gate step for a fixed selection gives the oracle's own gates."""
    for mode in (O.MODE_SOFTMAX_RENORM, O.MODE_SOFTMAX_FULL, O.MODE_SIGMOID_BIAS_RENORM):
        inp, _ = _inputs(11, 20, 32, 7, 3, 16, 0, mode)
        r = O.route(inp["h"], inp["w_router"], 3, mode, inp["b_router"], inp["b_select"])
        assert np.allclose(EB.gates_of(r.z, r.ids, mode), r.gates, rtol=1e-14, atol=0)


def test_logit_jacobian_closed_form():
    """The central-difference Jacobian of dL/dz in logit_propagation against
    a closed form: with one expert, gate_backward is zero (the probability
    is 1 whatever the logit) and the z-loss term is d_zloss (2/T) z, so
    d dz / dz = 2 d_zloss / T and the propagated variance is that squared
    times the logit's."""
    T, d = 12, 16
    inp, _ = _inputs(12, T, d, 1, 1, 16, 0, O.MODE_SOFTMAX_FULL)
    r = O.route(inp["h"], inp["w_router"], 1, O.MODE_SOFTMAX_FULL, inp["b_router"])
    m_z, v_z = EB.logit_scales(inp["h"], inp["w_router"], inp["b_router"])
    dg = np.random.default_rng(3).standard_normal((T, 1))
    m_g, v_g, m_dz, v_dz, v_dhr = EB.logit_propagation(
        r, dg, np.array([T]), 1, O.MODE_SOFTMAX_FULL, 0.01, 0.5, 0.7, inp["w_router"], m_z, v_z)
    c = 2.0 * 0.7 / T
    assert not np.any(m_g) and not np.any(v_g)
    assert np.allclose(m_dz, c * m_z, rtol=1e-6) and np.allclose(v_dz, c * c * v_z, rtol=1e-6)
    wr = np.asarray(inp["w_router"], np.float64)
    assert np.allclose(v_dhr, c * c * v_z * wr ** 2, rtol=1e-6)


def _emulated_f32_logits_backward(inp, dy, k, mode, cf, d_laux, d_zloss):
    """The oracle's backward with the router logits evaluated in fp32 (an
    fp32 product of h and W_r, the bias added in fp32) and the gates rounded
    to fp32; every other step exact. It isolates the logits' rounding, which
    the other emulation leaves out."""
    h = np.asarray(inp["h"], np.float64)
    wr = np.asarray(inp["w_router"], np.float64)
    T, d = h.shape
    N = wr.shape[0]
    z32 = np.asarray(inp["h"], np.float32) @ np.asarray(inp["w_router"], np.float32).T
    if inp["b_router"] is not None:
        z32 = z32 + np.asarray(inp["b_router"], np.float32)[None, :]
    r = O.route(h, wr, k, mode, inp["b_router"], inp["b_select"])
    z = z32.astype(np.float64)
    g = EB.gates_of(z, r.ids, mode).astype(np.float32).astype(np.float64)
    r = O.Routing(r.ids, g, z, r.sel, r.gap, r.stat_prob)
    disp = O.dispatch(r.ids, N, O.expert_capacity(cf, T, k, N) if cf else None)
    dh, dg = np.zeros((T, d)), np.zeros((T, k))
    dwg, dwu, dwd = [], [], []
    for e in range(N):
        wg, wu, wd = (np.asarray(inp[key][e], np.float64) for key in ("w_gate", "w_up", "w_down"))
        flats = disp.perm_src[disp.offsets[e]:disp.offsets[e + 1]]
        t, j = flats // k, flats % k
        dg[t, j] = np.sum(dy[t] * O.expert_ffn(h[t], wg, wu, wd), axis=-1)
        dx, a, b, c = O.expert_ffn_backward(h[t], wg, wu, wd, g[t, j][:, None] * dy[t])
        np.add.at(dh, t, dx)
        dwg.append(a)
        dwu.append(b)
        dwd.append(c)
    dz = O.gate_backward(r, dg, mode) + O.stats_backward(r, disp.counts, k, mode, 0.01, d_laux,
                                                         d_zloss)
    return O.LayerGrads(dh + dz @ wr, dz.T @ h, dz.sum(axis=0), np.stack(dwg), np.stack(dwu),
                        np.stack(dwd), None, dg, dz)


F32_LOGIT_CASES = [
    # seed, T, d, N, k, d_ff, mode, capacity, d_laux, d_zloss
    # one expert, half the tokens dropped: a dropped token's dh is the z-loss
    # term alone, proportional to its logit, some of which nearly cancel
    (33, 300, 32, 1, 1, 40, O.MODE_SOFTMAX_FULL, 0.5, 0.3, 0.3),
    (22, 120, 48, 6, 2, 32, O.MODE_SOFTMAX_RENORM, 0.75, 1.0, 1.0),
    (23, 90, 32, 9, 3, 24, O.MODE_SIGMOID_BIAS_RENORM, None, 0.3, 1.0),
]


@pytest.mark.parametrize("case", F32_LOGIT_CASES, ids=[str(c[0]) for c in F32_LOGIT_CASES])
def test_fp32_logit_error_inside_noise(case, monkeypatch):
    """fp32 router logits stay inside the noise gate of the fp32 path; the
    model without the logits' propagation fails the one-expert case."""
    seed, T, d, N, k, dff, mode, cf, d_laux, d_zloss = case
    inp = W.random_small(T, d, N, k, dff, 0, W.DTYPE_F32, mode, seed=seed, router_bias=True)
    dy = np.random.default_rng(seed).standard_normal((T, d)).astype(np.float32).astype(np.float64)
    args = _args(inp, dy, k, mode)
    ids = ref_ids(inp, k, mode)
    ref = O.layer_backward(*args, None, cf, d_laux, d_zloss, ids=ids)
    emu = _emulated_f32_logits_backward(inp, dy, k, mode, cf, d_laux, d_zloss)
    sc, nz = EB.grad_scales(*args, cf, d_laux, d_zloss, ids=ids, u_store=EB.U_F32, ref=ref)
    R, S, Z, E = _fields(ref), _fields(sc), _fields(nz), _fields(emu)
    for key in R:
        check_grad(E[key], R[key], S[key], Z[key], GRAD_TOL[W.DTYPE_F32], key)
    if N == 1:
        def no_logits(r, dg, counts, k_, mode_, alpha, la, lz, wr, m_z, v_z, step=1e-6):
            T_, N_ = r.z.shape
            z_ = lambda *s: np.zeros(s)
            return (z_(T_, r.ids.shape[1]), z_(T_, r.ids.shape[1]), z_(T_, N_), z_(T_, N_),
                    z_(T_, np.asarray(wr).shape[1]))
        monkeypatch.setattr(EB, "logit_propagation", no_logits)
        _, nz0 = EB.grad_scales(*args, cf, d_laux, d_zloss, ids=ids, u_store=EB.U_F32, ref=ref)
        with pytest.raises(AssertionError):
            check_grad_noise(emu.dh, ref.dh, nz0.dh, "dh")
