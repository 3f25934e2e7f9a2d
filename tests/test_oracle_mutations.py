"""Plant a plausible mistake in the oracle (on the CPU) and check that at
least one pin fails for it, so the pins constrain every step."""
import math

import numpy as np
import scipy.special
import pytest

import pins
from oracle import moe_oracle as O

_orig = {n: getattr(O, n) for n in ("router_logits", "softmax", "sigmoid", "topk", "group_limit",
                                     "dispatch", "expert_capacity", "silu", "expert_ffn", "combine",
                                     "load_stats", "route", "router_z_loss", "routing_entropy",
                                     "silu_grad", "expert_ffn_backward", "gate_backward",
                                     "stats_backward", "layer_backward", "row_rel_err",
                                     "near_tie_tokens")}


def _route_no_renorm(h, w, k, mode, b_router=None, b_select=None):
    r = _orig["route"](h, w, k, mode, b_router, b_select)
    if mode == O.MODE_SOFTMAX_RENORM:
        r.gates = np.take_along_axis(r.stat_prob, r.ids, axis=-1)
    return r


def _route_biased_gates(h, w, k, mode, b_router=None, b_select=None):
    r = _orig["route"](h, w, k, mode, b_router, b_select)
    if mode == O.MODE_SIGMOID_BIAS_RENORM:
        s = np.take_along_axis(r.sel, r.ids, axis=-1)
        r.gates = s / s.sum(axis=-1, keepdims=True)
    return r


def _logits_reversed(h, w, b=None):
    return _orig["router_logits"](h, np.asarray(w, float)[::-1], b)


def _topk_ascending(sel, k):
    ids, gap = _orig["topk"](-np.asarray(sel, float), k)
    return ids, gap


def _topk_high_index_ties(sel, k):
    sel = np.asarray(sel, float)
    ids, gap = _orig["topk"](sel[:, ::-1], k)
    return sel.shape[1] - 1 - ids, gap


def _dispatch_reversed(ids, N):
    d = _orig["dispatch"](ids, N)
    for e in range(N):
        lo, hi = d.offsets[e], d.offsets[e + 1]
        d.perm_src[lo:hi] = d.perm_src[lo:hi][::-1].copy()
    d.row_of[d.perm_src] = np.arange(d.perm_src.size)
    return d


def _combine_overwrite(out_rows, row_of, gates, has_shared=False):
    gates = np.asarray(gates, float)
    T, k = gates.shape
    y = np.zeros((T, out_rows.shape[1]))
    if has_shared:
        y += out_rows[T * k:T * k + T]
    rows = np.asarray(row_of).reshape(T, k)
    for j in range(k):
        y = gates[:, j:j + 1] * np.asarray(out_rows)[rows[:, j]]
    return y


def _combine_no_shared(out_rows, row_of, gates, has_shared=False):
    return _orig["combine"](out_rows, row_of, gates, False)


def _combine_slot0_gate(out_rows, row_of, gates, has_shared=False):
    g = np.repeat(np.asarray(gates, float)[:, :1], np.asarray(gates).shape[1], axis=1)
    return _orig["combine"](out_rows, row_of, g, has_shared)


def _group_mask_zero(sel, n_groups, topk_groups, topm):
    masked, gap = _orig["group_limit"](sel, n_groups, topk_groups, topm)
    return np.where(np.isinf(masked), 0.0, masked), gap


def _group_score_max(sel, n_groups, topk_groups, topm):
    return _orig["group_limit"](sel, n_groups, topk_groups, 1)


def _group_keep_worst(sel, n_groups, topk_groups, topm):
    return _orig["group_limit"](-np.asarray(sel, float), n_groups, topk_groups, topm)[0] * -1.0, \
        np.full(np.asarray(sel).shape[0], np.inf)


def _dispatch_drop_earliest(ids, N, capacity=None):
    d = _orig["dispatch"](ids, N, None)
    if capacity is None:
        return d
    flat = np.asarray(ids).reshape(-1)
    buckets = [np.nonzero(flat == e)[0] for e in range(N)]
    buckets = [b[max(0, len(b) - capacity):] for b in buckets]
    kept = np.array([len(b) for b in buckets])
    offsets = np.concatenate([[0], np.cumsum(kept)])
    perm = np.concatenate(buckets).astype(np.int64)
    row_of = np.full(flat.size, -1)
    row_of[perm] = np.arange(perm.size)
    return O.Dispatch(d.counts, offsets, perm, row_of, kept)


def _combine_negative_row(out_rows, row_of, gates, has_shared=False):
    gates = np.asarray(gates, float)
    T, k = gates.shape
    out_rows = np.asarray(out_rows, float)
    y = np.zeros((T, out_rows.shape[1]))
    if has_shared:
        y += out_rows[T * k:T * k + T]
    rows = np.asarray(row_of).reshape(T, k)
    for j in range(k):
        y += gates[:, j:j + 1] * out_rows[rows[:, j]]
    return y


def _ffn_bwd_gate_up_swapped(x, wg, wu, wd, dout):
    dx, dwg, dwu, dwd = _orig["expert_ffn_backward"](x, wg, wu, wd, dout)
    return dx, dwu, dwg, dwd


def _ffn_bwd_no_dx_up(x, wg, wu, wd, dout):
    x, dout = np.asarray(x, float), np.asarray(dout, float)
    gp = x @ np.asarray(wg, float).T
    up = x @ np.asarray(wu, float).T
    dact = dout @ np.asarray(wd, float)
    du = dact * O.silu(gp)
    dgp = dact * up * O.silu_grad(gp)
    dx, dwg, dwu, dwd = _orig["expert_ffn_backward"](x, wg, wu, wd, dout)
    return dgp @ np.asarray(wg, float), dwg, dwu, dwd


def _gate_bwd_mode_b_selected_only(routing, dg, mode):
    dz = _orig["gate_backward"](routing, dg, mode)
    if mode == O.MODE_SOFTMAX_FULL:
        mask = np.zeros_like(dz)
        np.put_along_axis(mask, routing.ids, 1.0, axis=-1)
        dz = dz * mask
    return dz


def _gate_bwd_mode_a_no_inner(routing, dg, mode):
    if mode != O.MODE_SOFTMAX_RENORM:
        return _orig["gate_backward"](routing, dg, mode)
    dz = np.zeros(routing.z.shape)
    np.put_along_axis(dz, routing.ids, routing.gates * np.asarray(dg, float), axis=-1)
    return dz


def _gate_bwd_mode_c_biased(routing, dg, mode):
    if mode != O.MODE_SIGMOID_BIAS_RENORM:
        return _orig["gate_backward"](routing, dg, mode)
    s = np.take_along_axis(routing.sel, routing.ids, axis=-1)     # biased scores
    g = routing.gates
    ds = (dg - (g * dg).sum(axis=-1, keepdims=True)) / s.sum(axis=-1, keepdims=True)
    dz = np.zeros(routing.z.shape)
    np.put_along_axis(dz, routing.ids, ds * s * (1 - s), axis=-1)
    return dz


def _layer_bwd_ignores_capacity(*a, **kw):
    if len(a) > 11:
        a = a[:11] + (None,) + a[12:]
    else:
        kw["capacity_factor"] = None
    return _orig["layer_backward"](*a, **kw)


def _layer_bwd_no_shared(*a, **kw):
    g = _orig["layer_backward"](*a, **kw)
    if g.dsh is not None:
        g.dsh = tuple(np.zeros_like(v) for v in g.dsh)
    return g


MUTATIONS = {
    "logits_drop_bias": ("router_logits", lambda h, w, b=None: _orig["router_logits"](h, w, None)),
    "logits_expert_index_reversed": ("router_logits", _logits_reversed),
    "softmax_wrong_axis": ("softmax", lambda z: np.exp(np.asarray(z, float)) / np.exp(np.asarray(z, float)).sum(axis=0, keepdims=True)),
    "sigmoid_sign": ("sigmoid", lambda z: 1.0 / (1.0 + np.exp(np.asarray(z, float)))),
    "topk_ascending": ("topk", _topk_ascending),
    "topk_ties_high_index": ("topk", _topk_high_index_ties),
    "mode_a_no_renorm": ("route", _route_no_renorm),
    "mode_c_biased_gates": ("route", _route_biased_gates),
    "dispatch_unstable": ("dispatch", _dispatch_reversed),
    "silu_is_relu": ("silu", lambda x: np.maximum(np.asarray(x, float), 0.0)),
    "silu_is_sigmoid": ("silu", lambda x: 1.0 / (1.0 + np.exp(-np.asarray(x, float)))),
    "ffn_gate_up_swapped": ("expert_ffn", lambda x, g, u, d: _orig["expert_ffn"](x, u, g, d)),
    "ffn_no_up": ("expert_ffn", lambda x, g, u, d: O.silu(np.asarray(x, float) @ np.asarray(g, float).T) @ np.asarray(d, float).T),
    "combine_overwrite": ("combine", _combine_overwrite),
    "combine_drops_shared": ("combine", _combine_no_shared),
    "combine_slot0_gate": ("combine", _combine_slot0_gate),
    "group_mask_zero": ("group_limit", _group_mask_zero),
    "group_score_max_only": ("group_limit", _group_score_max),
    "group_keep_worst": ("group_limit", _group_keep_worst),
    "z_loss_not_squared": ("router_z_loss", lambda z: float(np.mean(scipy.special.logsumexp(np.asarray(z, float), axis=-1)))),
    "z_loss_sum_not_mean": ("router_z_loss", lambda z: _orig["router_z_loss"](z) * np.asarray(z).shape[0]),
    "entropy_log2": ("routing_entropy", lambda q: _orig["routing_entropy"](q) / math.log(2)),
    "capacity_drops_earliest": ("dispatch", _dispatch_drop_earliest),
    "capacity_floor": ("expert_capacity", lambda cf, T, k, N: int(math.floor(float(np.float32(cf)) * (T * k) / N))),
    "combine_dropped_slot_wraps": ("combine", _combine_negative_row),
    "silu_grad_sigmoid_only": ("silu_grad", lambda x: O.sigmoid(x)),
    "ffn_bwd_gate_up_swapped": ("expert_ffn_backward", _ffn_bwd_gate_up_swapped),
    "ffn_bwd_dx_misses_up": ("expert_ffn_backward", _ffn_bwd_no_dx_up),
    "gate_bwd_mode_b_selected_only": ("gate_backward", _gate_bwd_mode_b_selected_only),
    "gate_bwd_mode_a_no_inner": ("gate_backward", _gate_bwd_mode_a_no_inner),
    "gate_bwd_mode_c_biased": ("gate_backward", _gate_bwd_mode_c_biased),
    "stats_bwd_zloss_no_factor_2": ("stats_backward",
                                    lambda r, c, k, m, a, dl=0.0, dz=0.0:
                                    _orig["stats_backward"](r, c, k, m, a, dl, dz / 2)),
    "stats_bwd_laux_sign": ("stats_backward",
                            lambda r, c, k, m, a, dl=0.0, dz=0.0:
                            _orig["stats_backward"](r, c, k, m, a, -dl, dz)),
    "layer_bwd_ignores_capacity": ("layer_backward", _layer_bwd_ignores_capacity),
    "layer_bwd_no_shared": ("layer_backward", _layer_bwd_no_shared),
    "row_rel_err_zero": ("row_rel_err", lambda y, r: np.zeros(np.asarray(y).shape[0])),
    "row_rel_err_tensor_scale": ("row_rel_err", lambda y, r: np.abs(np.asarray(y, float) - np.asarray(r, float)).max(axis=-1) / max(np.abs(np.asarray(r, float)).max(initial=0.0), 1e-300)),
    "row_rel_err_elementwise": ("row_rel_err", lambda y, r: (np.abs(np.asarray(y, float) - np.asarray(r, float)) / np.maximum(np.abs(np.asarray(r, float)), 1e-300)).max(axis=-1, initial=0.0)),
    "row_rel_err_mean": ("row_rel_err", lambda y, r: np.abs(np.asarray(y, float) - np.asarray(r, float)).mean(axis=-1) / np.maximum(np.abs(np.asarray(r, float)).max(axis=-1, initial=0.0), 1e-300)),
    "near_tie_inclusive": ("near_tie_tokens", lambda g, th=1e-4: np.asarray(g) <= th),
    "near_tie_never": ("near_tie_tokens", lambda g, th=1e-4: np.zeros(np.shape(g), bool)),
    "near_tie_fixed_threshold": ("near_tie_tokens", lambda g, th=1e-4: np.asarray(g) < 1e-4),
    "stats_f_over_T": ("load_stats", lambda c, sp, k, a: _orig["load_stats"](c, sp, 1, a)),
    "stats_no_N_factor": ("load_stats", lambda c, sp, k, a: (lambda f, p, l: (f, p, l / np.asarray(sp).shape[1]))(*_orig["load_stats"](c, sp, k, a))),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_pin_catches(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin()
        except Exception:            # AssertionError, or a shape error
            failed.append(pin.__name__)
    assert failed, f"no pin fails with mutation {name}"
