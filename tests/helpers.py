"""Shared helpers of the GPU parity tests: moving seeded host inputs to the
device in the library's dtypes, reading results back, and the comparison
rules (near-tie exclusion, per-row relative error)."""
import numpy as np

import workloads as W
from oracle import moe_oracle as O

TOL = {W.DTYPE_F32: 1e-4, W.DTYPE_BF16: 2e-2}
NEAR_TIE = 1e-4


def torch():
    import torch as _t
    return _t


def dev(a, dtype, device="cuda"):
    """numpy array (fp32 values; bf16-representable when dtype is bf16) ->
    device tensor of that dtype, bit-exact."""
    if a is None:
        return None
    t = torch()
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == W.DTYPE_BF16:
        bits = W.bf16_bits(a).view(np.int16)
        return t.from_numpy(bits.copy()).to(device).view(t.bfloat16)
    return t.from_numpy(a.copy()).to(device)


def dev_f32(a, device="cuda"):
    return None if a is None else torch().from_numpy(np.ascontiguousarray(a, np.float32)).to(device)


def host(t):
    """device tensor -> float64 (or int64) numpy array."""
    tt = torch()
    t = t.detach().cpu()
    if t.dtype in (tt.int32, tt.int64):
        return t.numpy().astype(np.int64)
    # buffers with rows a call does not write (dropped slots) may hold
    # signalling-NaN bit patterns; their cast is not an error
    with np.errstate(invalid="ignore"):
        return t.float().numpy().astype(np.float64)


def tdtype(dtype):
    t = torch()
    return t.bfloat16 if dtype == W.DTYPE_BF16 else t.float32


def oracle_weights(inp):
    return O.weights_getter(inp["w_gate"], inp["w_up"], inp["w_down"])


def oracle_shared(inp):
    if inp.get("sh_gate") is None:
        return None
    return (inp["sh_gate"], inp["sh_up"], inp["sh_down"])


def check_ids(gpu_ids, oracle_routing, k, grouped=False):
    """The selected expert set must match exactly for every token whose k-th
    and (k+1)-th selection scores (and, with a group limit, its last kept
    and first dropped group scores) are at least NEAR_TIE apart, and its slot
    order must be by descending oracle score, two slots appearing in either
    order only when their scores are closer than NEAR_TIE (fp32 scores can
    tie or flip where float64 ones differ by 1e-8). For near-tie tokens the
    GPU's selection must still be k distinct experts, and without a group
    limit a valid top-k within that margin. Returns the near-tie mask."""
    near = O.near_tie_tokens(oracle_routing.gap, NEAR_TIE)
    ok = ~near
    same = np.all(np.sort(gpu_ids, axis=1) == np.sort(oracle_routing.ids, axis=1), axis=1)
    assert np.all(same[ok]), np.nonzero(~same & ok)[0][:10]
    sel = np.take_along_axis(oracle_routing.sel, gpu_ids.astype(np.int64), axis=1)
    rising = (np.diff(sel, axis=1) > NEAR_TIE).any(axis=1)
    assert not np.any(rising & ok), np.nonzero(rising & ok)[0][:10]
    for t in np.nonzero(near)[0]:
        assert len(set(gpu_ids[t].tolist())) == k
        if not grouped:
            sel = oracle_routing.sel[t]
            kth = np.sort(sel)[::-1][k - 1]
            assert np.all(sel[gpu_ids[t]] >= kth - NEAR_TIE)
    return near


def check_close_rows(y, y_ref, tol, mask=None, what="y"):
    err = O.row_rel_err(y, y_ref)
    if mask is not None:
        err = err[mask]
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, f"{what}: max per-row relative error {worst:.3e} > {tol:.1e}"
    return worst


def check_grad_rows(y, y_ref, tol, what, floor=1e-2):
    """Per-row relative error of a gradient, each row's scale being the larger
    of its own max |y_ref| and floor times the tensor's: a row whose exact
    value is a sum that cancels far below the gradient's scale (a dot
    product of nearly opposite terms, or a token whose routed slots were all
    dropped) carries the rounding of its terms, not of its result, so it is
    compared at the tensor's scale."""
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    if y_ref.size == 0:
        return 0.0
    num = np.abs(y - y_ref).max(axis=-1)
    den = np.maximum(np.abs(y_ref).max(axis=-1), floor * np.abs(y_ref).max())
    err = num / np.where(den == 0, 1.0, den)
    worst = float(err.max())
    assert worst <= tol, f"{what}: max per-row error / row scale {worst:.3e} > {tol:.1e}"
    return worst


def align_slots(ids, ids_ref, vals_ref):
    """vals_ref (per slot of ids_ref) reordered to the slot order of ids, for
    tokens whose two id rows hold the same set."""
    oi = np.argsort(ids_ref, axis=1, kind="stable")
    gi = np.argsort(ids, axis=1, kind="stable")
    out = np.empty_like(np.asarray(vals_ref, np.float64))
    np.put_along_axis(out, gi, np.take_along_axis(np.asarray(vals_ref, np.float64), oi, axis=1),
                      axis=1)
    return out


def check_gates(g, g_ref, tol, mask, ids=None, ids_ref=None):
    """Per-slot relative error of the gates; with ids, g_ref is first taken
    in the GPU's slot order (the same experts, see check_ids)."""
    if ids is not None:
        g_ref = align_slots(ids, ids_ref, g_ref)
    err = np.abs(g - g_ref) / np.maximum(np.abs(g_ref), 1e-30)
    worst = float(err[mask].max()) if mask.any() else 0.0
    assert worst <= tol, f"gates: max relative error {worst:.3e} > {tol:.1e}"
    return worst
