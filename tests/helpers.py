"""Shared helpers of the GPU parity tests: moving seeded host inputs to the
device in the library's dtypes, reading results back, and the comparison
rules (near-tie exclusion, per-row relative error)."""
import numpy as np

import error_bounds as EB
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


def check_ids(gpu_ids, oracle_routing, k, mode, h, w_router, b_router=None, b_select=None,
              grouped=False):
    """The selected expert set must match exactly for every token whose k-th
    and (k+1)-th selection scores (and, with a group limit, its last kept
    and first dropped group scores) are at least NEAR_TIE apart. Its slots
    must come in descending order of the score the GPU compares (the logit
    in the softmax modes, sigma(z) + b_select in mode C), two slots
    appearing in either order only where their exact scores differ by less
    than the sum of the bounds on their fp32 errors (error_bounds.
    comparison_scores). For near-tie tokens the GPU's selection must still
    be k distinct experts, and without a group limit a valid top-k within
    NEAR_TIE. Returns the near-tie mask; prints how many slot pairs needed
    the fp32 allowance."""
    near = O.near_tie_tokens(oracle_routing.gap, NEAR_TIE)
    ok = ~near
    same = np.all(np.sort(gpu_ids, axis=1) == np.sort(oracle_routing.ids, axis=1), axis=1)
    assert np.all(same[ok]), np.nonzero(~same & ok)[0][:10]
    score, err = EB.comparison_scores(oracle_routing, mode, h, w_router, b_router, b_select)
    gi = gpu_ids.astype(np.int64)
    sc = np.take_along_axis(score, gi, axis=1)
    er = np.take_along_axis(err, gi, axis=1)
    rise = sc[:, 1:] - sc[:, :-1]                # > 0: a later slot scores higher
    allow = er[:, 1:] + er[:, :-1]
    bad = ((rise > allow).any(axis=1)) & ok
    assert not np.any(bad), (np.nonzero(bad)[0][:10], rise[bad][:3], allow[bad][:3])
    swaps = int(((rise > 0) & ok[:, None]).sum())
    if swaps:
        print(f"  slot order: {swaps} adjacent pair(s) within the fp32 score bound, "
              f"largest rise {rise[ok].max():.2e}", flush=True)
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


# Backward tolerance against the per-element magnitude scale M of
# error_bounds.grad_scales (|error| <= c u M for c roundings of relative size
# u on the longest path). bf16: at most three bf16 roundings lie on any path
# (an intermediate stored as bf16, an operand rounded before a GEMM, the
# output), plus fp32 accumulation: 4 u_bf16 = 1.5625e-2. fp32: the fp32
# bar of the forward, 1e-4, above n u_f32 for every sum of n <= 1,600 terms
# the fp32 tests form.
GRAD_TOL = {W.DTYPE_F32: 1e-4, W.DTYPE_BF16: 4 * EB.U_BF16}


def check_grad_elems(y, y_ref, scale, tol, what):
    """Element by element: |y - y_ref| <= tol * scale, where scale is the
    magnitude of the terms the element sums (error_bounds.grad_scales).
    Where the scale is zero every term is zero and the value must be exactly
    y_ref. Returns the largest |y - y_ref| / scale."""
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    scale = np.broadcast_to(np.asarray(scale, np.float64), y_ref.shape)
    assert y.shape == y_ref.shape, (what, y.shape, y_ref.shape)
    if y_ref.size == 0:
        return 0.0
    diff = np.abs(y - y_ref)
    zero = scale == 0
    assert not np.any(diff[zero]), f"{what}: non-zero where every term is zero"
    ratio = diff / np.where(zero, 1.0, scale)
    worst = float(ratio.max())
    assert worst <= tol, (f"{what}: max |error| / term scale {worst:.3e} > {tol:.3e} at "
                          f"{np.unravel_index(int(ratio.argmax()), ratio.shape)}")
    return worst


# Noise gate: per element |error| <= NOISE_MAX sigma and, over a tensor, the
# root-mean-square of error / sigma <= NOISE_RMS, sigma the propagated noise
# standard deviation of error_bounds.grad_scales. Independent uniform
# roundings give a root-mean-square near 1 or below (the model takes every
# rounding at its largest variance); twelve standard deviations of a sum of
# many such errors never occur, and a single rounding reaches sqrt(3).
NOISE_MAX, NOISE_RMS = 12.0, 3.0


def check_grad_noise(y, y_ref, sigma, what, kmax=NOISE_MAX, krms=NOISE_RMS):
    """|y - y_ref| against the noise scale sigma, element by element (at most
    kmax sigma) and over the tensor (root-mean-square at most krms). Where
    sigma is zero the value must be exact. Returns (max, rms) of
    |y - y_ref| / sigma."""
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    sigma = np.broadcast_to(np.asarray(sigma, np.float64), y_ref.shape)
    if y_ref.size == 0:
        return 0.0, 0.0
    diff = np.abs(y - y_ref)
    zero = sigma == 0
    assert not np.any(diff[zero]), f"{what}: non-zero error where no rounding reaches"
    ratio = diff / np.where(zero, 1.0, sigma)
    worst, rms = float(ratio.max()), float(np.sqrt(np.mean(ratio ** 2)))
    assert worst <= kmax, (f"{what}: max |error| / noise {worst:.2f} > {kmax} at "
                           f"{np.unravel_index(int(ratio.argmax()), ratio.shape)}")
    assert rms <= krms, f"{what}: rms |error| / noise {rms:.2f} > {krms}"
    return worst, rms


def check_grad(y, y_ref, scale, sigma, tol, what):
    """Both gates on one gradient: the exact bound tol * scale
    (check_grad_elems) and the noise gate (check_grad_noise). Returns
    (largest |error| / scale, largest |error| / sigma, rms |error| / sigma)."""
    m = check_grad_elems(y, y_ref, scale, tol, what)
    n_max, n_rms = check_grad_noise(y, y_ref, sigma, what)
    return m, n_max, n_rms


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
