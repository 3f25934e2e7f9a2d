"""moe_layer_fused_noalloc (the allocation-free fused forward, on the
library's static scratch) against moe_layer_fused with a caller workspace:
the same bits for every output, on two calls in a row, the second with a
smaller input, and the oracle's tolerance for y."""
import numpy as np
import pytest

import workloads as W
from oracle import moe_oracle as O
from helpers import TOL, check_close_rows, dev, dev_f32, host, oracle_shared, oracle_weights, torch

pytestmark = pytest.mark.gpu

import sparse_mixture_experts_35_amd as M  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()


def _run(s, inp, noalloc):
    t = torch()
    dt = s.dtype
    T, d, N, k = s.T, s.d, s.N, s.k
    td = t.bfloat16 if dt == W.DTYPE_BF16 else t.float32
    E = lambda n, ty: t.full(n if isinstance(n, tuple) else (n,), 7, dtype=ty,
                             device="cuda")                   # poisoned outputs
    out = dict(y=E((T, d), td), ids=E(T * k, t.int32), gates=E(T * k, t.float32),
               counts=E(N, t.int32), f=E(N, t.float32), p=E(N, t.float32), l_aux=E(1, t.float32),
               z_loss=E(1, t.float32), entropy=E(1, t.float32), cap=E(2, t.float32))
    args = (s, dev(inp["h"], dt), dev(inp["w_router"], dt), dev_f32(inp["b_router"]),
            dev_f32(inp["b_select"]), dev(inp["w_gate"], dt), dev(inp["w_up"], dt),
            dev(inp["w_down"], dt), dev(inp["sh_gate"], dt), dev(inp["sh_up"], dt),
            dev(inp["sh_down"], dt), out["y"], out["ids"], out["gates"], out["counts"], out["f"],
            out["p"], out["l_aux"])
    extra = dict(z_loss=out["z_loss"], entropy=out["entropy"], cap_stats=out["cap"])
    if noalloc:
        M.layer_fused_noalloc(*args, **extra)
    else:
        n = M.workspace_bytes(s)
        ws = t.empty(n, dtype=t.uint8, device="cuda")
        M.layer_fused(*args, ws=ws, ws_bytes=n, **extra)
    t.cuda.synchronize()
    return out


# (T, d, N, k, d_ff, d_ff_shared, dtype, mode, capacity): the first takes the
# tiled GEMMs (more than 64 rows per expert: split-K partials in the
# scratch), the second is a smaller decode batch (weight-streaming kernels,
# fused combine) run right after it on the same scratch, the third fp32
CALLS = [
    (300, 256, 8, 2, 128, 128, W.DTYPE_BF16, 0, 0.0),
    (16, 512, 16, 4, 256, 128, W.DTYPE_BF16, 2, 0.0),
    (40, 64, 6, 2, 64, 0, W.DTYPE_F32, 1, 1.0),
]


def test_noalloc_matches_fused_twice_then_smaller():
    t = torch()
    for i, (T, d, N, k, dff, dfs, dt, mode, cf) in enumerate(CALLS):
        s = M.Shape(T, d, N, k, dff, dfs, dt, mode, 0.01, capacity_factor=cf)
        inp = W.random_small(T, d, N, k, dff, dfs, dt, mode, seed=40 + i, router_bias=True)
        print(f"call {i}: T={T} d={d} N={N} k={k} d_ff={dff} shared={dfs} dtype={dt} "
              f"mode={mode} cf={cf}", flush=True)
        a = _run(s, inp, noalloc=True)
        b = _run(s, inp, noalloc=False)
        for key in a:
            assert t.equal(a[key], b[key]), f"call {i}: {key} differs from moe_layer_fused"
        ref = O.layer(inp["h"], inp["w_router"], k, mode, oracle_weights(inp), inp["b_router"],
                      inp["b_select"], oracle_shared(inp), 0.01, None, cf or None)
        ok = ~O.near_tie_tokens(ref.routing.gap)
        g_ids = host(a["ids"]).reshape(T, k)
        assert np.array_equal(np.sort(g_ids[ok], axis=1), np.sort(ref.routing.ids[ok], axis=1))
        worst = check_close_rows(host(a["y"]), ref.y, TOL[dt], ok, what=f"call {i}: y")
        print(f"call {i}: same bits as moe_layer_fused; y max row rel err {worst:.2e}", flush=True)


def test_noalloc_second_call_smaller_same_shape_family():
    """Two calls in a row on one layer's weights, the second on fewer tokens:
    the scratch keeps the first call's contents, which must not leak into the
    second (counters are cleared by the call that uses them)."""
    t = torch()
    d, N, k, dff = 256, 8, 2, 256
    big = W.random_small(200, d, N, k, dff, 0, W.DTYPE_BF16, 0, seed=3)
    small = {key: (v[:24] if key == "h" else v) for key, v in big.items()}
    for T, inp in ((200, big), (24, small)):
        s = M.Shape(T, d, N, k, dff, 0, W.DTYPE_BF16, 0, 0.01)
        a = _run(s, inp, noalloc=True)
        b = _run(s, inp, noalloc=False)
        for key in a:
            assert t.equal(a[key], b[key]), f"T={T}: {key} differs from moe_layer_fused"
        print(f"T={T}: same bits as moe_layer_fused", flush=True)


def test_noalloc_mixtral_decode_full_size():
    """The decode batch these callers run: the Mixtral-shaped layer at
    T = 16 (inputs drawn on the device as the benchmark draws them), the
    allocation-free call against moe_layer_fused, bit for bit, twice."""
    t = torch()
    w = W.MIXTRAL_DECODE
    inp = W.device_inputs(w)
    s = M.Shape(w.T, w.d, w.N, w.k, w.d_ff, w.d_ff_shared, w.dtype, w.mode, w.aux_alpha)
    outs = []
    for noalloc in (True, False, True):
        y = t.empty((w.T, w.d), dtype=t.bfloat16, device="cuda")
        ids = t.empty(w.T * w.k, dtype=t.int32, device="cuda")
        args = (s, inp["h"], inp["w_router"], inp["b_router"], inp["b_select"], inp["w_gate"],
                inp["w_up"], inp["w_down"], inp["sh_gate"], inp["sh_up"], inp["sh_down"], y, ids)
        if noalloc:
            M.layer_fused_noalloc(*args)
        else:
            n = M.workspace_bytes(s)
            ws = t.empty(n, dtype=t.uint8, device="cuda")
            M.layer_fused(*args, ws=ws, ws_bytes=n)
        t.cuda.synchronize()
        outs.append((y, ids))
    for y, ids in outs[1:]:
        assert t.equal(y, outs[0][0]) and t.equal(ids, outs[0][1])
    print(f"[{w.name}] allocation-free call: same bits as moe_layer_fused", flush=True)
