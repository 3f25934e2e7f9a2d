"""GPU parity: each C-ABI call, then the fused layer, against the float64
oracle on the same seeded inputs, at sizes the oracle finishes in seconds
that still span several tiles and ragged tails.

Rules: expert ids and the dispatch permutation bit-exact (tokens with a
k-th/(k+1)-th selection-score gap below 1e-4 excluded from the id check and
verified to be a valid top-k instead); outputs within max per-row relative
error 1e-4 (fp32) / 2e-2 (bf16); gates within 1e-4 (they are fp32 on both
paths)."""
import numpy as np
import pytest

import workloads as W
from oracle import moe_oracle as O
from helpers import (TOL, check_close_rows, check_gates, check_ids, dev, dev_f32, host,
                     oracle_shared, oracle_weights, tdtype, torch)

pytestmark = pytest.mark.gpu

import sparse_mixture_experts_35_amd as M  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()


def i32(n):
    t = torch()
    return t.empty(n, dtype=t.int32, device="cuda")


def f32(n):
    t = torch()
    return t.empty(n, dtype=t.float32, device="cuda")


def shape_of(T, d, N, k, d_ff, d_ff_shared=0, dtype=W.DTYPE_BF16, mode=0, alpha=0.01,
             groups=None, cf=0.0):
    g = groups or (0, 0, 0)
    return M.Shape(T, d, N, k, d_ff, d_ff_shared, dtype, mode, alpha, *g, cf)


def capacity_of(s):
    """The oracle's capacity C for the shape (None when dropless)."""
    return O.expert_capacity(s.capacity_factor, s.T, s.k, s.N) if s.capacity_factor else None


def groups_of(s):
    return (s.n_groups, s.topk_groups, s.group_topm) if s.n_groups else None


def workspace(s):
    t = torch()
    n = M.workspace_bytes(s)
    return t.empty(max(n, 1), dtype=t.uint8, device="cuda"), n


def run_steps(s, inp):
    """route -> dispatch -> expert_ffn -> combine through the separate
    C-ABI calls; returns every intermediate on the host."""
    t = torch()
    dt = s.dtype
    h = dev(inp["h"], dt)
    wr = dev(inp["w_router"], dt)
    br = dev_f32(inp["b_router"])
    bs = dev_f32(inp["b_select"])
    ws, nws = workspace(s)
    T, k, N = s.T, s.k, s.N
    ids, gates, p = i32(T * k), f32(T * k), f32(N)
    zl, ent = f32(1), f32(1)
    M.route(s, h, wr, br, bs, ids, gates, p, ws, nws, z_loss=zl, entropy=ent)
    counts, offsets, perm, row_of = i32(N), i32(N + 1), i32(T * k), i32(T * k)
    fo, la, cs = f32(N), f32(1), f32(2)
    M.dispatch(s, ids, counts, offsets, perm, row_of, p, fo, la, ws=ws, ws_bytes=nws, cap_stats=cs)
    wg, wu, wd = dev(inp["w_gate"], dt), dev(inp["w_up"], dt), dev(inp["w_down"], dt)
    sg, su, sd = dev(inp["sh_gate"], dt), dev(inp["sh_up"], dt), dev(inp["sh_down"], dt)
    rows_n = T * k + (T if s.d_ff_shared else 0)
    out_rows = t.empty((rows_n, s.d), dtype=tdtype(dt), device="cuda")
    M.expert_ffn(s, h, perm, offsets, wg, wu, wd, sg, su, sd, out_rows, ws, nws)
    y = t.empty((T, s.d), dtype=tdtype(dt), device="cuda")
    M.combine(s, out_rows, row_of, gates, y)
    t.cuda.synchronize()
    res = dict(ids=host(ids).reshape(T, k), gates=host(gates).reshape(T, k), p=host(p),
               counts=host(counts), offsets=host(offsets), perm=host(perm), row_of=host(row_of),
               f=host(fo), l_aux=float(host(la)[0]), out_rows=host(out_rows), y=host(y),
               z_loss=float(host(zl)[0]), entropy=float(host(ent)[0]), cap_stats=host(cs))
    # the fused call on the same inputs must agree bit for bit
    y2 = t.empty_like(y)
    ids2, g2, c2, f2, p2, l2 = i32(T * k), f32(T * k), i32(N), f32(N), f32(N), f32(1)
    zl2, ent2, cs2 = f32(1), f32(1), f32(2)
    M.layer_fused(s, h, wr, br, bs, wg, wu, wd, sg, su, sd, y2, ids2, g2, c2, f2, p2, l2, ws, nws,
                  z_loss=zl2, entropy=ent2, cap_stats=cs2)
    t.cuda.synchronize()
    res["fused"] = dict(y=host(y2), ids=host(ids2).reshape(T, k), gates=host(g2).reshape(T, k),
                        counts=host(c2), f=host(f2), p=host(p2), l_aux=float(host(l2)[0]),
                        z_loss=float(host(zl2)[0]), entropy=float(host(ent2)[0]),
                        cap_stats=host(cs2))
    return res


def check_all(s, inp, res, alpha=0.01):
    tol = TOL[s.dtype]
    r = O.route(inp["h"], inp["w_router"], s.k, s.mode, inp["b_router"], inp["b_select"],
                groups_of(s))
    near = check_ids(res["ids"], r, s.k, s.mode, inp["h"], inp["w_router"], inp["b_router"],
                     inp["b_select"], grouped=groups_of(s) is not None)
    ok = ~near
    check_gates(res["gates"], r.gates, 1e-4, ok, res["ids"], r.ids)
    # dispatch: bit-exact against the oracle's dispatch of the GPU's own ids
    cap = capacity_of(s)
    d = O.dispatch(res["ids"], s.N, cap)
    kept = int(d.offsets[-1])
    assert np.array_equal(res["counts"], d.counts)
    assert np.array_equal(res["offsets"], d.offsets)
    assert np.array_equal(res["perm"][:kept], d.perm_src)
    assert np.array_equal(res["row_of"], d.row_of)
    # capacity usage and dropped fraction: the fp32 rounding of the exact ratios
    want = O.capacity_stats(d, cap) if cap else (0.0, 0.0)
    assert np.array_equal(res["cap_stats"], np.float32(want).astype(np.float64)), \
        (res["cap_stats"], want)
    # stats
    f, p, l_aux = O.load_stats(d.counts, r.stat_prob, s.k, alpha)
    assert np.allclose(res["f"], f, rtol=1e-6, atol=0)
    assert np.allclose(res["p"], p, rtol=1e-4, atol=1e-7)
    assert abs(res["l_aux"] - l_aux) <= 1e-4 * abs(l_aux) + 1e-9
    # router z-loss and routing entropy over every token (fp32 on the GPU)
    zl_ref, ent_ref = O.router_z_loss(r.z), O.routing_entropy(r.stat_prob)
    assert abs(res["z_loss"] - zl_ref) <= 1e-4 * abs(zl_ref) + 1e-6, (res["z_loss"], zl_ref)
    assert abs(res["entropy"] - ent_ref) <= 1e-4 * abs(ent_ref) + 1e-6, (res["entropy"], ent_ref)
    # expert rows: oracle experts on the GPU's dispatch (rows past the kept
    # total are not written when the capacity drops slots)
    rows_ref = O.expert_rows(inp["h"], d, s.k, oracle_weights(inp), oracle_shared(inp))
    written = np.ones(rows_ref.shape[0], dtype=bool)
    written[kept:s.T * s.k] = False
    check_close_rows(res["out_rows"], rows_ref, tol, written, what="out_rows")
    # combine of the GPU's rows and gates
    y_comb = O.combine(np.where(written[:, None], res["out_rows"], 0.0), res["row_of"],
                       res["gates"], s.d_ff_shared > 0)
    check_close_rows(res["y"], y_comb, tol, what="combine")
    # end to end against the oracle's own routing (non-near-tie tokens). With
    # a capacity a near-tie choice can move later tokens' drops, so then the
    # reference keeps the oracle's gates and experts but the GPU's selection.
    ref = O.layer(inp["h"], inp["w_router"], s.k, s.mode, oracle_weights(inp), inp["b_router"],
                  inp["b_select"], oracle_shared(inp), alpha, groups_of(s),
                  capacity_factor=s.capacity_factor or None)
    y_ref = ref.y
    if cap and near.any():
        y_ref = O.combine(rows_ref, d.row_of, np.where(ok[:, None], r.gates, res["gates"]),
                          s.d_ff_shared > 0)
    worst = check_close_rows(res["y"], y_ref, tol, ok, what="y")
    # the fused call is the same kernels: identical bits
    fz = res["fused"]
    assert np.array_equal(fz["y"], res["y"])
    assert np.array_equal(fz["ids"], res["ids"])
    assert np.array_equal(fz["gates"], res["gates"])
    assert np.array_equal(fz["counts"], res["counts"])
    assert np.array_equal(fz["p"], res["p"]) and fz["l_aux"] == res["l_aux"]
    assert fz["z_loss"] == res["z_loss"] and fz["entropy"] == res["entropy"]
    assert np.array_equal(fz["cap_stats"], res["cap_stats"])
    return worst, int(near.sum())


CASES = [
    # name, T, d, N, k, d_ff, d_ff_shared, dtype, mode
    ("tiny_f32_top2", 64, 32, 4, 2, 64, 0, W.DTYPE_F32, 0),
    ("tiny_f32_switch", 64, 32, 4, 1, 64, 0, W.DTYPE_F32, 1),
    ("f32_sigmoid_shared", 37, 48, 9, 3, 40, 24, W.DTYPE_F32, 2),
    ("bf16_decode_T16", 16, 256, 8, 2, 384, 0, W.DTYPE_BF16, 0),
    ("bf16_decode_T40_shared", 40, 128, 16, 4, 192, 128, W.DTYPE_BF16, 2),
    ("bf16_decode_T64_full", 64, 128, 6, 2, 128, 0, W.DTYPE_BF16, 1),
    ("bf16_prefill_bm128", 300, 128, 5, 2, 192, 0, W.DTYPE_BF16, 0),
    ("bf16_prefill_bm128_shared", 257, 192, 12, 3, 128, 192, W.DTYPE_BF16, 2),
    ("bf16_prefill_bm256", 2304, 128, 2, 1, 320, 0, W.DTYPE_BF16, 1),
    # at least 768 rows per expert but too few 256-row tiles to fill the
    # chip: 128-row tiles on 32-deep slabs, two blocks per CU (routed and
    # shared GEMMs); fewer rows per expert take the three-stage 64-deep tiles
    ("bf16_prefill_bm128_k32", 900, 128, 2, 2, 192, 128, W.DTYPE_BF16, 0),
    ("bf16_prefill_many_experts", 520, 128, 64, 8, 128, 0, W.DTYPE_BF16, 0),
    ("bf16_k16_N512", 200, 64, 512, 16, 64, 0, W.DTYPE_BF16, 0),
    ("bf16_N1_k1", 100, 64, 1, 1, 64, 64, W.DTYPE_BF16, 0),
    # K of 4096 and more: the tiles past the last full round of a work queue
    # (here: every tile) are split along K and summed by the last split
    ("bf16_split_k4096", 256, 4096, 2, 1, 256, 0, W.DTYPE_BF16, 0),
    ("bf16_split_down_k8192", 256, 256, 2, 1, 8192, 0, W.DTYPE_BF16, 1),
    ("bf16_split_shared_k4096", 128, 4096, 4, 1, 128, 4096, W.DTYPE_BF16, 2),
    # one selection block and one dispatch chunk: selection and dispatch in
    # one kernel; at most 64 rows per expert: the combine inside the
    # weight-streaming down GEMM (bf16)
    ("bf16_decode_T1", 1, 128, 8, 2, 128, 0, W.DTYPE_BF16, 0),
    # one token: the weight-streaming kernels narrow their column blocks so
    # that the two experts' work covers the CUs (16 columns for both here,
    # with three chunks in flight per wave: eight turns of the ring of
    # register sets over the down GEMM's K = 8192)
    ("bf16_decode_T1_wide", 1, 256, 8, 2, 8192, 0, W.DTYPE_BF16, 0),
    # the ring stopping part-way through a turn: K of 23 (gate/up) and 11
    # (down) 64-deep chunks over four waves
    ("bf16_decode_T1_ring_tail", 1, 1472, 8, 2, 704, 0, W.DTYPE_BF16, 0),
    ("bf16_decode_T32_shared", 32, 256, 8, 2, 384, 128, W.DTYPE_BF16, 0),
    ("bf16_decode_T16_N64_sigmoid", 16, 128, 64, 6, 128, 0, W.DTYPE_BF16, 2),
    ("bf16_decode_T5_N512_k16_shared", 5, 64, 512, 16, 64, 64, W.DTYPE_BF16, 1),
    ("f32_decode_T16_switch", 16, 32, 4, 1, 64, 0, W.DTYPE_F32, 1),
    ("bf16_decode_T16_N128_k8", 16, 128, 128, 8, 64, 0, W.DTYPE_BF16, 0),
    ("bf16_decode_T12_N256_k8_sigmoid_shared", 12, 128, 256, 8, 64, 64, W.DTYPE_BF16, 2),
    # more than 64 experts: four experts per lane up to 256 (32 or 64 lanes a
    # token), eight beyond
    ("bf16_N256_k8_T40", 40, 64, 256, 8, 64, 0, W.DTYPE_BF16, 0),
    ("bf16_N100_k6_switch", 300, 128, 100, 6, 128, 0, W.DTYPE_BF16, 1),
    ("bf16_N200_sigmoid_shared", 150, 64, 200, 8, 64, 64, W.DTYPE_BF16, 2),
    ("f32_N128_k8", 40, 32, 128, 8, 32, 0, W.DTYPE_F32, 0),
    # d_ff_shared = d_ff: the shared expert runs as one more group of the
    # routed experts' launches (three-stage 128-row tiles, 256-row tiles, a
    # split-K tail in gate/up); with 512 routed experts it runs on its own
    ("bf16_shared_in_routed_mid", 700, 256, 16, 4, 256, 256, W.DTYPE_BF16, 0),
    ("bf16_shared_in_routed_bm256", 2304, 128, 2, 1, 320, 320, W.DTYPE_BF16, 1),
    ("bf16_shared_in_routed_split_k4096", 128, 4096, 4, 1, 128, 128, W.DTYPE_BF16, 2),
    ("bf16_shared_N512_alone", 300, 64, 512, 8, 64, 64, W.DTYPE_BF16, 2),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_layer_parity(case):
    name, T, d, N, k, dff, dfs, dt, mode = case
    inp = W.random_small(T, d, N, k, dff, dfs, dt, mode, seed=len(name), router_bias=(T % 2 == 0))
    s = shape_of(T, d, N, k, dff, dfs, dt, mode)
    print(f"case {name}", flush=True)
    res = run_steps(s, inp)
    worst, near = check_all(s, inp, res)
    print(f"{name}: worst row rel err {worst:.2e}, near-ties {near}")


GROUPED_CASES = [
    # name, T, d, N, k, d_ff, d_ff_shared, dtype, mode, (n_groups, topk_groups, group_topm)
    ("bf16_grouped_C_8x4_top2sum", 300, 128, 64, 8, 128, 128, W.DTYPE_BF16, 2, (8, 4, 2)),
    ("bf16_grouped_A_groupmax", 257, 192, 16, 2, 128, 0, W.DTYPE_BF16, 0, (4, 1, 1)),
    ("bf16_grouped_B_top2sum", 200, 128, 32, 4, 128, 0, W.DTYPE_BF16, 1, (8, 2, 2)),
    ("f32_grouped_C_shared", 64, 32, 12, 3, 40, 24, W.DTYPE_F32, 2, (3, 2, 2)),
    ("bf16_grouped_N256_64groups", 150, 64, 256, 8, 64, 0, W.DTYPE_BF16, 0, (64, 8, 4)),
    ("bf16_grouped_N512_16groups", 100, 64, 512, 16, 64, 0, W.DTYPE_BF16, 2, (16, 3, 8)),
    ("bf16_grouped_decode_T12", 12, 128, 32, 4, 128, 0, W.DTYPE_BF16, 2, (8, 2, 2)),
    ("bf16_grouped_decode_T9_N256", 9, 64, 256, 8, 64, 64, W.DTYPE_BF16, 2, (8, 4, 2)),
]


@pytest.mark.parametrize("case", GROUPED_CASES, ids=[c[0] for c in GROUPED_CASES])
def test_layer_parity_grouped(case):
    """Group-limited selection through every call and the fused layer."""
    name, T, d, N, k, dff, dfs, dt, mode, groups = case
    inp = W.random_small(T, d, N, k, dff, dfs, dt, mode, seed=len(name), router_bias=(T % 2 == 0))
    s = shape_of(T, d, N, k, dff, dfs, dt, mode, groups=groups)
    print(f"case {name}", flush=True)
    res = run_steps(s, inp)
    worst, near = check_all(s, inp, res)
    print(f"{name}: worst row rel err {worst:.2e}, near-ties {near}")


CAPACITY_CASES = [
    # name, T, d, N, k, d_ff, d_ff_shared, dtype, mode, groups, capacity_factor
    ("f32_cap_sigmoid_shared", 37, 48, 9, 3, 40, 24, W.DTYPE_F32, 2, None, 0.75),
    ("f32_cap_switch", 64, 32, 4, 1, 64, 0, W.DTYPE_F32, 1, None, 1.0),
    ("bf16_cap_prefill_bm128", 300, 128, 5, 2, 192, 0, W.DTYPE_BF16, 0, None, 1.0),
    # C = 33 rows per expert at most: the weight-streaming kernels
    ("bf16_cap_skinny", 520, 128, 64, 8, 128, 0, W.DTYPE_BF16, 0, None, 0.5),
    ("bf16_cap_bm256", 2304, 128, 2, 1, 320, 0, W.DTYPE_BF16, 1, None, 1.0),
    ("bf16_cap_grouped_shared", 300, 128, 64, 8, 128, 128, W.DTYPE_BF16, 2, (8, 4, 2), 1.25),
    # split-K tail with dropped rows
    ("bf16_cap_split_k4096", 256, 4096, 2, 1, 256, 0, W.DTYPE_BF16, 0, None, 0.6),
    # C = T k: nothing dropped, usage 1/N
    ("bf16_cap_keeps_all", 257, 192, 12, 3, 128, 0, W.DTYPE_BF16, 0, None, 12.0),
    # selection, dispatch with drops and the fused combine of a decode batch
    ("bf16_cap_decode_T16_shared", 16, 128, 8, 2, 192, 64, W.DTYPE_BF16, 0, None, 0.5),
]


@pytest.mark.parametrize("case", CAPACITY_CASES, ids=[c[0] for c in CAPACITY_CASES])
def test_layer_parity_capacity(case):
    """Expert capacity through every call and the fused layer: bit-exact
    dispatch with dropped slots (row_of = -1), exact usage and drop
    fraction, rows and y to tolerance."""
    name, T, d, N, k, dff, dfs, dt, mode, groups, cf = case
    inp = W.random_small(T, d, N, k, dff, dfs, dt, mode, seed=len(name), router_bias=(T % 2 == 0))
    s = shape_of(T, d, N, k, dff, dfs, dt, mode, groups=groups, cf=cf)
    print(f"case {name}", flush=True)
    res = run_steps(s, inp)
    worst, near = check_all(s, inp, res)
    dropped = int((res["row_of"] < 0).sum())
    if cf < N / k:
        assert dropped > 0, "the case is meant to drop slots"
    else:
        assert dropped == 0
    print(f"{name}: worst row rel err {worst:.2e}, near-ties {near}, dropped {dropped}")


def test_dispatch_capacity_worked_example_on_gpu():
    """The four-token grouping example with capacity factor 1 (C = 2): E2's
    third slot (token 3) is dropped, the rest keep their order."""
    import pins
    g = pins.golden("dispatch_grouping_example.json")
    s = shape_of(4, 64, 4, 2, 64, 0, W.DTYPE_BF16, 0, cf=1.0)
    t = torch()
    ids = t.tensor(np.array(g["ids"]).reshape(-1), dtype=t.int32, device="cuda")
    counts, offsets, perm, row_of, cs = i32(4), i32(5), i32(8), i32(8), f32(2)
    ws, nws = workspace(s)
    M.dispatch(s, ids, counts, offsets, perm, row_of, ws=ws, ws_bytes=nws, cap_stats=cs)
    t.cuda.synchronize()
    assert host(counts).tolist() == [2, 2, 3, 1]
    assert host(offsets).tolist() == [0, 2, 4, 6, 7]
    assert host(perm)[:7].tolist() == [0, 4, 2, 7, 1, 3, 5]
    assert host(row_of).tolist() == [0, 4, 2, 5, 1, 6, -1, 3]
    assert host(cs).tolist() == [7 / 8, 1 / 8]


def test_route_group_limited_worked_example_on_gpu():
    """Groups A = [0.90, 0.10], B = [0.80, 0.79], k = 2 (fp32, W_r = I):
    no limit -> {0, 2}; keep the group with the larger maximum -> {0, 1};
    keep the group with the larger top-2 sum -> {2, 3}; as sigmoid scores
    (mode C, zero bias) and as softmax probabilities (mode A)."""
    import pins
    g = pins.golden("group_limited_example.json")
    sc = np.array(g["scores"])
    G = g["n_groups"]
    for mode, z, b in ((2, np.log(sc / (1 - sc)), np.zeros(4)), (0, np.log(sc), None)):
        for groups, want in ((None, g["unrestricted"]), ((G, 1, 1), g["keep_1_group_by_max"]),
                             ((G, 1, 2), g["keep_1_group_by_top2_sum"])):
            s = shape_of(1, 4, 4, 2, 64, 0, W.DTYPE_F32, mode, groups=groups)
            ws, nws = workspace(s)
            ids, gates = i32(2), f32(2)
            M.route(s, dev_f32(z[None, :]), dev_f32(np.eye(4)), None, dev_f32(b), ids, gates, None,
                    ws, nws)
            torch().cuda.synchronize()
            assert host(ids).tolist() == want, (mode, groups)
            if mode == 2:
                assert np.allclose(host(gates), sc[want] / sc[want].sum(), rtol=1e-6, atol=0)


def test_tiny_workloads_exact_recipe():
    """The tiny fp32 workloads (top-2 renorm and top-1 Switch) at their
    stated sizes and seeds."""
    for w in (W.TINY, W.TINY_SWITCH):
        inp = W.host_inputs(w)
        s = shape_of(w.T, w.d, w.N, w.k, w.d_ff, 0, w.dtype, w.mode)
        res = run_steps(s, inp)
        worst, near = check_all(s, inp, res)
        assert near == 0
        assert worst < 1e-5


def test_route_worked_example_on_gpu():
    """Logits [2.2, 0.5, 1.8, -0.4] fed as h with W_r = I (fp32):
    softmax-renorm top-2 gives experts {0, 2} and gates within 5e-4 of the
    printed [0.599, 0.401]; [2, 1, 0] gives [0.731, 0.269]; Switch keeps the
    full-softmax probability."""
    import pins
    g = pins.golden("softmax_worked_example.json")
    s = shape_of(1, 4, 4, 2, 64, 0, W.DTYPE_F32, 0)
    ws, nws = workspace(s)
    ids, gates, p = i32(2), f32(2), f32(4)
    h = dev_f32(np.array([g["logits"]]))
    M.route(s, h, dev_f32(np.eye(4)), None, None, ids, gates, p, ws, nws)
    torch().cuda.synchronize()
    assert host(ids).tolist() == g["top2_experts"]
    assert np.all(np.abs(host(gates) - g["top2_gates_printed"]) <= g["printed_tolerance"])
    assert np.all(np.abs(host(p) - g["softmax_printed"]) <= g["printed_tolerance"])
    g2 = pins.golden("top2_renorm_example.json")
    s = shape_of(1, 3, 3, 2, 64, 0, W.DTYPE_F32, 0)
    M.route(s, dev_f32(np.array([g2["scores"]])), dev_f32(np.eye(3)), None, None, ids, gates,
            None, ws, nws)
    torch().cuda.synchronize()
    assert np.all(np.abs(host(gates) - g2["top2_gates_printed"]) <= g2["printed_tolerance"])
    s = shape_of(1, 3, 3, 2, 64, 0, W.DTYPE_F32, 1)
    M.route(s, dev_f32(np.array([g2["scores"]])), dev_f32(np.eye(3)), None, None, ids, gates,
            None, ws, nws)
    torch().cuda.synchronize()
    e = np.e
    assert np.allclose(host(gates), [e * e / (e * e + e + 1), e / (e * e + e + 1)], rtol=1e-6)


def test_route_ties_go_to_lower_index():
    s = shape_of(2, 4, 4, 2, 64, 0, W.DTYPE_F32, 0)
    ws, nws = workspace(s)
    ids, gates = i32(4), f32(4)
    h = dev_f32(np.array([[1.0, 3.0, 3.0, 2.0], [5.0, 5.0, 5.0, 5.0]]))
    M.route(s, h, dev_f32(np.eye(4)), None, None, ids, gates, None, ws, nws)
    torch().cuda.synchronize()
    assert host(ids).reshape(2, 2).tolist() == [[1, 2], [0, 1]]


def test_combine_worked_example_on_gpu():
    """2 tokens / 3 experts with hand-chosen expert outputs: y0 = [1.5, 1],
    y1 = [2.6, 2.2] -- a sum, never an overwrite."""
    import pins
    g = pins.golden("dispatch_combine_example.json")
    d = O.dispatch(np.array(g["ids"]), g["N"])
    eo = g["expert_outputs"]
    rows = np.zeros((4, 2))
    for (t, j), v in {(0, 0): eo["t0_e0"], (0, 1): eo["t0_e2"], (1, 0): eo["t1_e1"],
                      (1, 1): eo["t1_e2"]}.items():
        rows[d.row_of[t * 2 + j]] = v
    s = shape_of(2, 2, 3, 2, 64, 0, W.DTYPE_F32, 0)
    t = torch()
    y = t.empty((2, 2), dtype=t.float32, device="cuda")
    M.combine(s, dev_f32(rows), t.tensor(d.row_of, dtype=t.int32, device="cuda"),
              dev_f32(np.array(g["gates"])), y)
    t.cuda.synchronize()
    assert np.allclose(host(y), g["y_printed"], rtol=0, atol=1e-6)


def test_dispatch_grouping_example_on_gpu():
    import pins
    g = pins.golden("dispatch_grouping_example.json")
    s = shape_of(4, 64, 4, 2, 64, 0, W.DTYPE_BF16, 0)
    t = torch()
    ids = t.tensor(np.array(g["ids"]).reshape(-1), dtype=t.int32, device="cuda")
    counts, offsets, perm, row_of = i32(4), i32(5), i32(8), i32(8)
    ws, nws = workspace(s)
    M.dispatch(s, ids, counts, offsets, perm, row_of, ws=ws, ws_bytes=nws)
    t.cuda.synchronize()
    assert host(counts).tolist() == [2, 2, 3, 1]
    assert host(perm).tolist() == [0, 4, 2, 7, 1, 3, 6, 5]
    for e, toks in g["buckets_printed"].items():
        lo, hi = host(offsets)[int(e)], host(offsets)[int(e) + 1]
        assert (host(perm)[lo:hi] // 2).tolist() == toks


@pytest.mark.parametrize("T,N,k,cf", [(1, 1, 1, 0.0), (5, 7, 3, 0.0), (3000, 8, 2, 0.0),
                                      (2500, 128, 8, 0.0), (700, 512, 16, 0.0), (4097, 33, 5, 0.0),
                                      (1, 1, 1, 1.0), (5, 7, 3, 0.5), (3000, 8, 2, 1.0),
                                      (2500, 128, 8, 1.25), (700, 512, 16, 2.0),
                                      (4097, 33, 5, 0.1)])
def test_dispatch_random(T, N, k, cf):
    rng = np.random.default_rng(T * 31 + N)
    # skewed: low expert ids are more popular
    pr = 1.0 / np.arange(1, N + 1) ** 1.1
    pr /= pr.sum()
    ids = np.stack([rng.choice(N, size=k, replace=False, p=pr) for _ in range(T)]).astype(np.int32)
    s = shape_of(T, 64, N, k, 64, 0, W.DTYPE_BF16, 0, cf=cf)
    t = torch()
    counts, offsets, perm, row_of = i32(N), i32(N + 1), i32(T * k), i32(T * k)
    pm = dev_f32(np.full(N, 1.0 / N))
    fo, la, cs = f32(N), f32(1), f32(2)
    ws, nws = workspace(s)
    M.dispatch(s, t.from_numpy(ids.reshape(-1)).cuda(), counts, offsets, perm, row_of, pm, fo, la,
               ws=ws, ws_bytes=nws, cap_stats=cs)
    t.cuda.synchronize()
    cap = capacity_of(s)
    d = O.dispatch(ids, N, cap)
    assert np.array_equal(host(counts), d.counts)
    assert np.array_equal(host(offsets), d.offsets)
    assert np.array_equal(host(perm)[:d.perm_src.size], d.perm_src)
    assert np.array_equal(host(row_of), d.row_of)
    want = O.capacity_stats(d, cap) if cap else (0.0, 0.0)
    assert np.array_equal(host(cs), np.float32(want).astype(np.float64))
    assert np.allclose(host(fo), d.counts / (T * k), rtol=1e-6, atol=0)
    assert abs(float(host(la)[0]) - 0.01 * N * np.sum(d.counts / (T * k) / N)) < 1e-6


@pytest.mark.parametrize("T,d,N,k,dff,dfs", [(520, 128, 64, 8, 128, 128),
                                              (256, 256, 2, 1, 8192, 0),
                                              (2048, 4096, 2, 1, 256, 0)])
def test_deterministic_repeat(T, d, N, k, dff, dfs):
    """Same inputs twice: ids, permutation-dependent outputs and y identical
    (the first two shapes run on the three-stage 128-row tiles, the second
    with the split-K tail of the grouped GEMMs; the third on the 256-row
    tiles, with a split-K tail in gate/up)."""
    inp = W.random_small(T, d, N, k, dff, dfs, W.DTYPE_BF16, 2, seed=5)
    s = shape_of(T, d, N, k, dff, dfs, W.DTYPE_BF16, 2)
    a = run_steps(s, inp)
    b = run_steps(s, inp)
    for key in ("ids", "gates", "perm", "row_of", "out_rows", "y", "p", "l_aux"):
        assert np.array_equal(np.asarray(a[key]), np.asarray(b[key])), key


@pytest.mark.parametrize("T,N,k,mode,dff", [(300, 16, 4, 0, 128), (300, 16, 4, 2, 128),
                                            (12, 8, 2, 0, 128), (12, 64, 8, 2, 128)])
def test_nan_token_keeps_valid_routing(T, N, k, mode, dff):
    """A NaN in one token's hidden state makes all its logits NaN. The token
    still gets k distinct experts in [0, N) (a NaN selects as -inf, ties to
    the lower index), only its own y row is non-finite, and every other
    token's y matches the oracle run without it (tokens do not interact)."""
    d = 128
    inp = W.random_small(T, d, N, k, dff, 0, W.DTYPE_BF16, mode, seed=T + N)
    bad = T // 3
    h_nan = inp["h"].copy()
    h_nan[bad, 5] = np.nan
    s = shape_of(T, d, N, k, dff, 0, W.DTYPE_BF16, mode)
    dt = W.DTYPE_BF16
    t = torch()
    ws, nws = workspace(s)
    y = t.empty((T, d), dtype=t.bfloat16, device="cuda")
    ids, gates, counts = i32(T * k), f32(T * k), i32(N)
    M.layer_fused(s, dev(h_nan, dt), dev(inp["w_router"], dt), dev_f32(inp["b_router"]),
                  dev_f32(inp["b_select"]), dev(inp["w_gate"], dt), dev(inp["w_up"], dt),
                  dev(inp["w_down"], dt), None, None, None, y, ids, gates, counts, ws=ws,
                  ws_bytes=nws)
    t.cuda.synchronize()
    g_ids = host(ids).reshape(T, k)
    assert g_ids.min() >= 0 and g_ids.max() < N
    assert all(len(set(r.tolist())) == k for r in g_ids)
    assert g_ids[bad].tolist() == list(range(k)), g_ids[bad]
    assert host(counts).sum() == T * k
    yh = host(y)
    assert not np.isfinite(yh[bad]).any()
    others = np.arange(T) != bad
    assert np.isfinite(yh[others]).all()
    ref = O.layer(np.where(others[:, None], inp["h"], 0.0), inp["w_router"], k, mode,
                  oracle_weights(inp), inp["b_router"], inp["b_select"])
    ok = others & ~O.near_tie_tokens(ref.routing.gap)
    assert np.array_equal(np.sort(g_ids[ok], axis=1), np.sort(ref.routing.ids[ok], axis=1))
    check_close_rows(yh, ref.y, TOL[dt], ok, what="y (tokens other than the NaN one)")


def test_dispatch_ids_out_of_range_get_no_row():
    """Caller ids outside [0, N) take no bucket row: row_of = -1, and the
    other slots are placed as if they were absent (stable, by expert)."""
    T, N, k = 40, 6, 3
    rng = np.random.default_rng(11)
    ids = np.stack([rng.choice(N, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    ids[3, 1], ids[17, 0], ids[39, 2] = -1, N, 1 << 20
    s = shape_of(T, 64, N, k, 64)
    t = torch()
    counts, offsets, perm, row_of = i32(N), i32(N + 1), i32(T * k), i32(T * k)
    row_of.fill_(12345)
    ws, nws = workspace(s)
    M.dispatch(s, t.from_numpy(ids.reshape(-1)).cuda(), counts, offsets, perm, row_of, ws=ws,
               ws_bytes=nws)
    t.cuda.synchronize()
    flat = ids.reshape(-1)
    want_perm = np.concatenate([np.nonzero(flat == e)[0] for e in range(N)])
    want_counts = np.array([(flat == e).sum() for e in range(N)])
    want_row = np.full(T * k, -1)
    want_row[want_perm] = np.arange(want_perm.size)
    assert np.array_equal(host(counts), want_counts)
    assert np.array_equal(host(offsets), np.concatenate([[0], np.cumsum(want_counts)]))
    assert np.array_equal(host(perm)[:want_perm.size], want_perm)
    assert np.array_equal(host(row_of), want_row)


@pytest.mark.parametrize("T,N,k,dff", [(20, 8, 4, 256), (40, 4, 2, 128)])
def test_repeated_expert_ids_from_the_caller(T, N, k, dff):
    """Caller ids that name one expert twice for a token: that expert gets
    more rows than tokens (here more than the weight-streaming kernels take
    in one pass), every row is still computed, and combine adds both slots."""
    d = 128
    inp = W.random_small(T, d, N, k, dff, 0, W.DTYPE_BF16, 0, seed=T)
    rng = np.random.default_rng(T)
    ids = np.stack([np.concatenate([[0, 0], rng.choice(np.arange(1, N), size=k - 2,
                                                        replace=False)]) for _ in range(T)])
    ids = ids.astype(np.int32)
    gates = rng.uniform(0.1, 1.0, (T, k)).astype(np.float32)
    s = shape_of(T, d, N, k, dff)
    dt = W.DTYPE_BF16
    t = torch()
    ws, nws = workspace(s)
    counts, offsets, perm, row_of = i32(N), i32(N + 1), i32(T * k), i32(T * k)
    M.dispatch(s, t.from_numpy(ids.reshape(-1)).cuda(), counts, offsets, perm, row_of, ws=ws,
               ws_bytes=nws)
    out_rows = t.empty((T * k, d), dtype=t.bfloat16, device="cuda")
    M.expert_ffn(s, dev(inp["h"], dt), perm, offsets, dev(inp["w_gate"], dt),
                 dev(inp["w_up"], dt), dev(inp["w_down"], dt), None, None, None, out_rows, ws,
                 nws)
    y = t.empty((T, d), dtype=t.bfloat16, device="cuda")
    M.combine(s, out_rows, row_of, dev_f32(gates.reshape(-1)), y)
    t.cuda.synchronize()
    assert host(counts)[0] == 2 * T
    disp = O.dispatch(ids, N)
    assert np.array_equal(host(perm), disp.perm_src)
    rows_ref = O.expert_rows(inp["h"], disp, k, oracle_weights(inp))
    check_close_rows(host(out_rows), rows_ref, TOL[dt], what="out_rows")
    y_ref = O.combine(rows_ref, disp.row_of, gates.astype(np.float64))
    check_close_rows(host(y), y_ref, TOL[dt], what="y")
