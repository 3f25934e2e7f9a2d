"""C-ABI checks that need no GPU: the library loads, exports every function
include/moe.h declares, sizes workspaces, and rejects invalid arguments
before making any HIP call (so these run on a machine without a GPU).

Fake device pointers are only passed in cases that fail validation; the
library never dereferences them there."""
import ctypes
import os
import re

import pytest

import sparse_mixture_experts_35_amd as M

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe.h")
FAKE = 0x10000   # 64 KiB-aligned, never dereferenced


def declared_functions():
    src = open(HDR, encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = M.lib()
    names = declared_functions()
    assert set(names) == set(M.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.moe_abi_version() == 6


def test_status_strings():
    lib = M.lib()
    for st, name in [(0, "MOE_OK"), (1, "MOE_ERR_INVALID_ARG"), (2, "MOE_ERR_UNSUPPORTED"),
                     (3, "MOE_ERR_WORKSPACE"), (4, "MOE_ERR_HIP")]:
        assert lib.moe_status_string(st).decode() == name


def shape(**kw):
    base = dict(T=64, d=64, N=8, k=2, d_ff=128, d_ff_shared=0, dtype=M.BF16,
                mode=M.SOFTMAX_RENORM, aux_alpha=0.01)
    base.update(kw)
    return M.Shape(**base)


def test_workspace_bytes():
    a = M.workspace_bytes(shape())
    b = M.workspace_bytes(shape(T=128))
    c = M.workspace_bytes(shape(d_ff_shared=128))
    assert 0 < a < b and a < c
    assert M.workspace_bytes(shape(k=9)) == 0          # invalid shape
    assert M.workspace_bytes(shape(T=0)) > 0           # N-sized scratch remains


def fused(s, **over):
    args = dict(h=FAKE, w_router=FAKE, b_router=None, b_select=None, w_gate=FAKE, w_up=FAKE,
                w_down=FAKE, sh_gate=None, sh_up=None, sh_down=None, y=FAKE, ws=FAKE,
                ws_bytes=1 << 40)
    args.update(over)
    lib = M.lib()
    st = lib.moe_layer_fused(ctypes.byref(s), args["h"], args["w_router"], args["b_router"],
                             args["b_select"], args["w_gate"], args["w_up"], args["w_down"],
                             args["sh_gate"], args["sh_up"], args["sh_down"], args["y"],
                             None, None, None, None, None, None, None, None, None, args["ws"],
                             args["ws_bytes"], None)
    return st, lib.moe_last_error().decode()


@pytest.mark.parametrize("kw,want,msg", [
    (dict(T=-1), M.ERR_INVALID_ARG, "T < 0"),
    (dict(d=0), M.ERR_INVALID_ARG, ">= 1"),
    (dict(N=0), M.ERR_INVALID_ARG, ">= 1"),
    (dict(k=0), M.ERR_INVALID_ARG, ">= 1"),
    (dict(k=9), M.ERR_INVALID_ARG, "not enough candidate"),
    (dict(N=513, k=2), M.ERR_UNSUPPORTED, "N > 512"),
    (dict(N=32, k=17), M.ERR_UNSUPPORTED, "k > 16"),
    (dict(d=96), M.ERR_UNSUPPORTED, "multiples of 64"),
    (dict(d_ff=100), M.ERR_UNSUPPORTED, "multiples of 64"),
    (dict(d_ff_shared=32), M.ERR_UNSUPPORTED, "multiples of 64"),
    (dict(dtype=7), M.ERR_INVALID_ARG, "dtype"),
    (dict(mode=3), M.ERR_INVALID_ARG, "mode"),
    (dict(aux_alpha=float("nan")), M.ERR_INVALID_ARG, "aux_alpha"),
    (dict(T=1 << 28, d=4096), M.ERR_UNSUPPORTED, "2^31"),
    (dict(topk_groups=1), M.ERR_INVALID_ARG, "need n_groups > 0"),
    (dict(n_groups=3, topk_groups=1, group_topm=1), M.ERR_INVALID_ARG, "divide N"),
    (dict(n_groups=4, topk_groups=0, group_topm=1), M.ERR_INVALID_ARG, "topk_groups"),
    (dict(n_groups=4, topk_groups=5, group_topm=1), M.ERR_INVALID_ARG, "topk_groups"),
    (dict(n_groups=4, topk_groups=2, group_topm=3), M.ERR_INVALID_ARG, "group_topm"),
    (dict(n_groups=8, topk_groups=1, group_topm=1), M.ERR_INVALID_ARG, "fewer than k"),
    (dict(N=256, n_groups=128, topk_groups=8, group_topm=1), M.ERR_UNSUPPORTED, "n_groups > 64"),
    (dict(N=256, n_groups=8, topk_groups=4, group_topm=9), M.ERR_UNSUPPORTED, "group_topm > 8"),
    (dict(capacity_factor=-0.5), M.ERR_INVALID_ARG, "capacity_factor"),
    (dict(capacity_factor=float("inf")), M.ERR_INVALID_ARG, "capacity_factor"),
    (dict(capacity_factor=float("nan")), M.ERR_INVALID_ARG, "capacity_factor"),
    (dict(N=8, capacity_factor=8.5), M.ERR_INVALID_ARG, "capacity_factor"),
])
def test_bad_shapes(kw, want, msg):
    st, err = fused(shape(**kw))
    assert st == want, err
    assert msg in err


def test_bad_pointers_and_workspace():
    s = shape()
    assert fused(s, h=None)[0] == M.ERR_INVALID_ARG
    st, err = fused(s, w_gate=FAKE + 8)
    assert st == M.ERR_INVALID_ARG and "aligned" in err
    st, err = fused(s, b_select=FAKE)
    assert st == M.ERR_INVALID_ARG and "b_select" in err
    st, err = fused(shape(mode=M.SIGMOID_BIAS_RENORM))
    assert st == M.ERR_INVALID_ARG and "b_select" in err
    st, err = fused(s, sh_gate=FAKE, sh_up=FAKE, sh_down=FAKE)
    assert st == M.ERR_INVALID_ARG and "d_ff_shared" in err
    st, err = fused(shape(d_ff_shared=128))
    assert st == M.ERR_INVALID_ARG and "sh_gate" in err
    st, err = fused(s, ws_bytes=M.workspace_bytes(s) - 1)
    assert st == M.ERR_WORKSPACE and "too small" in err
    st, err = fused(s, ws=None)
    assert st == M.ERR_WORKSPACE


def test_zero_tokens_is_a_noop():
    s = shape(T=0)
    st, err = fused(s, ws_bytes=M.workspace_bytes(s))
    assert st == M.OK, err
    s = shape(T=0, capacity_factor=1.25)
    st, err = fused(s, ws_bytes=M.workspace_bytes(s))
    assert st == M.OK, err


def test_capacity_factor_limits_accepted():
    """0 (dropless) and every factor up to N validate (checked with T = 0 so
    that nothing launches)."""
    for cf in (0.0, 1e-6, 1.0, 1.25, 8.0):
        s = shape(T=0, capacity_factor=cf)
        st, err = fused(s, ws_bytes=M.workspace_bytes(s))
        assert st == M.OK, (cf, err)


def test_other_entry_points_validate():
    lib = M.lib()
    s = shape(k=9)
    assert lib.moe_route(ctypes.byref(s), FAKE, FAKE, None, None, FAKE, FAKE, None, None, None,
                         FAKE, 1 << 40, None) == M.ERR_INVALID_ARG
    s = shape()
    assert lib.moe_route(ctypes.byref(s), FAKE, FAKE, None, None, None, FAKE, None, None, None,
                         FAKE, 1 << 40, None) == M.ERR_INVALID_ARG
    assert lib.moe_route(ctypes.byref(s), FAKE, FAKE, None, None, FAKE, FAKE, None, None, None,
                         FAKE, 16, None) == M.ERR_WORKSPACE
    assert lib.moe_route(ctypes.byref(s), FAKE, FAKE, None, None, FAKE, FAKE, None, FAKE + 2,
                         None, FAKE, 1 << 40, None) == M.ERR_INVALID_ARG   # misaligned z_loss
    assert lib.moe_dispatch(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE,
                            None, None, 0, None) == M.ERR_INVALID_ARG     # l_aux without p_mean
    assert lib.moe_dispatch(ctypes.byref(s), FAKE, None, FAKE, FAKE, FAKE, None, None, None,
                            None, None, 0, None) == M.ERR_INVALID_ARG
    assert lib.moe_dispatch(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None,
                            FAKE + 2, None, 0, None) == M.ERR_INVALID_ARG  # misaligned cap_stats
    assert lib.moe_expert_ffn(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                              None, FAKE, FAKE, 8, None) == M.ERR_WORKSPACE
    assert lib.moe_combine(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE + 4, None) == M.ERR_INVALID_ARG
    assert lib.moe_layer_fused_marked(ctypes.byref(s), *([FAKE] * 3), None, *([FAKE] * 3),
                                      None, None, None, FAKE, *([None] * 9), FAKE, 1 << 40, None,
                                      None) == M.ERR_INVALID_ARG


def test_missing_library_raises(monkeypatch, tmp_path):
    monkeypatch.setattr(M, "_lib", None)
    monkeypatch.setattr(M, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(M.MoEError):
        M.lib()


@pytest.mark.parametrize("lang,compiler", [("c", "gcc"), ("c++", "g++")])
def test_header_compiles(lang, compiler, tmp_path):
    """include/moe.h is a self-contained C and C++ header."""
    import shutil
    import subprocess
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not available")
    src = tmp_path / ("use.c" if lang == "c" else "use.cpp")
    src.write_text('#include "moe.h"\nint main(void) { return (int)moe_abi_version(); }\n')
    r = subprocess.run([compiler, "-fsyntax-only", "-Wall", "-Werror", "-I", os.path.dirname(HDR),
                        str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def backward(s, **over):
    names = ["h", "w_router", "b_router", "w_gate", "w_up", "w_down", "sh_gate", "sh_up",
             "sh_down", "topk_ids", "topk_gates", "counts", "offsets", "perm_src", "row_of",
             "preact", "dy"]
    outs = ["dh", "dw_router", "db_router", "dw_gate", "dw_up", "dw_down", "dsh_gate", "dsh_up",
            "dsh_down", "dgates"]
    args = {n: FAKE for n in names + outs}
    for n in ("b_router", "sh_gate", "sh_up", "sh_down", "preact", "db_router", "dsh_gate",
              "dsh_up", "dsh_down", "dgates"):
        args[n] = None
    args.update(d_laux=0.0, d_zloss=0.0, ws=FAKE, ws_bytes=1 << 40)
    args.update(over)
    lib = M.lib()
    st = lib.moe_layer_backward(ctypes.byref(s), *[args[n] for n in names], args["d_laux"],
                                args["d_zloss"], *[args[n] for n in outs], args["ws"],
                                args["ws_bytes"], None)
    return st, lib.moe_last_error().decode()


def test_backward_validates():
    s = shape()
    assert M.backward_workspace_bytes(s) > M.workspace_bytes(s) > 0
    assert M.backward_workspace_bytes(shape(k=9)) == 0
    assert backward(shape(T=0), ws_bytes=M.backward_workspace_bytes(shape(T=0)))[0] == M.OK
    st, err = backward(s, dy=None)
    assert st == M.ERR_INVALID_ARG and "dy" in err
    st, err = backward(s, dw_router=FAKE + 2)
    assert st == M.ERR_INVALID_ARG and "dw_router" in err
    st, err = backward(s, dsh_gate=FAKE)
    assert st == M.ERR_INVALID_ARG and "d_ff_shared" in err
    st, err = backward(shape(d_ff_shared=128), sh_gate=FAKE, sh_up=FAKE, sh_down=FAKE)
    assert st == M.ERR_INVALID_ARG and "dsh_gate" in err
    st, err = backward(s, d_laux=float("nan"))
    assert st == M.ERR_INVALID_ARG and "finite" in err
    st, err = backward(s, ws_bytes=M.backward_workspace_bytes(s) - 1)
    assert st == M.ERR_WORKSPACE
    st, err = backward(shape(T=1 << 20, d=4096, d_ff=14336, N=8, k=2))
    assert st == M.ERR_UNSUPPORTED and "2^31" in err


def test_forward_train_validates():
    lib = M.lib()
    s = shape()
    def call(**over):
        a = dict(h=FAKE, w_router=FAKE, b_router=None, b_select=None, w_gate=FAKE, w_up=FAKE,
                 w_down=FAKE, sh_gate=None, sh_up=None, sh_down=None, y=FAKE, topk_ids=FAKE,
                 topk_gates=FAKE, counts=FAKE, offsets=FAKE, perm_src=FAKE, row_of=FAKE,
                 preact=None, p_out=None, l_aux=None, z_loss=None, entropy=None)
        a.update(over)
        st = lib.moe_layer_forward_train(ctypes.byref(s), *a.values(), FAKE, 1 << 40, None)
        return st, lib.moe_last_error().decode()
    st, err = call(offsets=None)
    assert st == M.ERR_INVALID_ARG and "offsets" in err
    st, err = call(preact=FAKE + 2)
    assert st == M.ERR_INVALID_ARG and "preact" in err
    st, err = call(h=None)
    assert st == M.ERR_INVALID_ARG and "h" in err


def test_noalloc_rejects_shapes_beyond_its_scratch():
    """The allocation-free call checks its arguments and its scratch limit
    before any HIP call: a shape that needs more than the 64 MiB static
    scratch (the Mixtral prefill layer: Act alone is 235 MB) is refused with
    MOE_ERR_WORKSPACE, a bad shape with MOE_ERR_INVALID_ARG."""
    lib = M.lib()
    big = M.Shape(4096, 4096, 8, 2, 14336, 0, M.BF16, M.SOFTMAX_RENORM, 0.01)
    st = lib.moe_layer_fused_noalloc(ctypes.byref(big), *([FAKE] * 3 + [None] * 1 + [FAKE] * 3
                                                         + [None] * 3 + [FAKE] + [None] * 9),
                                     None)
    assert st == M.ERR_WORKSPACE
    assert "64" in lib.moe_last_error().decode() or "67108864" in lib.moe_last_error().decode()
    bad = shape(k=9)
    st = lib.moe_layer_fused_noalloc(ctypes.byref(bad), *([FAKE] * 3 + [None] + [FAKE] * 3
                                                         + [None] * 3 + [FAKE] + [None] * 9),
                                     None)
    assert st == M.ERR_INVALID_ARG


def test_binding_rejects_short_and_strided_tensors():
    """A tensor argument smaller than the bytes the call uses through it, or
    not contiguous, raises MoEError in the binding before the library runs
    (the C ABI takes bare pointers and cannot tell). out_rows holds T k rows
    (and T more with a shared expert); one row short is refused."""
    torch = pytest.importorskip("torch")
    T, d, N, k, dff = 4, 64, 4, 2, 64
    s = M.Shape(T, d, N, k, dff, 0, M.BF16)
    bf = torch.bfloat16
    h = torch.zeros((T, d), dtype=bf)
    wg, wu = torch.zeros((N, dff, d), dtype=bf), torch.zeros((N, dff, d), dtype=bf)
    wd = torch.zeros((N, d, dff), dtype=bf)
    perm, off = torch.zeros(T * k, dtype=torch.int32), torch.zeros(N + 1, dtype=torch.int32)
    ws = torch.zeros(64, dtype=torch.uint8)
    short = torch.zeros((T * k - 1, d), dtype=bf)
    with pytest.raises(M.MoEError, match="out_rows holds"):
        M.expert_ffn(s, h, perm, off, wg, wu, wd, None, None, None, short, ws, 64)
    strided = torch.zeros((T, 2 * d), dtype=bf)[:, ::2]
    with pytest.raises(M.MoEError, match="h is not contiguous"):
        M.expert_ffn(s, strided, perm, off, wg, wu, wd, None, None, None,
                     torch.zeros((T * k, d), dtype=bf), ws, 64)
    with pytest.raises(M.MoEError, match="ws holds"):
        M.expert_ffn(s, h, perm, off, wg, wu, wd, None, None, None,
                     torch.zeros((T * k, d), dtype=bf), ws, 65)
    s2 = M.Shape(T, d, N, k, dff, 32, M.BF16)
    with pytest.raises(M.MoEError, match="out_rows holds"):
        M.combine(s2, torch.zeros((T * k, d), dtype=bf), perm, torch.zeros(T * k), h)
