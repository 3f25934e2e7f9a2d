"""Thin Python binding of the MoE HIP library (libmoe_hip.so).

Argument marshalling only: every step of the layer runs in the library's
HIP kernels. PyTorch supplies device memory and the current HIP stream.
The library must be built (``python -m sparse_mixture_experts_35_amd.build``
or ``__graft_entry__.build()``); importing works without it, but every call
raises ``MoEError`` when it is missing. There is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_hip.so")

F32, BF16 = 0, 1
SOFTMAX_RENORM, SOFTMAX_FULL, SIGMOID_BIAS_RENORM = 0, 1, 2
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4
MAX_EXPERTS, MAX_TOPK, MAX_GROUPS, MAX_GROUP_TOPM = 512, 16, 64, 8

EXPORTS = ("moe_abi_version", "moe_status_string", "moe_last_error", "moe_workspace_bytes",
           "moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_layer_fused",
           "moe_layer_fused_marked", "moe_layer_forward_train", "moe_backward_workspace_bytes",
           "moe_layer_backward", "moe_layer_fused_noalloc")

NOALLOC_SCRATCH_BYTES = 64 << 20     # MOE_NOALLOC_SCRATCH_BYTES


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {_status_name(status)}: {detail}")


class Shape(ctypes.Structure):
    """moe_shape: sizes, dtype, gate mode, L_aux alpha, the optional group
    limit (n_groups contiguous expert groups, the topk_groups best by the sum
    of their group_topm largest selection scores stay candidates) and the
    optional expert capacity factor (0 = dropless)."""
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("N", ctypes.c_int32),
                ("k", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("d_ff_shared", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("mode", ctypes.c_int32), ("aux_alpha", ctypes.c_float),
                ("n_groups", ctypes.c_int32), ("topk_groups", ctypes.c_int32),
                ("group_topm", ctypes.c_int32), ("capacity_factor", ctypes.c_float)]

    def __init__(self, T, d, N, k, d_ff, d_ff_shared=0, dtype=BF16, mode=SOFTMAX_RENORM,
                 aux_alpha=0.01, n_groups=0, topk_groups=0, group_topm=0, capacity_factor=0.0):
        super().__init__(T, d, N, k, d_ff, d_ff_shared, dtype, mode, aux_alpha, n_groups,
                         topk_groups, group_topm, capacity_factor)


_lib = None
_P = ctypes.c_void_p
_SIG = {
    "moe_abi_version": (ctypes.c_int, []),
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(Shape)]),
    "moe_route": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_P] * 9 + [_P, ctypes.c_size_t, _P]),
    "moe_dispatch": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_P] * 9 + [_P, ctypes.c_size_t, _P]),
    "moe_expert_ffn": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_P] * 10 + [_P, ctypes.c_size_t, _P]),
    "moe_combine": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_P] * 5),
    "moe_layer_fused": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_P] * 20 + [_P, ctypes.c_size_t, _P]),
    "moe_layer_fused_marked": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_P] * 20
                               + [_P, ctypes.c_size_t, _P, _P]),
    "moe_layer_fused_noalloc": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_P] * 20 + [_P]),
    "moe_backward_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(Shape)]),
    "moe_layer_forward_train": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_P] * 22
                                + [_P, ctypes.c_size_t, _P]),
    "moe_layer_backward": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_P] * 17
                           + [ctypes.c_float, ctypes.c_float] + [_P] * 10
                           + [_P, ctypes.c_size_t, _P]),
}


def lib() -> ctypes.CDLL:
    """The loaded library; raises MoEError if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MoEError(ERR_HIP, "load", f"{LIB_PATH} is missing; build it with "
                           "`python -m sparse_mixture_experts_35_amd.build`")
        # PyTorch ships its own HIP runtime. With torch loaded first this
        # library binds to that runtime, so torch's tensors and streams are
        # valid here; loading this library first and torch afterwards ended
        # in "no ROCm-capable device is detected" and a crashed process.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIG.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def _status_name(st):
    try:
        return lib().moe_status_string(st).decode()
    except Exception:
        return str(st)


def _check(st, where):
    if st != OK:
        raise MoEError(st, where, lib().moe_last_error().decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _bytes_of(shape: Shape) -> dict:
    """Bytes the library reads or writes through each array argument (the
    layouts of include/moe.h)."""
    es = 2 if shape.dtype == BF16 else 4
    T, d, N, k = shape.T, shape.d, shape.N, shape.k
    f, fs = shape.d_ff, shape.d_ff_shared
    R = T * k
    return dict(h=T * d * es, w_router=N * d * es, b_router=4 * N, b_select=4 * N,
                topk_ids=4 * R, topk_gates=4 * R, p_mean=4 * N, p_out=4 * N, f_out=4 * N,
                counts=4 * N, offsets=4 * (N + 1), perm_src=4 * R, row_of=4 * R, l_aux=4,
                z_loss=4, entropy=4, cap_stats=8, w_gate=N * f * d * es, w_up=N * f * d * es,
                w_down=N * d * f * es, sh_gate=fs * d * es, sh_up=fs * d * es,
                sh_down=d * fs * es, out_rows=(R + (T if fs else 0)) * d * es, y=T * d * es,
                dy=T * d * es, dh=T * d * es, preact=4 * preact_floats(shape),
                dw_router=4 * N * d, db_router=4 * N, dw_gate=N * f * d * es,
                dw_up=N * f * d * es, dw_down=N * d * f * es, dsh_gate=fs * d * es,
                dsh_up=fs * d * es, dsh_down=d * fs * es, dgates=4 * R)


def _args(shape: Shape, where: str, ws_bytes: int = 0):
    """arg(t, name): the pointer of t. A tensor must be contiguous and hold
    at least the bytes the call uses through it (a raw int pointer is passed
    as it is): a short buffer raises MoEError instead of being overrun."""
    need = _bytes_of(shape)
    need["ws"] = int(ws_bytes)

    def arg(t, name):
        if t is None or isinstance(t, int):
            return _ptr(t)
        if not t.is_contiguous():
            raise MoEError(ERR_INVALID_ARG, where, f"{name} is not contiguous")
        have = t.numel() * t.element_size()
        if have < need[name]:
            raise MoEError(ERR_INVALID_ARG, where,
                           f"{name} holds {have} bytes; this shape needs {need[name]}")
        return t.data_ptr()
    return arg


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def workspace_bytes(shape: Shape) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(shape)))


def route(shape, h, w_router, b_router, b_select, topk_ids, topk_gates, p_mean, ws,
          ws_bytes, stream=None, z_loss=None, entropy=None):
    a = _args(shape, "moe_route", ws_bytes)
    _check(lib().moe_route(ctypes.byref(shape), a(h, "h"), a(w_router, "w_router"),
                           a(b_router, "b_router"), a(b_select, "b_select"),
                           a(topk_ids, "topk_ids"), a(topk_gates, "topk_gates"),
                           a(p_mean, "p_mean"), a(z_loss, "z_loss"), a(entropy, "entropy"),
                           a(ws, "ws"), ws_bytes, _stream(stream)), "moe_route")


def dispatch(shape, topk_ids, counts, offsets, perm_src, row_of, p_mean=None, f_out=None,
             l_aux=None, ws=None, ws_bytes=0, stream=None, cap_stats=None):
    a = _args(shape, "moe_dispatch", ws_bytes)
    _check(lib().moe_dispatch(ctypes.byref(shape), a(topk_ids, "topk_ids"), a(counts, "counts"),
                              a(offsets, "offsets"), a(perm_src, "perm_src"),
                              a(row_of, "row_of"), a(p_mean, "p_mean"), a(f_out, "f_out"),
                              a(l_aux, "l_aux"), a(cap_stats, "cap_stats"), a(ws, "ws"),
                              ws_bytes, _stream(stream)), "moe_dispatch")


def expert_ffn(shape, h, perm_src, offsets, w_gate, w_up, w_down, sh_gate, sh_up, sh_down,
               out_rows, ws, ws_bytes, stream=None):
    a = _args(shape, "moe_expert_ffn", ws_bytes)
    _check(lib().moe_expert_ffn(ctypes.byref(shape), a(h, "h"), a(perm_src, "perm_src"),
                                a(offsets, "offsets"), a(w_gate, "w_gate"), a(w_up, "w_up"),
                                a(w_down, "w_down"), a(sh_gate, "sh_gate"), a(sh_up, "sh_up"),
                                a(sh_down, "sh_down"), a(out_rows, "out_rows"), a(ws, "ws"),
                                ws_bytes, _stream(stream)), "moe_expert_ffn")


def combine(shape, out_rows, row_of, topk_gates, y, stream=None):
    a = _args(shape, "moe_combine")
    _check(lib().moe_combine(ctypes.byref(shape), a(out_rows, "out_rows"), a(row_of, "row_of"),
                             a(topk_gates, "topk_gates"), a(y, "y"), _stream(stream)),
           "moe_combine")


def layer_fused(shape, h, w_router, b_router, b_select, w_gate, w_up, w_down, sh_gate, sh_up,
                sh_down, y, topk_ids=None, topk_gates=None, counts=None, f_out=None,
                p_out=None, l_aux=None, ws=None, ws_bytes=0, stream=None, events=None,
                z_loss=None, entropy=None, cap_stats=None):
    a = _args(shape, "moe_layer_fused", ws_bytes)
    args = (ctypes.byref(shape), a(h, "h"), a(w_router, "w_router"), a(b_router, "b_router"),
            a(b_select, "b_select"), a(w_gate, "w_gate"), a(w_up, "w_up"), a(w_down, "w_down"),
            a(sh_gate, "sh_gate"), a(sh_up, "sh_up"), a(sh_down, "sh_down"), a(y, "y"),
            a(topk_ids, "topk_ids"), a(topk_gates, "topk_gates"), a(counts, "counts"),
            a(f_out, "f_out"), a(p_out, "p_out"), a(l_aux, "l_aux"), a(z_loss, "z_loss"),
            a(entropy, "entropy"), a(cap_stats, "cap_stats"), a(ws, "ws"), ws_bytes,
            _stream(stream))
    if events is None:
        _check(lib().moe_layer_fused(*args), "moe_layer_fused")
    else:
        arr = (ctypes.c_void_p * 6)(*events)
        _check(lib().moe_layer_fused_marked(*args, ctypes.cast(arr, ctypes.c_void_p)),
               "moe_layer_fused_marked")


def layer_fused_noalloc(shape, h, w_router, b_router, b_select, w_gate, w_up, w_down, sh_gate,
                        sh_up, sh_down, y, topk_ids=None, topk_gates=None, counts=None,
                        f_out=None, p_out=None, l_aux=None, stream=None, z_loss=None,
                        entropy=None, cap_stats=None):
    """moe_layer_fused_noalloc: the fused layer on the library's static
    scratch (no workspace argument)."""
    a = _args(shape, "moe_layer_fused_noalloc")
    _check(lib().moe_layer_fused_noalloc(
        ctypes.byref(shape), a(h, "h"), a(w_router, "w_router"), a(b_router, "b_router"),
        a(b_select, "b_select"), a(w_gate, "w_gate"), a(w_up, "w_up"), a(w_down, "w_down"),
        a(sh_gate, "sh_gate"), a(sh_up, "sh_up"), a(sh_down, "sh_down"), a(y, "y"),
        a(topk_ids, "topk_ids"), a(topk_gates, "topk_gates"), a(counts, "counts"),
        a(f_out, "f_out"), a(p_out, "p_out"), a(l_aux, "l_aux"), a(z_loss, "z_loss"),
        a(entropy, "entropy"), a(cap_stats, "cap_stats"), _stream(stream)),
        "moe_layer_fused_noalloc")


def layer_forward_train(shape, h, w_router, b_router, b_select, w_gate, w_up, w_down, sh_gate,
                        sh_up, sh_down, y, topk_ids, topk_gates, counts, offsets, perm_src,
                        row_of, preact=None, p_out=None, l_aux=None, z_loss=None, entropy=None,
                        ws=None, ws_bytes=0, stream=None):
    a = _args(shape, "moe_layer_forward_train", ws_bytes)
    _check(lib().moe_layer_forward_train(
        ctypes.byref(shape), a(h, "h"), a(w_router, "w_router"), a(b_router, "b_router"),
        a(b_select, "b_select"), a(w_gate, "w_gate"), a(w_up, "w_up"), a(w_down, "w_down"),
        a(sh_gate, "sh_gate"), a(sh_up, "sh_up"), a(sh_down, "sh_down"), a(y, "y"),
        a(topk_ids, "topk_ids"), a(topk_gates, "topk_gates"), a(counts, "counts"),
        a(offsets, "offsets"), a(perm_src, "perm_src"), a(row_of, "row_of"),
        a(preact, "preact"), a(p_out, "p_out"), a(l_aux, "l_aux"), a(z_loss, "z_loss"),
        a(entropy, "entropy"), a(ws, "ws"), ws_bytes, _stream(stream)),
        "moe_layer_forward_train")


def preact_floats(shape: Shape) -> int:
    """fp32 elements of moe_layer_forward_train's pre-activation output."""
    return (shape.T * shape.k * 2 * shape.d_ff
            + (shape.T * 2 * shape.d_ff_shared if shape.d_ff_shared else 0))


def backward_workspace_bytes(shape: Shape) -> int:
    return int(lib().moe_backward_workspace_bytes(ctypes.byref(shape)))


def layer_backward(shape, h, w_router, b_router, w_gate, w_up, w_down, sh_gate, sh_up, sh_down,
                   topk_ids, topk_gates, counts, offsets, perm_src, row_of, dy, dh, dw_router,
                   db_router, dw_gate, dw_up, dw_down, dsh_gate=None, dsh_up=None, dsh_down=None,
                   dgates=None, d_laux=0.0, d_zloss=0.0, ws=None, ws_bytes=0, stream=None,
                   preact=None):
    a = _args(shape, "moe_layer_backward", ws_bytes)
    _check(lib().moe_layer_backward(
        ctypes.byref(shape), a(h, "h"), a(w_router, "w_router"), a(b_router, "b_router"),
        a(w_gate, "w_gate"), a(w_up, "w_up"), a(w_down, "w_down"), a(sh_gate, "sh_gate"),
        a(sh_up, "sh_up"), a(sh_down, "sh_down"), a(topk_ids, "topk_ids"),
        a(topk_gates, "topk_gates"), a(counts, "counts"), a(offsets, "offsets"),
        a(perm_src, "perm_src"), a(row_of, "row_of"), a(preact, "preact"), a(dy, "dy"),
        float(d_laux), float(d_zloss), a(dh, "dh"), a(dw_router, "dw_router"),
        a(db_router, "db_router"), a(dw_gate, "dw_gate"), a(dw_up, "dw_up"),
        a(dw_down, "dw_down"), a(dsh_gate, "dsh_gate"), a(dsh_up, "dsh_up"),
        a(dsh_down, "dsh_down"), a(dgates, "dgates"), a(ws, "ws"), ws_bytes, _stream(stream)),
        "moe_layer_backward")


class MoELayer:
    """Convenience wrapper: holds the shape and a workspace tensor, allocates
    outputs with torch, calls moe_layer_fused."""

    def __init__(self, shape: Shape, device="cuda"):
        import torch
        self.shape = shape
        self.device = device
        self.ws_bytes = workspace_bytes(shape)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=device)

    def __call__(self, h, w_router, w_gate, w_up, w_down, b_router=None, b_select=None,
                 sh_gate=None, sh_up=None, sh_down=None, stats=True, out=None, events=None):
        import torch
        s = self.shape
        y = out if out is not None else torch.empty_like(h)
        res = {"y": y}
        if stats:
            dev = h.device
            res.update(topk_ids=torch.empty((s.T, s.k), dtype=torch.int32, device=dev),
                       topk_gates=torch.empty((s.T, s.k), dtype=torch.float32, device=dev),
                       counts=torch.empty(s.N, dtype=torch.int32, device=dev),
                       f=torch.empty(s.N, dtype=torch.float32, device=dev),
                       p=torch.empty(s.N, dtype=torch.float32, device=dev),
                       l_aux=torch.empty(1, dtype=torch.float32, device=dev),
                       z_loss=torch.empty(1, dtype=torch.float32, device=dev),
                       entropy=torch.empty(1, dtype=torch.float32, device=dev),
                       cap_stats=torch.empty(2, dtype=torch.float32, device=dev))
        layer_fused(s, h, w_router, b_router, b_select, w_gate, w_up, w_down, sh_gate, sh_up,
                    sh_down, y, res.get("topk_ids"), res.get("topk_gates"), res.get("counts"),
                    res.get("f"), res.get("p"), res.get("l_aux"), self.ws, self.ws_bytes,
                    events=events, z_loss=res.get("z_loss"), entropy=res.get("entropy"),
                    cap_stats=res.get("cap_stats"))
        return res
