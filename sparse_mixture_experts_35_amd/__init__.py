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


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def workspace_bytes(shape: Shape) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(shape)))


def route(shape, h, w_router, b_router, b_select, topk_ids, topk_gates, p_mean, ws,
          ws_bytes, stream=None, z_loss=None, entropy=None):
    _check(lib().moe_route(ctypes.byref(shape), _ptr(h), _ptr(w_router), _ptr(b_router),
                           _ptr(b_select), _ptr(topk_ids), _ptr(topk_gates), _ptr(p_mean),
                           _ptr(z_loss), _ptr(entropy), _ptr(ws), ws_bytes, _stream(stream)),
           "moe_route")


def dispatch(shape, topk_ids, counts, offsets, perm_src, row_of, p_mean=None, f_out=None,
             l_aux=None, ws=None, ws_bytes=0, stream=None, cap_stats=None):
    _check(lib().moe_dispatch(ctypes.byref(shape), _ptr(topk_ids), _ptr(counts), _ptr(offsets),
                              _ptr(perm_src), _ptr(row_of), _ptr(p_mean), _ptr(f_out),
                              _ptr(l_aux), _ptr(cap_stats), _ptr(ws), ws_bytes, _stream(stream)),
           "moe_dispatch")


def expert_ffn(shape, h, perm_src, offsets, w_gate, w_up, w_down, sh_gate, sh_up, sh_down,
               out_rows, ws, ws_bytes, stream=None):
    _check(lib().moe_expert_ffn(ctypes.byref(shape), _ptr(h), _ptr(perm_src), _ptr(offsets),
                                _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(sh_gate),
                                _ptr(sh_up), _ptr(sh_down), _ptr(out_rows), _ptr(ws), ws_bytes,
                                _stream(stream)), "moe_expert_ffn")


def combine(shape, out_rows, row_of, topk_gates, y, stream=None):
    _check(lib().moe_combine(ctypes.byref(shape), _ptr(out_rows), _ptr(row_of),
                             _ptr(topk_gates), _ptr(y), _stream(stream)), "moe_combine")


def layer_fused(shape, h, w_router, b_router, b_select, w_gate, w_up, w_down, sh_gate, sh_up,
                sh_down, y, topk_ids=None, topk_gates=None, counts=None, f_out=None,
                p_out=None, l_aux=None, ws=None, ws_bytes=0, stream=None, events=None,
                z_loss=None, entropy=None, cap_stats=None):
    args = (ctypes.byref(shape), _ptr(h), _ptr(w_router), _ptr(b_router), _ptr(b_select),
            _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(sh_gate), _ptr(sh_up), _ptr(sh_down),
            _ptr(y), _ptr(topk_ids), _ptr(topk_gates), _ptr(counts), _ptr(f_out), _ptr(p_out),
            _ptr(l_aux), _ptr(z_loss), _ptr(entropy), _ptr(cap_stats), _ptr(ws), ws_bytes,
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
    _check(lib().moe_layer_fused_noalloc(
        ctypes.byref(shape), _ptr(h), _ptr(w_router), _ptr(b_router), _ptr(b_select),
        _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(sh_gate), _ptr(sh_up), _ptr(sh_down),
        _ptr(y), _ptr(topk_ids), _ptr(topk_gates), _ptr(counts), _ptr(f_out), _ptr(p_out),
        _ptr(l_aux), _ptr(z_loss), _ptr(entropy), _ptr(cap_stats), _stream(stream)),
        "moe_layer_fused_noalloc")


def layer_forward_train(shape, h, w_router, b_router, b_select, w_gate, w_up, w_down, sh_gate,
                        sh_up, sh_down, y, topk_ids, topk_gates, counts, offsets, perm_src,
                        row_of, preact=None, p_out=None, l_aux=None, z_loss=None, entropy=None,
                        ws=None, ws_bytes=0, stream=None):
    _check(lib().moe_layer_forward_train(
        ctypes.byref(shape), _ptr(h), _ptr(w_router), _ptr(b_router), _ptr(b_select),
        _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(sh_gate), _ptr(sh_up), _ptr(sh_down),
        _ptr(y), _ptr(topk_ids), _ptr(topk_gates), _ptr(counts), _ptr(offsets), _ptr(perm_src),
        _ptr(row_of), _ptr(preact), _ptr(p_out), _ptr(l_aux), _ptr(z_loss), _ptr(entropy),
        _ptr(ws), ws_bytes, _stream(stream)), "moe_layer_forward_train")


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
    _check(lib().moe_layer_backward(
        ctypes.byref(shape), _ptr(h), _ptr(w_router), _ptr(b_router), _ptr(w_gate), _ptr(w_up),
        _ptr(w_down), _ptr(sh_gate), _ptr(sh_up), _ptr(sh_down), _ptr(topk_ids),
        _ptr(topk_gates), _ptr(counts), _ptr(offsets), _ptr(perm_src), _ptr(row_of),
        _ptr(preact), _ptr(dy),
        float(d_laux), float(d_zloss), _ptr(dh), _ptr(dw_router), _ptr(db_router), _ptr(dw_gate),
        _ptr(dw_up), _ptr(dw_down), _ptr(dsh_gate), _ptr(dsh_up), _ptr(dsh_down), _ptr(dgates),
        _ptr(ws), ws_bytes, _stream(stream)), "moe_layer_backward")


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
