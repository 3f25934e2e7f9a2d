"""Seeded synthetic inputs for the sparse MoE FFN layer.

This module is shared by the tests, the benchmark and the oracle checks. It
holds only input generation (random draws, bf16 rounding of the draws, the
RMS normalisation of the hidden states, the skew bias recipe); it contains
none of the layer's arithmetic (no router, scoring, top-k, dispatch, expert
FFN or combine).

Workloads follow the shapes the pages discuss:
  * tiny fp32 layer (T=64, d=32, N=4, top-2 renorm; also top-1 full softmax);
  * Mixtral-8x7B-shaped layer (d=4096, 8 experts, top-2) at prefill (T=4096)
    and decode (T=16) batch sizes [page "拆解 MoE：单个 Token 如何经过专家层",
    router step; page "MOE 专家选择与路由机制", §十 model table];
  * Qwen3-30B-A3B-shaped fine-grained layer (128 experts, top-8) with skewed
    loads [page "MOE 专家选择与路由机制", §十 and §十二 load skew];
  * DeepSeek-V3-shaped layer (256 routed experts, top-8, one shared expert,
    sigmoid scoring with a selection bias) [page "拆解 MoE ...", router step
    and shared-expert paragraph; page "MoE：router 怎样选 expert", first
    section].

Seeds are per tensor and per expert: numpy draws use
``SeedSequence([cfg_id, tensor_id, expert])``; torch device draws use the
seed ``(cfg_id << 40) | (tensor_id << 20) | expert``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

# Gate modes, numbered as in include/moe.h.
MODE_SOFTMAX_RENORM = 0       # top-k, then renormalise over the selected
MODE_SOFTMAX_FULL = 1         # keep the full-softmax probability (Switch)
MODE_SIGMOID_BIAS_RENORM = 2  # select on sigmoid + bias, renorm unbiased

DTYPE_F32 = 0
DTYPE_BF16 = 1

# tensor ids used in the seeds
TID_H, TID_WR, TID_BR, TID_BSEL, TID_WG, TID_WU, TID_WD = 1, 2, 3, 4, 5, 6, 7
TID_SG, TID_SU, TID_SD, TID_PERM = 8, 9, 10, 11


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    T: int
    d: int
    N: int
    k: int
    d_ff: int
    d_ff_shared: int = 0
    dtype: int = DTYPE_BF16
    mode: int = MODE_SOFTMAX_RENORM
    aux_alpha: float = 0.01
    h_normalised: bool = True        # x ~ N(0,1), h = x / rms(x) / sqrt(d)
    router_std: Optional[float] = 0.02   # None: 1/sqrt(d)
    expert_std: Optional[float] = 0.02   # None: 1/sqrt(fan_in)
    router_bias: str = "none"        # "none" | "zipf"
    zipf_s: float = 1.1
    select_bias: float = 0.0         # b_sel ~ U(-a, a) when mode C
    capacity_factor: float = 0.0     # 0: dropless; else C = ceil(cf * T * k / N)
    groups: Optional[tuple] = None   # (n_groups, topk_groups, group_topm) or None

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def rows(self) -> int:
        return self.T * self.k + (self.T if self.d_ff_shared else 0)

    def flops(self) -> float:
        """Algorithmic expert FLOPs: 6*d*d_ff per (token, selected expert)
        plus 6*d*d_ff_shared per token. Padding never counts."""
        f = 6.0 * self.d * self.d_ff * self.T * self.k
        if self.d_ff_shared:
            f += 6.0 * self.d * self.d_ff_shared * self.T
        return f


TINY = Workload("tiny_fp32_T64_d32_N4_top2", 1, T=64, d=32, N=4, k=2, d_ff=64,
                dtype=DTYPE_F32, h_normalised=False, router_std=None,
                expert_std=None)
TINY_SWITCH = TINY.replace(name="tiny_fp32_T64_d32_N4_top1_switch", k=1,
                           mode=MODE_SOFTMAX_FULL)
MIXTRAL_PREFILL = Workload("mixtral_8x7b_prefill_T4096", 2, T=4096, d=4096,
                           N=8, k=2, d_ff=14336)
MIXTRAL_PREFILL_R1 = MIXTRAL_PREFILL.replace(
    name="mixtral_8x7b_prefill_T4096_router_std1", router_std=1.0)
MIXTRAL_DECODE = MIXTRAL_PREFILL.replace(name="mixtral_8x7b_decode_T16",
                                         cfg_id=3, T=16)
QWEN3_30B = Workload("qwen3_30b_a3b_T8192_zipf", 4, T=8192, d=2048, N=128,
                     k=8, d_ff=768, router_std=1.0, router_bias="zipf")
DEEPSEEK_V3 = Workload("deepseek_v3_T4096_shared", 5, T=4096, d=7168, N=256,
                       k=8, d_ff=2048, d_ff_shared=2048,
                       mode=MODE_SIGMOID_BIAS_RENORM, router_std=1.0,
                       select_bias=0.1)

# the skewed fine-grained layer with an expert capacity: the popular experts
# overflow and drop their latest tokens (same inputs as the dropless one)
QWEN3_30B_CAP = QWEN3_30B.replace(name="qwen3_30b_a3b_T8192_zipf_cap1.25",
                                  capacity_factor=1.25)

# the DeepSeek-V3-shaped layer with group-limited selection: 8 groups of 32
# experts, the 4 best by the sum of their top-2 scores stay candidates
DEEPSEEK_V3_GROUPED = DEEPSEEK_V3.replace(name="deepseek_v3_T4096_shared_groups8_keep4",
                                          groups=(8, 4, 2))

ALL = {w.name: w for w in (TINY, TINY_SWITCH, MIXTRAL_PREFILL,
                           MIXTRAL_PREFILL_R1, MIXTRAL_DECODE, QWEN3_30B,
                           QWEN3_30B_CAP, DEEPSEEK_V3, DEEPSEEK_V3_GROUPED)}


# --------------------------------------------------------------- host draws
def _rng(cfg_id: int, tid: int, expert: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg_id, tid, expert]))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns the
    rounded values as fp32 (exactly representable in bf16)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
         & np.uint32(0xFFFF0000))
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of values already representable in bf16."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
            >> np.uint32(16)).astype(np.uint16)


def _hidden(w: Workload, rng: np.random.Generator) -> np.ndarray:
    x = rng.standard_normal((w.T, w.d), dtype=np.float32)
    if w.h_normalised and w.T:
        # input recipe: RMS-normalise each row, then scale by 1/sqrt(d) so
        # that every row has unit Euclidean norm
        rms = np.sqrt(np.mean(x.astype(np.float64) ** 2, axis=1, keepdims=True))
        x = (x / rms / math.sqrt(w.d)).astype(np.float32)
    return x


def zipf_router_bias(w: Workload) -> np.ndarray:
    """b_r[i] = ln(w_pi(i)), w_j proportional to j^-s, pi a seeded
    permutation: skews expert popularity along a Zipf law."""
    j = np.arange(1, w.N + 1, dtype=np.float64)
    wj = j ** (-w.zipf_s)
    wj /= wj.sum()
    perm = _rng(w.cfg_id, TID_PERM).permutation(w.N)
    return np.log(wj[perm]).astype(np.float32)


def host_inputs(w: Workload, with_weights: bool = True) -> dict:
    """All inputs of workload ``w`` drawn on the host (numpy).

    Values are fp32 arrays; for bf16 workloads every activation and weight is
    rounded to bf16 so the same numbers can be handed to the GPU. Biases stay
    fp32. Keys: h, w_router, b_router, b_select, w_gate, w_up, w_down,
    sh_gate, sh_up, sh_down (None where absent).
    """
    rnd = round_to_bf16 if w.dtype == DTYPE_BF16 else (lambda a: a)
    rstd = w.router_std if w.router_std is not None else 1.0 / math.sqrt(w.d)
    out = {"h": rnd(_hidden(w, _rng(w.cfg_id, TID_H))),
           "w_router": rnd(_rng(w.cfg_id, TID_WR).standard_normal(
               (w.N, w.d), dtype=np.float32) * np.float32(rstd)),
           "b_router": zipf_router_bias(w) if w.router_bias == "zipf" else None,
           "b_select": None}
    if w.mode == MODE_SIGMOID_BIAS_RENORM:
        a = w.select_bias
        out["b_select"] = _rng(w.cfg_id, TID_BSEL).uniform(
            -a, a, size=w.N).astype(np.float32)
    for key in ("w_gate", "w_up", "w_down", "sh_gate", "sh_up", "sh_down"):
        out[key] = None
    if not with_weights:
        return out

    def expert_std(fan_in):
        return w.expert_std if w.expert_std is not None else 1.0 / math.sqrt(fan_in)

    def draw(tid, e, shape, fan_in):
        return rnd(_rng(w.cfg_id, tid, e).standard_normal(shape, dtype=np.float32)
                   * np.float32(expert_std(fan_in)))

    out["w_gate"] = np.stack([draw(TID_WG, e, (w.d_ff, w.d), w.d) for e in range(w.N)])
    out["w_up"] = np.stack([draw(TID_WU, e, (w.d_ff, w.d), w.d) for e in range(w.N)])
    out["w_down"] = np.stack([draw(TID_WD, e, (w.d, w.d_ff), w.d_ff) for e in range(w.N)])
    if w.d_ff_shared:
        out["sh_gate"] = draw(TID_SG, 0, (w.d_ff_shared, w.d), w.d)
        out["sh_up"] = draw(TID_SU, 0, (w.d_ff_shared, w.d), w.d)
        out["sh_down"] = draw(TID_SD, 0, (w.d, w.d_ff_shared), w.d_ff_shared)
    return out


# ------------------------------------------------------------- device draws
def device_seed(cfg_id: int, tid: int, expert: int = 0) -> int:
    return (cfg_id << 40) | (tid << 20) | expert


def device_inputs(w: Workload, device="cuda", with_weights: bool = True) -> dict:
    """Inputs of workload ``w`` drawn on the GPU with torch's generator
    (for the full-size workloads). Returns torch tensors in the workload's
    dtype (biases fp32). The oracle reads them back with ``.cpu()``.
    with_weights=False: the routing inputs only (h, w_router, the biases),
    the same values; the expert weights are None."""
    import torch

    tdt = torch.bfloat16 if w.dtype == DTYPE_BF16 else torch.float32
    g = torch.Generator(device=device)

    def randn(shape, tid, e, std):
        g.manual_seed(device_seed(w.cfg_id, tid, e))
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        return (x * std).to(tdt)

    g.manual_seed(device_seed(w.cfg_id, TID_H, 0))
    x = torch.randn((w.T, w.d), generator=g, device=device, dtype=torch.float32)
    if w.h_normalised and w.T:
        rms = x.double().pow(2).mean(dim=1, keepdim=True).sqrt().float()
        x = x / rms / math.sqrt(w.d)
    rstd = w.router_std if w.router_std is not None else 1.0 / math.sqrt(w.d)
    out = {"h": x.to(tdt), "w_router": randn((w.N, w.d), TID_WR, 0, rstd),
           "b_router": None, "b_select": None}
    if w.router_bias == "zipf":
        out["b_router"] = torch.from_numpy(zipf_router_bias(w)).to(device)
    if w.mode == MODE_SIGMOID_BIAS_RENORM:
        g.manual_seed(device_seed(w.cfg_id, TID_BSEL, 0))
        a = w.select_bias
        out["b_select"] = (torch.rand((w.N,), generator=g, device=device) * 2 * a - a).float()

    def estd(fan_in):
        return w.expert_std if w.expert_std is not None else 1.0 / math.sqrt(fan_in)

    if not with_weights:
        for key in ("w_gate", "w_up", "w_down", "sh_gate", "sh_up", "sh_down"):
            out[key] = None
        return out

    def stack(tid, shape, fan_in):
        t = torch.empty((w.N,) + shape, device=device, dtype=tdt)
        for e in range(w.N):
            t[e] = randn(shape, tid, e, estd(fan_in))
        return t

    out["w_gate"] = stack(TID_WG, (w.d_ff, w.d), w.d)
    out["w_up"] = stack(TID_WU, (w.d_ff, w.d), w.d)
    out["w_down"] = stack(TID_WD, (w.d, w.d_ff), w.d_ff)
    out["sh_gate"] = out["sh_up"] = out["sh_down"] = None
    if w.d_ff_shared:
        out["sh_gate"] = randn((w.d_ff_shared, w.d), TID_SG, 0, estd(w.d))
        out["sh_up"] = randn((w.d_ff_shared, w.d), TID_SU, 0, estd(w.d))
        out["sh_down"] = randn((w.d, w.d_ff_shared), TID_SD, 0, estd(w.d_ff_shared))
    return out


def random_small(T, d, N, k, d_ff, d_ff_shared=0, dtype=DTYPE_F32,
                 mode=MODE_SOFTMAX_RENORM, seed=0, router_std=1.0,
                 select_bias=0.1, router_bias=False) -> dict:
    """Small random inputs for parity cases of arbitrary shape (host).

    Rows of h have norm about 1, so with unit-std gate/up weights the gate
    pre-activations are about N(0,1) and SiLU works in its curved range."""
    rng = np.random.default_rng(np.random.SeedSequence([99, seed, T, d, N, k, d_ff]))
    rnd = round_to_bf16 if dtype == DTYPE_BF16 else (lambda a: a.astype(np.float32))

    def nrm(shape, std):
        return rnd((rng.standard_normal(shape) * std).astype(np.float32))

    out = {"h": nrm((T, d), 1.0 / math.sqrt(d)),
           "w_router": nrm((N, d), router_std),
           "b_router": (rng.standard_normal(N).astype(np.float32) if router_bias else None),
           "b_select": (rng.uniform(-select_bias, select_bias, N).astype(np.float32)
                        if mode == MODE_SIGMOID_BIAS_RENORM else None),
           "w_gate": nrm((N, d_ff, d), 1.0),
           "w_up": nrm((N, d_ff, d), 1.0),
           "w_down": nrm((N, d, d_ff), 1.0 / math.sqrt(d_ff)),
           "sh_gate": None, "sh_up": None, "sh_down": None}
    if d_ff_shared:
        out["sh_gate"] = nrm((d_ff_shared, d), 1.0)
        out["sh_up"] = nrm((d_ff_shared, d), 1.0)
        out["sh_down"] = nrm((d, d_ff_shared), 1.0 / math.sqrt(d_ff_shared))
    return out
