"""Benchmark of the MoE layer forward pass on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --copy-calibration    # plain 1 GiB copy, for counter scaling

A step is one moe_layer_fused call (route, dispatch, gate/up GEMM + SwiGLU,
down GEMM, combine, load statistics) over one batch of synthetic tokens whose
inputs are already resident in HBM. Prints ONE JSON line.

  value     whole-layer tokens/s (T * K / wall time of the K timed steps
            between two device synchronisations)
  roofline  the dominant kernel (the grouped gate/up GEMM), timed with HIP
            events that the library records on its own stream around that
            stage in each of the K timed steps, against the MI355X peak that
            bounds it: bf16 dense MFMA 2.5166 PFLOP/s when its rows per
            expert make it compute-bound, HBM 8 TB/s when it streams weights
            (decode batches). traffic: HBM bytes per launch from rocprofv3
            FETCH_SIZE / WRITE_SIZE counters scaled by a plain copy's
            readings (a committed summary under profiles/), reported only
            while the kernel sources match the ones that were counted
  decode    the same layer at a decode batch (16 tokens) on the same
            weights: tokens/s and HBM GB/s of the touched experts' weights;
            other_batches: ms per step and HBM fraction at 1, 4, 32 and 64
            tokens
  backward  moe_layer_backward on the same workload (the forward's selection
            made once beforehand): ms per call and the algorithmic TFLOP/s of
            the gradients (2x the forward's expert flops plus the router's);
            train_step: moe_layer_forward_train (keeping the pre-activations)
            then the backward that uses them, per step
  variants  the fine-grained skewed layer (128 experts, top-8) dropless and
            with expert capacity 1.25 (capacity usage, dropped fraction),
            and the DeepSeek-V3-shaped layer without and with group-limited
            selection: tokens/s, stage times, gate/up MFMA rate over the rows
            computed, router z-loss and routing entropy
  cpu_baseline  the float64 oracle on a bounded sample of the workload,
            timed on this host's cores (a reported baseline, not a target)
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "MoE-layer tokens/sec at 1 MI355X; % bf16 MFMA peak (prefill), % HBM BW (decode)"
PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
GEMM_SOURCES = ("gemm_bf16.hip", "common.hpp")
VARIANTS = (W.QWEN3_30B, W.QWEN3_30B_CAP, W.DEEPSEEK_V3, W.DEEPSEEK_V3_GROUPED)


def gemm_source_hash():
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(ROOT, "sparse_mixture_experts_35_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    counter summary, or None when there is none or the kernel sources have
    changed since the counters were taken."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                key, val = line.split(":", 1)
                kv[key.strip()] = val.strip()
    if kv.get("gemm_source_sha256_16") != gemm_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def library_gemm(torch, w, steps=10, warmup=3, seconds=0.0):
    """Context only: the vendor library (hipBLASLt through torch.bmm) on the
    uniform-batch equivalent of the gate/up GEMM of the workload, N
    experts x [T k / N rows, d] x [d, 2 d_ff], bf16. Prints one JSON line.
    seconds > 0: back to back for that long instead (power sampling)."""
    rows = w.T * w.k // w.N
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    a = torch.randn(w.N, rows, w.d, generator=g, device="cuda").to(torch.bfloat16)
    b = torch.randn(w.N, w.d, 2 * w.d_ff, generator=g, device="cuda").to(torch.bfloat16)
    c = torch.empty(w.N, rows, 2 * w.d_ff, device="cuda", dtype=torch.bfloat16)
    for _ in range(warmup):
        torch.bmm(a, b, out=c)
    if seconds > 0:
        torch.cuda.synchronize()
        t0, n = time.time(), 0
        print(json.dumps({"sustain_start_unix": t0}), flush=True)
        while time.time() - t0 < seconds:
            for _ in range(20):
                torch.bmm(a, b, out=c)
            torch.cuda.synchronize()
            n += 20
        dt = time.time() - t0
        fl = 2.0 * w.N * rows * w.d * 2 * w.d_ff
        print(json.dumps({"library_gemm": "torch.bmm (hipBLASLt)", "sustain_s": dt, "steps": n,
                          "ms": dt / n * 1e3, "tflops": fl / (dt / n) / 1e12,
                          "sustain_end_unix": time.time()}), flush=True)
        return
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(steps):
        torch.bmm(a, b, out=c)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    fl = 2.0 * w.N * rows * w.d * 2 * w.d_ff
    tf = fl / (ms * 1e-3) / 1e12
    print(json.dumps({"library_gemm": "torch.bmm (hipBLASLt)", "workload": w.name,
                      "shape": [w.N, rows, w.d, 2 * w.d_ff], "ms": ms, "tflops": tf,
                      "frac_mfma_peak": tf / PEAK_BF16_TFLOPS}), flush=True)


def copy_calibration(torch, gib=1, reps=5):
    """A plain device copy of a known size: its FETCH_SIZE / WRITE_SIZE
    readings per dispatch give the bytes-per-count scale of the counters."""
    n = gib << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "reps": reps,
                      "ms_per_copy": dt * 1e3, "gb_s": 2 * n / dt / 1e9}), flush=True)


def hip_events(n):
    """Create n hipEvent_t handles through the HIP runtime (the library
    records them on its own stream)."""
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    evs = []
    for _ in range(n):
        e = ctypes.c_void_p()
        if hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        evs.append(e.value)

    def elapsed(a, b):
        ms = ctypes.c_float()
        if hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy():
        for e in evs:
            hip.hipEventDestroy(e)
    return evs, elapsed, destroy


def run_layer(M, torch, w, inp, steps, warmup, gate_up_events=True, alt_weights=None):
    """warmup untimed steps, then `steps` timed steps. In the timed steps the
    library records HIP events on its stream only around the gate/up GEMM
    (gate_up_events; none otherwise): each event record costs the stream a
    few microseconds. A further `steps` untimed steps record all six stage
    boundaries for the stage breakdown. alt_weights: a second copy of the
    expert weights (w_gate, w_up, w_down) that every other step uses, so
    that no step finds its weights in the 256 MB Infinity Cache."""
    g = w.groups or (0, 0, 0)
    s = M.Shape(w.T, w.d, w.N, w.k, w.d_ff, w.d_ff_shared, w.dtype, w.mode, w.aux_alpha, *g,
                capacity_factor=w.capacity_factor)
    layer = M.MoELayer(s)
    args = dict(b_router=inp["b_router"], b_select=inp["b_select"], sh_gate=inp["sh_gate"],
                sh_up=inp["sh_up"], sh_down=inp["sh_down"])
    y = torch.empty_like(inp["h"])
    res = None

    sets = [(inp["w_gate"], inp["w_up"], inp["w_down"])]
    if alt_weights is not None:
        sets.append(alt_weights)
    step_no = [0]

    def call(events=None):
        wg, wu, wd = sets[step_no[0] % len(sets)]
        step_no[0] += 1
        return layer(inp["h"], inp["w_router"], wg, wu, wd, out=y, events=events, **args)

    for _ in range(warmup):
        res = call()
    evs, elapsed, destroy = hip_events(6 * steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        e = evs[6 * i:6 * i + 6]
        res = call([None, None, e[2], e[3], None, None] if gate_up_events else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gate_up_timed = (sum(elapsed(evs[6 * i + 2], evs[6 * i + 3]) for i in range(steps)) / steps
                     if gate_up_events else None)
    # stage breakdown (untimed)
    for i in range(steps):
        call(evs[6 * i:6 * i + 6])
    torch.cuda.synchronize()
    names = ["route", "dispatch", "gate_up", "down", "combine"]
    stage = {n: 0.0 for n in names}
    total = 0.0
    for i in range(steps):
        e = evs[6 * i:6 * i + 6]
        for j, n in enumerate(names):
            stage[n] += elapsed(e[j], e[j + 1]) / steps
        total += elapsed(e[0], e[5]) / steps
    destroy()
    counts = res["counts"].cpu().numpy()
    run_layer.last = {k_: v.cpu().numpy() for k_, v in res.items()
                      if k_ in ("cap_stats", "z_loss", "entropy", "l_aux")}
    run_layer.gate_up_timed = gate_up_timed
    return wall, stage, total, counts


def gateup_work(w, counts):
    """Algorithmic work of the gate/up stage: flops 4*d*d_ff per routed row
    (+ 4*d*d_ff_shared per token); bytes: weights of the touched experts
    once, the gathered token rows, the SwiGLU output."""
    rows = int(counts.sum())
    flops = 4.0 * w.d * w.d_ff * rows + 4.0 * w.d * w.d_ff_shared * w.T
    touched = int((counts > 0).sum())
    eb = 2 if w.dtype == W.DTYPE_BF16 else 4
    wbytes = (touched * 2 * w.d_ff * w.d + (2 * w.d_ff_shared * w.d if w.d_ff_shared else 0)) * eb
    act_bytes = (rows * w.d + rows * w.d_ff + (w.T * (w.d + w.d_ff_shared) if w.d_ff_shared else 0)) * eb
    return flops, wbytes + act_bytes, touched


def layer_work(w, counts):
    rows = int(counts.sum())
    flops = 6.0 * w.d * w.d_ff * rows + 6.0 * w.d * w.d_ff_shared * w.T
    touched = int((counts > 0).sum())
    eb = 2 if w.dtype == W.DTYPE_BF16 else 4
    wbytes = (touched * 3 * w.d_ff * w.d + 3 * w.d_ff_shared * w.d) * eb
    return flops, wbytes, touched



def stage_work(w, counts):
    """Algorithmic work of each GEMM stage and of the layer: flops (padding
    rows never count) and bytes (each touched expert's weights once, the
    activations each stage reads and writes, the Act and out_rows round
    trips). counts: the rows each expert computes."""
    rows = int(counts.sum())
    touched = int((counts > 0).sum())
    eb = 2 if w.dtype == W.DTYPE_BF16 else 4
    d, f, fs, T = w.d, w.d_ff, w.d_ff_shared, w.T
    gu_fl = 4.0 * d * f * rows + 4.0 * d * fs * T
    dn_fl = 2.0 * d * f * rows + 2.0 * d * fs * T
    gu_b = (touched * 2 * f * d + 2 * fs * d + rows * (d + f) + (T * (d + fs) if fs else 0)) * eb
    dn_b = (touched * f * d + fs * d + rows * (f + d) + (T * (fs + d) if fs else 0)) * eb
    route_b = (T * d + w.N * d) * eb
    combine_b = (rows + (T if fs else 0) + T) * d * eb
    return {"gate_up": (gu_fl, gu_b), "down": (dn_fl, dn_b),
            "layer": (gu_fl + dn_fl, gu_b + dn_b + route_b + combine_b)}


def fractions(flops, nbytes, ms):
    """Achieved rates of algorithmic work over a duration, as fractions of
    both MI355X peaks (bf16 dense MFMA and HBM)."""
    s = ms * 1e-3
    tf, gbs = flops / s / 1e12, nbytes / s / 1e9
    return {"ms": ms, "tflops": tf, "frac_mfma_peak": tf / PEAK_BF16_TFLOPS,
            "gbs": gbs, "frac_hbm_peak": gbs / PEAK_HBM_GBS,
            "algorithmic_flops": flops, "algorithmic_bytes": nbytes}


def kept_counts(w, counts):
    """Rows each expert computes: all routed slots, or at most C of them."""
    if not w.capacity_factor:
        return counts
    C = math.ceil(float(np.float32(w.capacity_factor)) * (w.T * w.k) / w.N)
    return np.minimum(counts, C)


def run_variant(M, torch, w, steps, warmup):
    """One workload of the variant list: whole-layer throughput, stage times
    and the gate/up GEMM's MFMA rate over the rows it computes."""
    inp = W.device_inputs(w)
    torch.cuda.synchronize()
    wall, stage, _, counts = run_layer(M, torch, w, inp, steps, warmup)
    extra = run_layer.last
    kept = kept_counts(w, counts)
    flops_gu, _, touched = gateup_work(w, kept)
    gu = flops_gu / (run_layer.gate_up_timed * 1e-3) / 1e12
    sw = stage_work(w, kept)
    out = {"workload": w.name, "tokens_per_s": w.T * steps / wall,
           "ms_per_step": wall / steps * 1e3, "stages_ms": stage,
           "layer": fractions(*sw["layer"], wall / steps * 1e3),
           "kernels": {"gate_up": fractions(*sw["gate_up"], run_layer.gate_up_timed),
                       "down": fractions(*sw["down"], stage["down"])},
           "gate_up_tflops": gu, "gate_up_frac_mfma_peak": gu / PEAK_BF16_TFLOPS,
           "rows_computed": int(kept.sum()), "experts_touched": touched,
           "z_loss": float(extra["z_loss"][0]), "entropy": float(extra["entropy"][0])}
    if w.capacity_factor:
        out.update(capacity_factor=w.capacity_factor, capacity_usage=float(extra["cap_stats"][0]),
                   dropped_fraction=float(extra["cap_stats"][1]))
    if w.groups:
        out["groups"] = {"n_groups": w.groups[0], "topk_groups": w.groups[1],
                         "group_topm": w.groups[2]}
    del inp
    torch.cuda.empty_cache()
    return out


def run_backward(M, torch, w, inp, steps, warmup):
    """moe_layer_backward on the workload: the forward's selection and
    dispatch are made once (moe_route, moe_dispatch) before the clock
    starts; each timed step is one backward call (recomputing the router
    logits and gate/up pre-activations) with a fixed upstream gradient and
    both auxiliary-loss weights set. Timed with events on the stream the
    library launches on."""
    g = w.groups or (0, 0, 0)
    s = M.Shape(w.T, w.d, w.N, w.k, w.d_ff, w.d_ff_shared, w.dtype, w.mode, w.aux_alpha, *g,
                capacity_factor=w.capacity_factor)
    T, d, N, k, dff, dfs = w.T, w.d, w.N, w.k, w.d_ff, w.d_ff_shared
    dev = inp["h"].device
    E = lambda shp, dt=inp["h"].dtype: torch.empty(shp, dtype=dt, device=dev)
    nws = M.workspace_bytes(s)
    ws = E(nws, torch.uint8)
    ids, gates = E(T * k, torch.int32), E(T * k, torch.float32)
    M.route(s, inp["h"], inp["w_router"], inp["b_router"], inp["b_select"], ids, gates, None, ws,
            nws)
    counts, offsets = E(N, torch.int32), E(N + 1, torch.int32)
    perm, row_of = E(T * k, torch.int32), E(T * k, torch.int32)
    M.dispatch(s, ids, counts, offsets, perm, row_of, ws=ws, ws_bytes=nws)
    del ws
    gen = torch.Generator(device=dev)
    gen.manual_seed(12345)
    dy = torch.randn((T, d), generator=gen, device=dev).to(inp["h"].dtype)
    out = dict(dh=E((T, d)), dw_router=E((N, d), torch.float32), db_router=E(N, torch.float32),
               dw_gate=E((N, dff, d)), dw_up=E((N, dff, d)), dw_down=E((N, d, dff)),
               dgates=E(T * k, torch.float32))
    if dfs:
        out.update(dsh_gate=E((dfs, d)), dsh_up=E((dfs, d)), dsh_down=E((d, dfs)))
    nb = M.backward_workspace_bytes(s)
    bws = E(nb, torch.uint8)

    def step():
        M.layer_backward(s, inp["h"], inp["w_router"], inp["b_router"], inp["w_gate"],
                         inp["w_up"], inp["w_down"], inp["sh_gate"], inp["sh_up"], inp["sh_down"],
                         ids, gates, counts, offsets, perm, row_of, dy, out["dh"],
                         out["dw_router"], out["db_router"], out["dw_gate"], out["dw_up"],
                         out["dw_down"], out.get("dsh_gate"), out.get("dsh_up"),
                         out.get("dsh_down"), out["dgates"], 1.0, 1e-3, bws, nb)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(steps):
        step()
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_ev = a.elapsed_time(b) / steps
    # training step: the training forward keeps the dispatch and the gate/up
    # pre-activations, the backward uses them (no recompute)
    pre = E(M.preact_floats(s), torch.float32)
    nws = M.workspace_bytes(s)
    fws = E(nws, torch.uint8)
    y = E((T, d))
    ids_t, gates_t, counts_t = E(T * k, torch.int32), E(T * k, torch.float32), E(N, torch.int32)
    off_t, perm_t, row_t = E(N + 1, torch.int32), E(T * k, torch.int32), E(T * k, torch.int32)

    def train_step(evs=None):
        if evs:
            evs[0].record()
        M.layer_forward_train(s, inp["h"], inp["w_router"], inp["b_router"], inp["b_select"],
                              inp["w_gate"], inp["w_up"], inp["w_down"], inp["sh_gate"],
                              inp["sh_up"], inp["sh_down"], y, ids_t, gates_t, counts_t, off_t,
                              perm_t, row_t, preact=pre, ws=fws, ws_bytes=nws)
        if evs:
            evs[1].record()
        M.layer_backward(s, inp["h"], inp["w_router"], inp["b_router"], inp["w_gate"],
                         inp["w_up"], inp["w_down"], inp["sh_gate"], inp["sh_up"],
                         inp["sh_down"], ids_t, gates_t, counts_t, off_t, perm_t, row_t, dy,
                         out["dh"], out["dw_router"], out["db_router"], out["dw_gate"],
                         out["dw_up"], out["dw_down"], out.get("dsh_gate"), out.get("dsh_up"),
                         out.get("dsh_down"), out["dgates"], 1.0, 1e-3, bws, nb, preact=pre)
        if evs:
            evs[2].record()

    for _ in range(warmup):
        train_step()
    torch.cuda.synchronize()
    tev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t1 = time.perf_counter()
    for i in range(steps):
        train_step(tev[i])
    torch.cuda.synchronize()
    twall = time.perf_counter() - t1
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in tev) / steps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in tev) / steps
    del fws, pre
    c = counts.cpu().numpy()
    rows = int(np.minimum(c, kept_counts(w, c)).sum())
    # algorithmic flops: dh rows (4 d d_ff) + v (2 d d_ff) + dW_gate/up (4 d d_ff) + dW_down
    # (2 d d_ff) per kept row, the same for the shared expert per token, and the router's
    # dz W_r and dz^T h (4 d N per token); the recompute of the pre-activations is not counted
    flops = 12.0 * d * dff * rows + 12.0 * d * dfs * T + 4.0 * d * N * T
    tf = flops / (ms_ev * 1e-3) / 1e12
    res = {"workload": w.name, "ms_per_step": wall / steps * 1e3, "events_ms": ms_ev,
           "tokens_per_s": T * steps / wall, "algorithmic_tflop": flops / 1e12,
           "tflops": tf, "frac_mfma_peak": tf / PEAK_BF16_TFLOPS,
           "workspace_gb": nb / 1e9,
           "train_step": {"ms_per_step": twall / steps * 1e3,
                          "tokens_per_s": T * steps / twall,
                          "forward_train_ms": fwd_ms, "backward_with_preact_ms": bwd_ms,
                          "backward_tflops": flops / (bwd_ms * 1e-3) / 1e12}}
    del bws, out
    torch.cuda.empty_cache()
    return res

def cpu_baseline(w, inp, sample_tokens, min_seconds=10.0, max_reps=5):
    """The float64 oracle on the first `sample_tokens` tokens (routing,
    their experts, combine, statistics), timed on the host and repeated
    until at least `min_seconds` have passed; inputs are copied to host
    memory before the clock starts."""
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    S = min(sample_tokens, w.T)
    h = inp["h"][:S].float().cpu().numpy()
    wr = inp["w_router"].float().cpu().numpy()
    br = None if inp["b_router"] is None else inp["b_router"].cpu().numpy()
    bs = None if inp["b_select"] is None else inp["b_select"].cpu().numpy()
    r0 = O.route(h, wr, w.k, w.mode, br, bs)
    need = sorted(set(r0.ids.reshape(-1).tolist()))
    host_w = {e: (inp["w_gate"][e].float().cpu().numpy(), inp["w_up"][e].float().cpu().numpy(),
                  inp["w_down"][e].float().cpu().numpy()) for e in need}
    sh = None
    if inp["sh_gate"] is not None:
        sh = tuple(inp[k_].float().cpu().numpy() for k_ in ("sh_gate", "sh_up", "sh_down"))
    reps = 0
    t0 = time.perf_counter()
    while True:
        r = O.route(h, wr, w.k, w.mode, br, bs)
        d = O.dispatch(r.ids, w.N)
        rows = O.expert_rows(h, d, w.k, lambda e: host_w[e], sh)
        O.combine(rows, d.row_of, r.gates, sh is not None)
        O.load_stats(d.counts, r.stat_prob, w.k, w.aux_alpha)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or reps >= max_reps:
            break
    what = "all" if S == w.T else f"the first {S} of"
    return {"value": S * reps / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{what} {w.T} tokens of {w.name} (route, dispatch, their {len(need)} "
                      f"experts, combine, stats) in float64 numpy, {reps} pass(es) in {dt:.1f} s"}


def run_tiny(M, torch, steps=200, warmup=20):
    """The tiny fp32 configuration (both of its routing modes) on the GPU:
    latency per fused step, host-drawn inputs moved to the device first."""
    res = []
    for w in (W.TINY, W.TINY_SWITCH):
        host = W.host_inputs(w)
        inp = {k_: (None if v is None else torch.from_numpy(v).cuda()) for k_, v in host.items()}
        torch.cuda.synchronize()
        wall, stage, _, counts = run_layer(M, torch, w, inp, steps, warmup, gate_up_events=False)
        ms = wall / steps * 1e3
        res.append({"workload": w.name, "ms_per_step": ms, "tokens_per_s": w.T * steps / wall,
                    "layer": fractions(*stage_work(w, counts)["layer"], ms)})
    return res


def host_info():
    """CPU model, logical CPUs, CPUs this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return {"cpu_model": model, "nproc": os.cpu_count() or 1, "usable_cpus": usable}


def cpu_extras(torch, w, inp, decode_tokens, variants):
    """The rest of the CPU-baseline leg: the oracle on the tiny fp32
    configuration with one BLAS thread and with all of them, and the
    oracle's near-tie count (k-th minus (k+1)-th selection score below 1e-4,
    the tokens whose expert set may legitimately differ from the GPU's) for
    every configuration this run measured."""
    from oracle import moe_oracle as O
    from threadpoolctl import threadpool_limits

    def oracle_layer_rate(wt, host, seconds=2.0):
        sh = None if host["sh_gate"] is None else (host["sh_gate"], host["sh_up"], host["sh_down"])
        reps, t0 = 0, time.perf_counter()
        while True:
            O.layer(host["h"], host["w_router"], wt.k, wt.mode,
                    O.weights_getter(host["w_gate"], host["w_up"], host["w_down"]),
                    host["b_router"], host["b_select"], sh, wt.aux_alpha)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= seconds:
                return wt.T * reps / dt

    tiny = []
    for wt in (W.TINY, W.TINY_SWITCH):
        host = W.host_inputs(wt)
        with threadpool_limits(limits=1):
            one = oracle_layer_rate(wt, host)
        tiny.append({"workload": wt.name, "tokens_per_s_1_thread": one,
                     "tokens_per_s_all_threads": oracle_layer_rate(wt, host)})

    def near(wt, h, wr, br, bs):
        r = O.route(h, wr, wt.k, wt.mode, br, bs, wt.groups)
        return {"tokens": int(h.shape[0]), "near_tie": int(O.near_tie_tokens(r.gap).sum())}

    f64 = lambda t: None if t is None else t.float().cpu().numpy().astype(np.float64)
    ties = {}
    hw = f64(inp["h"])
    args = (f64(inp["w_router"]), f64(inp["b_router"]), f64(inp["b_select"]))
    ties[w.name] = near(w, hw, *args)
    if decode_tokens and decode_tokens < w.T:
        ties[f"{w.name} (first {decode_tokens} tokens, decode)"] = near(w, hw[:decode_tokens], *args)
    for v in variants:
        vi = W.device_inputs(v, with_weights=False)
        ties[v.name] = near(v, f64(vi["h"]), f64(vi["w_router"]), f64(vi["b_router"]),
                            f64(vi["b_select"]))
        del vi
    for wt in (W.TINY, W.TINY_SWITCH):
        host = W.host_inputs(wt, with_weights=False)
        ties[wt.name] = near(wt, host["h"], host["w_router"], host["b_router"], host["b_select"])
    return {"tiny_fp32": tiny, "near_tie_tokens": ties}


def sustain(M, torch, w, inp, seconds):
    """The fused step back to back for `seconds` (for sampling board power
    and clocks from outside, e.g. amd-smi): prints one JSON line."""
    g = w.groups or (0, 0, 0)
    s = M.Shape(w.T, w.d, w.N, w.k, w.d_ff, w.d_ff_shared, w.dtype, w.mode, w.aux_alpha, *g,
                capacity_factor=w.capacity_factor)
    layer = M.MoELayer(s)
    y = torch.empty_like(inp["h"])
    args = dict(b_router=inp["b_router"], b_select=inp["b_select"], sh_gate=inp["sh_gate"],
                sh_up=inp["sh_up"], sh_down=inp["sh_down"])
    for _ in range(3):
        layer(inp["h"], inp["w_router"], inp["w_gate"], inp["w_up"], inp["w_down"], out=y, **args)
    torch.cuda.synchronize()
    t0, n = time.time(), 0
    print(json.dumps({"sustain_start_unix": t0}), flush=True)
    while time.time() - t0 < seconds:
        for _ in range(20):
            layer(inp["h"], inp["w_router"], inp["w_gate"], inp["w_up"], inp["w_down"], out=y,
                  **args)
        torch.cuda.synchronize()
        n += 20
    dt = time.time() - t0
    print(json.dumps({"workload": w.name, "sustain_s": dt, "steps": n,
                      "ms_per_step": dt / n * 1e3, "sustain_end_unix": time.time()}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=W.MIXTRAL_PREFILL.name, choices=sorted(W.ALL))
    ap.add_argument("--decode-tokens", type=int, default=16)
    ap.add_argument("--cpu-sample", type=int, default=1 << 30,
                    help="tokens of the workload the CPU baseline runs (default: all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-decode-batches", action="store_true",
                    help="skip the decode batches other than --decode-tokens")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward-pass measurement")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the capacity / group-limited / fine-grained variant workloads")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--sustain", type=float, default=0.0,
                    help="run the workload's fused step back to back for this many seconds "
                         "(board power and clock sampling) and exit")
    ap.add_argument("--no-tiny", action="store_true",
                    help="skip the tiny fp32 configuration's GPU timing")
    ap.add_argument("--library-gemm", action="store_true",
                    help="time the vendor library on the uniform-batch equivalent of the "
                         "workload's gate/up GEMM (context) and exit")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported by this "
              "single-GPU build (sharding is described in the design notes, not built)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_mixture_experts_35_amd as M
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if a.copy_calibration:
        copy_calibration(torch)
        return
    if a.library_gemm:
        library_gemm(torch, W.ALL[a.workload], a.steps, a.warmup, a.sustain)
        return
    M.lib()   # fail loudly if the HIP library is missing

    w = W.ALL[a.workload]
    inp = W.device_inputs(w)
    torch.cuda.synchronize()
    if a.sustain > 0:
        sustain(M, torch, w, inp, a.sustain)
        return
    wall, stage, total_ev, counts = run_layer(M, torch, w, inp, a.steps, a.warmup)
    gu_ms = run_layer.gate_up_timed
    ms = wall / a.steps * 1e3
    tok_s = w.T * a.steps / wall
    flops_gu, bytes_gu, touched = gateup_work(w, counts)
    lflops, lbytes, _ = layer_work(w, counts)
    rows_per_expert = counts.sum() / max(touched, 1)
    mfma_bound = rows_per_expert > 64
    gu_s = gu_ms * 1e-3
    if mfma_bound:
        achieved = flops_gu / gu_s / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": measured_traffic(w.name, "grouped_gemm_gateup"),
                "kernel": "grouped_gemm_kernel (gate/up + SwiGLU)",
                "algorithmic_per_launch": flops_gu, "avg_launch_ms": gu_ms}
    else:
        achieved = bytes_gu / gu_s / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS,
                "traffic": measured_traffic(w.name, "skinny_gemm_gateup"),
                "kernel": "skinny_gemm_kernel (gate/up + SwiGLU)",
                "algorithmic_per_launch": bytes_gu, "avg_launch_ms": gu_ms}
    out = {
        "metric": METRIC, "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if w.dtype == W.DTYPE_BF16 else "f32",
        "data": "synthetic (seeded random inputs and random-init weights of this shape)",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "N": w.N, "k": w.k, "d_ff": w.d_ff,
                   "d_ff_shared": w.d_ff_shared, "gate_mode": w.mode,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "layer": {**fractions(*stage_work(w, counts)["layer"], ms),
                  "weight_gbs": lbytes / (ms * 1e-3) / 1e9,
                  "stages_ms": stage, "events_total_ms": total_ev,
                  "experts_touched": touched, "max_rows": int(counts.max())},
        "kernels": {"gate_up": fractions(*stage_work(w, counts)["gate_up"], gu_ms),
                    "down": fractions(*stage_work(w, counts)["down"], stage["down"])},
    }
    if not a.no_decode and w.T > a.decode_tokens:
        wd = w.replace(name=re.sub(r"prefill_T\d+", f"decode_T{a.decode_tokens}", w.name),
                       T=a.decode_tokens)
        dinp = dict(inp)
        dinp["h"] = inp["h"][:a.decode_tokens].contiguous()
        # a second copy of the expert weights, alternated step by step: the
        # weights come from HBM, never from the Infinity Cache
        alt = tuple(inp[key].clone() for key in ("w_gate", "w_up", "w_down"))
        dwall, dstage, _, dcounts = run_layer(M, torch, wd, dinp, max(a.steps, 20), a.warmup,
                                              gate_up_events=False, alt_weights=alt)
        dsteps = max(a.steps, 20)
        dms = dwall / dsteps * 1e3
        _, dbytes, dtouched = layer_work(wd, dcounts)
        out["decode"] = {"workload": wd.name, "tokens_per_s": wd.T * dsteps / dwall,
                         "ms_per_step": dms, "experts_touched": dtouched,
                         "layer": fractions(*stage_work(wd, dcounts)["layer"], dms),
                         "weight_bytes": dbytes,
                         "hbm_gbs_layer": dbytes / (dms * 1e-3) / 1e9,
                         "frac_hbm_peak_layer": dbytes / (dms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "stages_ms": dstage, "weight_copies_alternated": 2}
        # other decode batch sizes, the same way (the first tb tokens)
        others = []
        for tb in () if a.no_decode_batches else (1, 4, 32, 64):
            if tb == a.decode_tokens or tb >= w.T:
                continue
            wb = w.replace(name=re.sub(r"prefill_T\d+", f"decode_T{tb}", w.name), T=tb)
            binp = dict(inp)
            binp["h"] = inp["h"][:tb].contiguous()
            bwall, _, _, bcounts = run_layer(M, torch, wb, binp, dsteps, a.warmup,
                                             gate_up_events=False, alt_weights=alt)
            bms = bwall / dsteps * 1e3
            _, bbytes, btouched = layer_work(wb, bcounts)
            others.append({"T": tb, "ms_per_step": bms, "experts_touched": btouched,
                           "max_rows": int(bcounts.max()), "weight_bytes": bbytes,
                           "frac_hbm_peak_layer": bbytes / (bms * 1e-3) / 1e9 / PEAK_HBM_GBS})
        out["decode"]["other_batches"] = others
        del alt
        # weight-streaming kernels: algorithmic bytes (touched experts' weights,
        # rows in and out) against the counted HBM bytes per launch
        gb = {"gate_up": gateup_work(wd, dcounts)[1],
              "down": dtouched * w.d * w.d_ff * 2 + int(dcounts.sum()) * (w.d + w.d_ff) * 2}
        dsw = stage_work(wd, dcounts)
        out["decode"]["kernels"] = {
            n: {**fractions(dsw[n][0], gb[n], dstage[n]),
                "traffic": measured_traffic(wd.name, f"skinny_gemm_{n.replace('_', '')}")}
            for n in ("gate_up", "down")}
    if not a.no_backward:
        out["backward"] = run_backward(M, torch, w, inp, a.steps, a.warmup)
    if not a.no_variants:
        del inp
        torch.cuda.empty_cache()
        out["variants"] = [run_variant(M, torch, v, a.steps, a.warmup) for v in VARIANTS]
        inp = W.device_inputs(w)
    if not a.no_tiny:
        out["tiny_fp32"] = run_tiny(M, torch)
    if not a.no_cpu_baseline:
        cb = cpu_baseline(w, inp, a.cpu_sample)
        cb.update(host_info())
        cb.update(cpu_extras(torch, w, inp, 0 if a.no_decode else a.decode_tokens,
                             () if a.no_variants else VARIANTS))
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
