"""GPU parity over a seeded sweep of shapes: every C-ABI call and the fused
layer against the float64 oracle (the rules of test_gpu_parity), on shapes
drawn at random from the ranges the library supports — 1 to 700 tokens, 1 to
512 experts, k up to 16, d or d_ff up to 8192, both dtypes, the three gate
modes, with and without a shared expert, a group limit and an expert
capacity — so that the kernel
variants meet combinations the hand-picked cases do not (selection layouts,
single-block selection + dispatch, skinny and tiled GEMMs, split-K tails,
the fused decode combine), and the backward pass on the first 40 of them;
then 24 larger shapes (800 to 6,000 tokens)."""
import math

import numpy as np
import pytest

import workloads as W
from test_gpu_parity import capacity_of, check_all, run_steps, shape_of

pytestmark = pytest.mark.gpu


def _groups(rng, N, k):
    divs = [g for g in range(2, min(N, 64) + 1) if N % g == 0]
    if not divs:
        return None
    ng = int(rng.choice(divs))
    gsz = N // ng
    keep = int(rng.integers(math.ceil(k / gsz), ng + 1))
    topm = int(rng.integers(1, min(gsz, 8) + 1))
    return (ng, keep, topm)


def sweep_cases(n=96, seed=2024):
    """Deterministic list of (name, T, d, N, k, d_ff, d_ff_shared, dtype,
    mode, groups, capacity_factor)."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        bf16 = rng.random() < 0.8
        dt = W.DTYPE_BF16 if bf16 else W.DTYPE_F32
        d = int(rng.choice([64, 128, 192, 256] if bf16 else [16, 32, 48, 64]))
        dff = int(rng.choice([64, 128, 192, 320] if bf16 else [16, 40, 64]))
        N = int(rng.choice([1, 2, 3, 5, 8, 13, 16, 31, 64, 100, 128, 257, 512]))
        wide = rng.random()
        if bf16 and wide < 0.15:       # long K in gate/up: split-K tails
            d = int(rng.choice([1024, 2048, 4096]))
            N = int(rng.choice([1, 2, 3, 5, 8]))
        elif bf16 and wide < 0.3:      # long K in down
            dff = int(rng.choice([2048, 4096, 8192]))
            N = int(rng.choice([1, 2, 3, 5, 8]))
        k = int(rng.integers(1, min(N, 16) + 1))
        T = int(rng.choice([1, 2, 7, 16, 33, 64, 129, 300, 700]))
        dfs = int(rng.choice([0, 0, 64, 128] if bf16 else [0, 24]))
        mode = int(rng.integers(0, 3))
        if N * d * dff > (8 << 20):          # keep the host weights small
            continue
        groups = _groups(rng, N, k) if (N >= 4 and rng.random() < 0.3) else None
        cf = 0.0 if rng.random() < 0.7 else min(float(rng.choice([0.25, 0.5, 1.0, 1.5])), N)
        name = (f"s{len(cases):02d}_{'bf16' if bf16 else 'f32'}_T{T}_d{d}_N{N}_k{k}_ff{dff}"
                f"_sh{dfs}_m{mode}" + (f"_g{groups[0]}-{groups[1]}-{groups[2]}" if groups else "")
                + (f"_cf{cf}" if cf else ""))
        cases.append((name, T, d, N, k, dff, dfs, dt, mode, groups, cf))
    return cases


CASES = sweep_cases()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_sweep(case):
    name, T, d, N, k, dff, dfs, dt, mode, groups, cf = case
    inp = W.random_small(T, d, N, k, dff, dfs, dt, mode, seed=len(name) + T,
                         router_bias=(T % 2 == 0))
    s = shape_of(T, d, N, k, dff, dfs, dt, mode, groups=groups, cf=cf)
    print(f"case {name}", flush=True)
    res = run_steps(s, inp)
    worst, near = check_all(s, inp, res)
    cap = capacity_of(s)
    dropped = int((res["row_of"] < 0).sum())
    if cap is None:
        assert dropped == 0
    print(f"{name}: worst row rel err {worst:.2e}, near-ties {near}, dropped {dropped}")


# The backward pass on the first 40 shapes of the sweep, with the auxiliary
# loss weights drawn too.
BWD_CASES = CASES[:40]


@pytest.mark.parametrize("case", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_sweep_backward(case):
    from test_gpu_backward import check_backward, run_backward
    name, T, d, N, k, dff, dfs, dt, mode, groups, cf = case
    inp = W.random_small(T, d, N, k, dff, dfs, dt, mode, seed=len(name) + T,
                         router_bias=(T % 2 == 0))
    s = shape_of(T, d, N, k, dff, dfs, dt, mode, groups=groups, cf=cf)
    rng = np.random.default_rng(len(name) + 3)
    d_laux, d_zloss = (float(x) for x in rng.choice([0.0, 0.3, 1.0], size=2))
    dy = rng.standard_normal((T, d)).astype(np.float32)
    if dt == W.DTYPE_BF16:
        dy = W.round_to_bf16(dy)
    print(f"case {name} d_laux {d_laux} d_zloss {d_zloss}", flush=True)
    res = run_backward(s, inp, dy, d_laux, d_zloss)
    worst = check_backward(s, inp, dy, res, d_laux, d_zloss)
    print(f"{name}: " + ", ".join(f"{k_} {v[0]:.1e}/{v[1]:.1f}/{v[2]:.2f}" for k_, v in worst.items()))


def large_cases(n=24, seed=5):
    """Deterministic list of larger shapes (800 to 6,000 tokens; up to 512
    experts): many dispatch chunks, grouped tiles with split-K tails, the
    selection's one-pass blocks."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        bf16 = rng.random() < 0.85
        dt = W.DTYPE_BF16 if bf16 else W.DTYPE_F32
        T = int(rng.integers(800, 6001))
        N = int(rng.choice([2, 8, 16, 60, 64, 128, 200, 256, 512]))
        k = int(rng.integers(1, min(N, 8) + 1))
        d = int(rng.choice([64, 128, 256] if bf16 else [32, 64]))
        dff = int(rng.choice([64, 128, 256, 384] if bf16 else [32, 48]))
        dfs = int(rng.choice([0, 0, 128] if bf16 else [0, 32]))
        mode = int(rng.integers(0, 3))
        groups = _groups(rng, N, k) if (N >= 4 and rng.random() < 0.25) else None
        cf = 0.0 if rng.random() < 0.75 else float(rng.choice([0.5, 1.0, 1.25]))
        name = (f"L{i:02d}_{'bf16' if bf16 else 'f32'}_T{T}_d{d}_N{N}_k{k}_ff{dff}_sh{dfs}_m{mode}"
                + (f"_g{groups[0]}-{groups[1]}-{groups[2]}" if groups else "")
                + (f"_cf{cf}" if cf else ""))
        cases.append((name, T, d, N, k, dff, dfs, dt, mode, groups, cf))
    return cases


LARGE = large_cases()


@pytest.mark.parametrize("case", LARGE, ids=[c[0] for c in LARGE])
def test_sweep_large(case):
    name, T, d, N, k, dff, dfs, dt, mode, groups, cf = case
    inp = W.random_small(T, d, N, k, dff, dfs, dt, mode, seed=len(name) + T,
                         router_bias=(T % 2 == 0))
    s = shape_of(T, d, N, k, dff, dfs, dt, mode, groups=groups, cf=cf)
    print(f"case {name}", flush=True)
    res = run_steps(s, inp)
    worst, near = check_all(s, inp, res)
    print(f"{name}: worst row rel err {worst:.2e}, near-ties {near}")
