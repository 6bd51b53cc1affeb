"""Seeded synthetic inputs for the fine-grained MoE FFN layer.

This module draws random numbers and nothing else: it holds none of the
layer's arithmetic (no routing, no expert FFN, no combine).  Both the CPU
oracle and the HIP path receive the same arrays from it.

Shapes follow the dots.llm1 pages: 128 routed experts, top-6, 2 shared
experts, hidden size 5120 ("How dots.llm1's 14B MoE Architecture Matches 72B
LLM Performance", section "MoE Architecture Specifications"; "dots.llm1
Technical Report" summary, section "Method").  The expert SwiGLU width 1408 is
a chosen value; the pages do not fix it.

Draw order for every workload: x, router weight, selection bias, routed W1,
routed W2, shared W1, shared W2, upstream gradient dY.

Layouts (all row-major):
  x          [T, H]        bf16 values (fp32 for the tiny workload)
  w_router   [H, E]        fp32
  bias       [E]           fp32 (selection bias)
  w1         [E, 2F, H]    rows 0..F-1 are the gate projection, F..2F-1 up
  w2         [E, H, F]
  w1_sh      [S, 2F, H]    per shared expert, same convention as w1
  w2_sh      [S, H, F]
  dy         [T, H]

Two backends draw them: NumPy's PCG64 on the host (any workload that fits
host memory quickly) and torch's device generator (the full-size workloads,
drawn straight into HBM).  The two backends give different values for one
seed; a test always feeds both sides from one backend.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    E: int
    K: int
    S: int
    F: int
    seed: int
    x_std: float = 1.0
    w_std: float = 0.02
    router_std: float = 0.02
    bias_std: float = 1e-3
    bias_kind: str = "normal"  # "normal" | "zipf"
    zipf_s: float = 1.2
    all_fp32: bool = False     # tiny workload: no bf16 rounding of x / W1 / W2
    backward: bool = False

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads: a tiny all-fp32 layer, then dots.llm1 shapes at decode
# (T=256), prefill (T=8192), skewed load (T=16384) and forward+backward (T=8192).
WORKLOADS = {
    "tiny": Workload("tiny", T=128, H=64, E=8, K=2, S=1, F=32, seed=0,
                     bias_std=0.02, all_fp32=True),
    "decode": Workload("decode", T=256, H=5120, E=128, K=6, S=2, F=1408, seed=1),
    "prefill": Workload("prefill", T=8192, H=5120, E=128, K=6, S=2, F=1408, seed=2),
    "skew": Workload("skew", T=16384, H=5120, E=128, K=6, S=2, F=1408, seed=3,
                     bias_kind="zipf"),
    "fwdbwd": Workload("fwdbwd", T=8192, H=5120, E=128, K=6, S=2, F=1408, seed=4,
                       backward=True),
}


# ----------------------------------------------------------------------------
# bf16 helpers (input preparation only: round-to-nearest-even of fp32 values)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even; NaN -> canonical qNaN."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        rounded[nan] = 0x7FC0
    return rounded


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_round(a: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 value, returned as fp32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(a))


def zipf_bias(E: int, s: float) -> np.ndarray:
    """Selection bias 0.5*ln(p_e), p_e proportional to (e+1)^-s (expert 0 most popular)."""
    w = np.array([(e + 1) ** (-s) for e in range(E)], dtype=np.float64)
    p = w / w.sum()
    return (0.5 * np.log(p)).astype(np.float32)


# ----------------------------------------------------------------------------
# NumPy backend
# ----------------------------------------------------------------------------
def generate_numpy(w: Workload, with_dy: bool | None = None) -> dict:
    """All inputs as NumPy arrays.

    x, w1, w2, w1_sh, w2_sh, dy are fp32 arrays holding bf16-exact values
    (unless the workload is all-fp32); the router weight and bias are fp32.
    """
    rng = np.random.default_rng(w.seed)
    T, H, E, K, S, F = w.T, w.H, w.E, w.K, w.S, w.F
    rnd = (lambda a: a) if w.all_fp32 else bf16_round

    def normal(shape, std):
        return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)

    x = rnd(normal((T, H), w.x_std))
    w_router = normal((H, E), w.router_std)
    if w.bias_kind == "zipf":
        bias = zipf_bias(E, w.zipf_s)
    else:
        bias = normal((E,), w.bias_std)
    w1 = np.empty((E, 2 * F, H), np.float32)
    for e in range(E):
        w1[e] = rnd(normal((2 * F, H), w.w_std))
    w2 = np.empty((E, H, F), np.float32)
    for e in range(E):
        w2[e] = rnd(normal((H, F), w.w_std))
    w1_sh = rnd(normal((S, 2 * F, H), w.w_std))
    w2_sh = rnd(normal((S, H, F), w.w_std))
    out = dict(x=x, w_router=w_router, bias=bias, w1=w1, w2=w2,
               w1_sh=w1_sh, w2_sh=w2_sh)
    if w.backward if with_dy is None else with_dy:
        out["dy"] = rnd(normal((T, H), 1.0))
    return out


# ----------------------------------------------------------------------------
# torch device backend (full-size workloads straight into HBM)
# ----------------------------------------------------------------------------
def generate_torch(w: Workload, device, with_dy: bool | None = None) -> dict:
    """All inputs as torch tensors on `device`.

    x, w1, w2, w1_sh, w2_sh, dy are bfloat16 (fp32 for an all-fp32 workload);
    router weight and bias are fp32.  Drawn in chunks so peak extra memory is
    one expert's fp32 weights.
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(w.seed)
    T, H, E, K, S, F = w.T, w.H, w.E, w.K, w.S, w.F
    dt = torch.float32 if w.all_fp32 else torch.bfloat16

    def normal(shape, std, dtype=dt):
        return (torch.randn(shape, generator=g, device=device, dtype=torch.float32)
                * std).to(dtype)

    x = normal((T, H), w.x_std)
    w_router = normal((H, E), w.router_std, torch.float32)
    if w.bias_kind == "zipf":
        bias = torch.from_numpy(zipf_bias(E, w.zipf_s)).to(device)
    else:
        bias = normal((E,), w.bias_std, torch.float32)
    w1 = torch.empty((E, 2 * F, H), dtype=dt, device=device)
    for e in range(E):
        w1[e] = normal((2 * F, H), w.w_std)
    w2 = torch.empty((E, H, F), dtype=dt, device=device)
    for e in range(E):
        w2[e] = normal((H, F), w.w_std)
    w1_sh = normal((S, 2 * F, H), w.w_std)
    w2_sh = normal((S, H, F), w.w_std)
    out = dict(x=x, w_router=w_router, bias=bias, w1=w1, w2=w2,
               w1_sh=w1_sh, w2_sh=w2_sh)
    if w.backward if with_dy is None else with_dy:
        out["dy"] = normal((T, H), 1.0)
    return out


# ----------------------------------------------------------------------------
# The expert-parallel shard (one GPU's share when the layer is split over 8)
# ----------------------------------------------------------------------------
# With expert parallelism over 8 GPUs each GPU holds 16 of the 128 routed
# experts and receives, through the dispatch exchange, the rows its experts
# were picked for: 8 GPUs x 8192 tokens x 6 picks / 128 experts = 3072 rows
# per expert at near-uniform routing ("dots.llm1 Technical Report" summary,
# "Method": expert-parallel training with the all-to-all overlapped).
EP_SHARD = dict(E=16, rows=3072, H=5120, F=1408, seed=5)


def generate_shard_torch(device, E: int, rows: int, H: int, F: int, seed: int) -> dict:
    """Inputs of the grouped expert products at the shard, drawn on `device`
    in the order x_rows, w1, w2, dy_rows (bf16): x_rows [E*rows, H] ~ N(0,1)
    (the received rows, grouped by expert), w1 [E, 2F, H] and w2 [E, H, F]
    ~ N(0, 0.02), dy_rows [E*rows, H] ~ N(0,1) (the returned gradient rows)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def normal(shape, std):
        return (torch.randn(shape, generator=g, device=device, dtype=torch.float32)
                * std).to(torch.bfloat16)

    x_rows = normal((E * rows, H), 1.0)
    w1 = torch.empty((E, 2 * F, H), dtype=torch.bfloat16, device=device)
    for e in range(E):
        w1[e] = normal((2 * F, H), 0.02)
    w2 = torch.empty((E, H, F), dtype=torch.bfloat16, device=device)
    for e in range(E):
        w2[e] = normal((H, F), 0.02)
    dy_rows = normal((E * rows, H), 1.0)
    return dict(x_rows=x_rows, w1=w1, w2=w2, dy_rows=dy_rows)


def useful_flops(w: Workload, backward: bool) -> float:
    """Algorithmic flops of the layer, padding rows excluded.

    forward : 2HE (router) + (K+S)*6HF (three H x F products per active expert)
    backward: adds 4HK (sparse router backward: dW_r and dx_r on the K selected
              logits) and twice the expert products again (dgrad + wgrad).
    """
    T, H, E, K, S, F = w.T, w.H, w.E, w.K, w.S, w.F
    fwd = 2 * H * E + (K + S) * 6 * H * F
    if not backward:
        return float(T) * fwd
    return float(T) * (2 * H * E + 4 * H * K + 3 * (K + S) * 6 * H * F)


def gemm_useful_flops(w: Workload, backward: bool) -> float:
    """Flops of the expert GEMMs alone (routed + shared), padding excluded."""
    T, H, K, S, F = w.T, w.H, w.K, w.S, w.F
    return float(T) * (K + S) * 6 * H * F * (3 if backward else 1)

