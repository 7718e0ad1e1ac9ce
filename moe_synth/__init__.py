"""Seeded synthetic inputs for the routed 4-bit MoE layer.

Shared by the tests, the bench and the oracle's callers. Holds only random
number generation and the workload shapes: none of the method's arithmetic
(no quantization, routing, GEMM or combine). Inputs are synthetic stand-ins
for the pages' real-text workloads (no dataset or checkpoint is used):
  x      ~ N(0, 1) rounded to bf16 (RNE), [T, H]
  W_r    ~ N(0, 0.02) fp32, [E, H]
  b_r    per-expert prior log p_e (Zipf s=1.2 over a seeded rank order) or none
  w13    ~ N(0, 0.02) fp32, [E, 2I, H]   (rows [0, I) gate, [I, 2I) up)
  w2     ~ N(0, 0.02) fp32, [E, H, I]
  b13, b2 (the gpt-oss expert form only) ~ N(0, 0.1) fp32, [E, 2I] and [E, H]
Layer l of workload c uses seed 1000*c + l; each tensor draws from its own
stream, and each expert of a weight stack from its own sub-stream so any
single expert can be regenerated alone.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

FMT_NF4 = 0
FMT_MXFP4 = 1

_STREAM = {"x": 1, "router_w": 2, "router_b": 3, "w13": 4, "w2": 5, "b13": 6, "b2": 7}


@dataclass(frozen=True)
class Workload:
    """One MoE-layer workload: shapes, format, routing prior, token counts."""
    wid: int
    name: str
    fmt: int
    E: int
    top_k: int
    H: int
    I: int
    tokens: tuple
    layers: int = 1
    zipf_s: float = 0.0          # 0 -> no prior (uniform expected load)
    renormalize: int = 1
    notes: str = field(default="", compare=False)


WORKLOADS = {
    "tiny": Workload(0, "tiny", FMT_NF4, 8, 2, 256, 128, (16,), layers=1,
                     notes="E=8 top_k=2 H=256 I=128 T=16, NF4 blocksize 64"),
    "olmoe_decode": Workload(1, "olmoe_decode", FMT_NF4, 64, 8, 2048, 1024, (1,), layers=64,
                             notes="OLMoE-1B-7B-shaped layer, T=1, 64 rotated layers"),
    "olmoe_prefill": Workload(2, "olmoe_prefill", FMT_NF4, 64, 8, 2048, 1024, (4096,), layers=8,
                              notes="OLMoE-1B-7B-shaped layer, T=4096, uniform expected load"),
    "qwen3_zipf": Workload(3, "qwen3_zipf", FMT_NF4, 128, 8, 2048, 768, (1, 16, 512), layers=64,
                           zipf_s=1.2, notes="Qwen3-30B-A3B-shaped layer, Zipf(1.2) expert prior"),
    "gptoss_mxfp4": Workload(4, "gptoss_mxfp4", FMT_MXFP4, 128, 4, 2880, 2880, (1, 2048), layers=16,
                             notes="gpt-oss-120b-shaped MXFP4 layer"),
}


def _rng(wl: Workload, layer: int, what: str, sub: int = 0) -> np.random.Generator:
    return np.random.default_rng([1000 * wl.wid + layer, _STREAM[what], sub])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16 (round to nearest even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def make_x(wl: Workload, T: int, layer: int = 0) -> np.ndarray:
    """Activations as bf16 bits [T, H]."""
    x = _rng(wl, layer, "x", T).standard_normal((T, wl.H), dtype=np.float32)
    return f32_to_bf16_bits(x)


def make_router(wl: Workload, layer: int = 0):
    """(W_r fp32 [E, H], b_r fp32 [E] or None)."""
    W = (_rng(wl, layer, "router_w").standard_normal((wl.E, wl.H), dtype=np.float32)
         * np.float32(0.02))
    b = None
    if wl.zipf_s > 0:
        rank = _rng(wl, layer, "router_b").permutation(wl.E) + 1
        p = rank.astype(np.float64) ** (-wl.zipf_s)
        b = np.log(p / p.sum()).astype(np.float32)
    return W.astype(np.float32), b


def make_expert(wl: Workload, layer: int, which: str, e: int) -> np.ndarray:
    """fp32 weights of one expert: which='w13' -> [2I, H], 'w2' -> [H, I]."""
    shape = (2 * wl.I, wl.H) if which == "w13" else (wl.H, wl.I)
    g = _rng(wl, layer, which, e + 1)
    return (g.standard_normal(shape, dtype=np.float32) * np.float32(0.02)).astype(np.float32)


def make_stack(wl: Workload, layer: int, which: str, experts=None) -> np.ndarray:
    """fp32 weight stack [E, N, K] (or only the listed experts, in order)."""
    ids = range(wl.E) if experts is None else experts
    return np.stack([make_expert(wl, layer, which, int(e)) for e in ids])


def make_biases(wl: Workload, layer: int = 0):
    """Per-expert biases of the gpt-oss expert form: (b13 fp32 [E, 2I], b2 fp32 [E, H])."""
    b13 = _rng(wl, layer, "b13").standard_normal((wl.E, 2 * wl.I), dtype=np.float32) * np.float32(0.1)
    b2 = _rng(wl, layer, "b2").standard_normal((wl.E, wl.H), dtype=np.float32) * np.float32(0.1)
    return b13.astype(np.float32), b2.astype(np.float32)


def make_stack_torch(wl: Workload, layer: int, which: str, device):
    """fp32 weight stack [E, N, K] drawn on a torch device (fast path for big
    workloads; torch's own Philox stream, seeded like the numpy one)."""
    import torch
    shape = (wl.E, 2 * wl.I, wl.H) if which == "w13" else (wl.E, wl.H, wl.I)
    g = torch.Generator(device=device)
    g.manual_seed((1000 * wl.wid + layer) * 16 + _STREAM[which])
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return t.mul_(0.02)


def custom(E, top_k, H, I, fmt=FMT_NF4, zipf_s=0.0, wid=9, renormalize=1) -> Workload:
    return Workload(wid, f"custom_{E}_{top_k}_{H}_{I}", fmt, E, top_k, H, I, (1,),
                    zipf_s=zipf_s, renormalize=renormalize)
