"""Seeded synthetic inputs for the grouped W4A16 MoE layer.

This module only draws numbers: activations, router weights and expert weights
with the shapes and distributions of the evaluated workloads, rounded to bf16.
It holds none of the layer's arithmetic (no quantisation, routing, permutation
or contraction), so both the CPU oracle and the HIP path may take their inputs
from here without sharing any of the method.

The evaluation in ExactMoE (page "Every Expert Counts: ExactMoE for
Memory-Efficient W4A16 Inference", Abstract) uses a trained OLMoE-1B-7B model;
no weights are available here, so seeded Gaussian / uniform tensors of the same
shapes stand in for them.

Every tensor is a pure function of (seed, shape, distribution, device): torch's
seeded generator (mt19937 on the CPU, Philox on the GPU) draws float32 values
that are rounded once to bf16 (round-to-nearest-even).  The two devices give
different streams for one seed, so a test draws each tensor on one device and
copies the bf16 bits wherever else they are needed.  Large banks are drawn on
the GPU.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import torch

SEED_BASE = 20260815

# tensor-kind tags mixed into per-tensor seeds
_KIND = {"x": 1, "router": 2, "w13": 3, "w2": 4, "zipf_perm": 5, "ar_noise": 6, "misc": 7}


@dataclass(frozen=True)
class LayerShape:
    """Shape of one MoE FFN layer: d_model, experts, top-k, expert intermediate."""
    d: int
    E: int
    k: int
    I: int


@dataclass(frozen=True)
class Workload:
    name: str
    shape: LayerShape
    layers: int
    tokens: List[int]
    router: str = "normal"          # "normal" | "uniform" | "zipf"
    slots: Optional[int] = None
    zipf_s: float = 1.2
    ar_rho: float = 0.9
    weight_std: float = 0.02
    router_std: float = 0.02
    x_std: float = 1.0
    notes: str = ""


TINY = Workload("tiny", LayerShape(d=256, E=8, k=2, I=512), layers=1, tokens=[16],
                notes="T=16, d=256, E=8, top-2, I=512")
OLMOE_DECODE = Workload("olmoe_decode", LayerShape(d=2048, E=64, k=8, I=1024), layers=16,
                        tokens=[1, 4, 16], notes="OLMoE-1B-7B-shaped decode, 16 layers, all experts resident")
OLMOE_PREFILL = Workload("olmoe_prefill", LayerShape(d=2048, E=64, k=8, I=1024), layers=16,
                         tokens=[512, 4096], router="uniform",
                         notes="OLMoE-shaped batched prefill, uniform router weights")
OLMOE_SLOT = Workload("olmoe_slot16", LayerShape(d=2048, E=64, k=8, I=1024), layers=16,
                      tokens=[16], router="zipf", slots=16,
                      notes="OLMoE-shaped decode with 16 GPU slots, Zipf(1.2) popularity, AR(1) locality")
LARGE = Workload("large_expert", LayerShape(d=4096, E=8, k=2, I=14336), layers=4,
                 tokens=[1, 64, 1024], notes="d=4096, E=8, top-2, I=14336")

WORKLOADS = {w.name: w for w in (TINY, OLMOE_DECODE, OLMOE_PREFILL, OLMOE_SLOT, LARGE)}


def tensor_seed(workload: str, layer: int, kind: str, step: int = 0) -> int:
    """Deterministic 63-bit seed for one tensor of one workload."""
    h = SEED_BASE
    for v in (sum(ord(c) * 131 ** i for i, c in enumerate(workload)), layer, _KIND[kind], step):
        h = (h * 6364136223846793005 + 1442695040888963407 + v) & ((1 << 63) - 1)
    return h


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal_bf16(shape, std: float, seed: int, device="cpu") -> torch.Tensor:
    """N(0, std^2) drawn in float32 and rounded once to bf16."""
    t = torch.randn(shape, generator=_gen(seed, device), device=device, dtype=torch.float32)
    return t.mul_(std).to(torch.bfloat16)


def uniform_bf16(shape, lo: float, hi: float, seed: int, device="cpu") -> torch.Tensor:
    t = torch.rand(shape, generator=_gen(seed, device), device=device, dtype=torch.float32)
    return t.mul_(hi - lo).add_(lo).to(torch.bfloat16)


def expert_weights(wl: Workload, layer: int, device="cpu", experts: Optional[List[int]] = None):
    """Expert weights of one layer as bf16: (w13 [E, 2I, d], w2 [E, d, I]).

    w13 rows 0..I-1 are the gate projection, rows I..2I-1 the up projection.
    If ``experts`` is given only those experts are drawn (same values as in the
    full bank: every expert has its own seed).
    """
    s = wl.shape
    ids = range(s.E) if experts is None else experts
    w13 = torch.stack([normal_bf16((2 * s.I, s.d), wl.weight_std,
                                   tensor_seed(wl.name, layer, "w13", e), device) for e in ids])
    w2 = torch.stack([normal_bf16((s.d, s.I), wl.weight_std,
                                  tensor_seed(wl.name, layer, "w2", e), device) for e in ids])
    return w13, w2


def zipf_log_popularity(wl: Workload, layer: int) -> torch.Tensor:
    """log p_{pi(e)} with p_r proportional to r^-s over ranks r=1..E, pi a seeded permutation."""
    E = wl.shape.E
    ranks = torch.arange(1, E + 1, dtype=torch.float64)
    logp = -wl.zipf_s * torch.log(ranks)
    logp = logp - torch.logsumexp(logp, 0)
    perm = torch.randperm(E, generator=_gen(tensor_seed(wl.name, layer, "zipf_perm"), "cpu"))
    return logp[perm]


def router_weight(wl: Workload, layer: int, device="cpu") -> torch.Tensor:
    """Router weight [E, d] bf16.

    normal: N(0, router_std^2).  uniform: U(-a, a) with the same std.
    zipf: normal, with input channel 0 reserved as a bias channel that carries the
    per-expert log popularity (activations hold 1.0 in that channel), so the
    router itself produces Zipf-biased logits through its ordinary dot product.
    """
    s = wl.shape
    seed = tensor_seed(wl.name, layer, "router")
    if wl.router == "uniform":
        a = wl.router_std * math.sqrt(3.0)
        return uniform_bf16((s.E, s.d), -a, a, seed, device)
    w = normal_bf16((s.E, s.d), wl.router_std, seed, device)
    if wl.router == "zipf":
        w[:, 0] = zipf_log_popularity(wl, layer).to(torch.float32).to(torch.bfloat16).to(device)
    return w


def activations(wl: Workload, T: int, layer: int, step: int = 0, device="cpu") -> torch.Tensor:
    """Activations x [T, d] bf16 ~ N(0, x_std^2) (fresh per layer and step)."""
    s = wl.shape
    x = normal_bf16((T, s.d), wl.x_std, tensor_seed(wl.name, layer, "x", step * 1000 + T), device)
    if wl.router == "zipf":
        x[:, 0] = 1.0
    return x


def ar1_activation_sequence(wl: Workload, T: int, layer: int, steps: int, device="cpu"):
    """Decode steps with per-step locality: x_s = rho*x_{s-1} + sqrt(1-rho^2)*z_s.

    Drawn in float32, each step rounded to bf16; channel 0 is the bias channel
    (1.0) when the workload uses Zipf-biased routing.
    """
    s = wl.shape
    rho = wl.ar_rho
    prev = torch.randn((T, s.d), generator=_gen(tensor_seed(wl.name, layer, "ar_noise", 0), device),
                       device=device, dtype=torch.float32) * wl.x_std
    out = []
    for st in range(steps):
        if st > 0:
            z = torch.randn((T, s.d), generator=_gen(tensor_seed(wl.name, layer, "ar_noise", st), device),
                            device=device, dtype=torch.float32) * wl.x_std
            prev = rho * prev + math.sqrt(1.0 - rho * rho) * z
        xb = prev.to(torch.bfloat16)
        if wl.router == "zipf":
            xb[:, 0] = 1.0
        out.append(xb)
    return out


def residual_stream_sequence(wl: Workload, T: int, steps: int, rho_layer: float = 0.9, device="cpu"):
    """Decode steps of every layer's MoE input, [steps][layers] of [T, d] bf16, with
    locality across steps and across layers: each layer has its own AR(1) sequence
    a (ar1_activation_sequence, coefficient ar_rho over steps), and
    x[s][0] = a_0[s], x[s][l+1] = rho_layer * x[s][l] + sqrt(1 - rho_layer^2) * a_{l+1}[s]
    (consecutive layers see correlated inputs, as along a residual stream; every
    x[.][l] keeps unit variance and step coefficient ar_rho).  Mixed in float32,
    each input rounded once to bf16; channel 0 is the bias channel (1.0) when the
    workload uses Zipf-biased routing."""
    per = [ar1_activation_sequence(wl, T, l, steps, device) for l in range(wl.layers)]
    c = math.sqrt(1.0 - rho_layer * rho_layer)
    out = []
    for st in range(steps):
        prev = per[0][st].to(torch.float32)
        row = [per[0][st]]
        for l in range(1, wl.layers):
            cur = rho_layer * prev + c * per[l][st].to(torch.float32)
            if wl.router == "zipf":
                cur[:, 0] = 1.0
            row.append(cur.to(torch.bfloat16))
            prev = cur
        out.append(row)
    return out


def random_topk_ids(T: int, E: int, k: int, seed: int) -> torch.Tensor:
    """Distinct expert ids per token (uniform), int32 [T, k]; used for permutation tests."""
    g = _gen(seed, "cpu")
    return torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(T)]).to(torch.int32) \
        if T > 0 else torch.zeros((0, k), dtype=torch.int32)
