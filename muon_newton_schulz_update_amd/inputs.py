"""Seeded synthetic inputs for the Muon step (shapes and value distributions).

This module draws random numbers and rounds them to their storage types; it
holds none of the method's arithmetic. Both the HIP path and the float64
oracle read the *stored* tensors it returns (the ground truth).

Shapes come from the pages' models:
  * the GPT-2-124M-shaped Track-3 model (12 layers, width 768) of the Aurora
    record page (www.xxmr.cn/news/295280, section 复现与扩展建议);
  * the 3.8B Llama-style decoder of "将 3.8B LLM 培训至 0.384 CORE，仅需 998 美元"
    (www.66bd.net/article/34366): width 3072, 24 query / 8 key-value heads of
    128, relu^2 MLP of 4 x width, 28 layers.
Gradients are N(0, sd^2) with a log-normal (sigma = 1) scale per row (uneven
leverage); momenta N(0, sd^2) (or zero); weights N(0, 0.02^2). Each tensor
has its own seed, derived from (workload, matrix index, tensor kind), so any
subset of a batch can be regenerated alone.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

# tensor kinds (part of the seed)
_ROWSCALE, _GRAD, _MOM, _WEIGHT = 0, 1, 2, 3


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int                       # seed namespace
    shapes: tuple                  # ((rows, cols), ...)
    grad_dtype: torch.dtype
    grad_sd: float
    mom: str                       # "normal" | "zero" | "rowscaled"
    mom_sd: float
    weights: bool
    weight_dtype: torch.dtype
    weight_sd: float = 0.02
    config: tuple = ()             # config overrides as (key, value) pairs
    description: str = ""


def _gpt2_layer():
    return ((768, 768),) * 4 + ((3072, 768), (768, 3072))


def _llama38_layer():
    # q, o: 3072 x 3072; k, v: 1024 x 3072 (8 kv heads x 128); up 12288 x 3072; down 3072 x 12288
    return ((3072, 3072), (1024, 3072), (1024, 3072), (3072, 3072), (12288, 3072), (3072, 12288))


WORKLOADS = {
    "single_fp32_256x1024": Workload(
        "single_fp32_256x1024", 0, ((256, 1024),), torch.float32, 1.0, "rowscaled", 1.0,
        True, torch.float32,
        description="one fp32 256x1024 matrix; G and M N(0,1) sharing one log-normal row scale; "
                    "W N(0,0.02^2); full Aurora+Contra+floor step"),
    "ns_48x768sq_bf16": Workload(
        "ns_48x768sq_bf16", 1, ((768, 768),) * 48, torch.bfloat16, 1e-3, "zero", 0.0,
        False, torch.bfloat16, config=(("contra", 0.0),),
        description="48 square bf16 768x768 grads (12 layers x q,k,v,o of a d=768 GPT), "
                    "zero momentum, plain NS (square short-circuit, no Contra, no weights)"),
    "gpt2_124m_matrices": Workload(
        "gpt2_124m_matrices", 2, _gpt2_layer() * 12, torch.bfloat16, 1e-3, "normal", 1e-3,
        True, torch.bfloat16,
        description="GPT-2-124M-shaped matrix set: 12 x {4 x 768^2, 3072x768, 768x3072}; "
                    "bf16 grads, fp32 momentum, bf16 weights; full step"),
    "llama3p8b_layer": Workload(
        "llama3p8b_layer", 3, _llama38_layer(), torch.bfloat16, 1e-4, "normal", 1e-4,
        True, torch.bfloat16,
        description="one 3.8B-style GQA decoder layer (d=3072): q,o 3072^2, k,v 1024x3072, "
                    "up 12288x3072, down 3072x12288; full step"),
    "llama3p8b_all_layers": Workload(
        "llama3p8b_all_layers", 4, _llama38_layer() * 28, torch.bfloat16, 1e-4, "normal", 1e-4,
        True, torch.bfloat16,
        description="all 28 layers of the 3.8B-style model: 168 matrices, 2,818,572,288 "
                    "matrix parameters; full step with fp32 momentum resident in HBM"),
}


def seed_of(wid: int, index: int, kind: int, salt: int = 0) -> int:
    return ((wid * 1_000_003 + index) * 8 + kind) * 1_000_033 + salt


def _normal(shape, seed, device, sd=1.0):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * sd


def row_scales(rows: int, seed: int, device) -> torch.Tensor:
    """exp(N(0,1)) per row, shape (rows, 1)."""
    return torch.exp(_normal((rows, 1), seed, device))


def make_matrix(w: Workload, index: int, device, salt: int = 0):
    """(grad, momentum, weight-or-None) of matrix `index` of workload `w`."""
    rows, cols = w.shapes[index]
    rs = row_scales(rows, seed_of(w.wid, index, _ROWSCALE, salt), device)
    g = (_normal((rows, cols), seed_of(w.wid, index, _GRAD, salt), device, w.grad_sd) * rs).to(w.grad_dtype)
    if w.mom == "zero":
        m = torch.zeros((rows, cols), device=device, dtype=torch.float32)
    elif w.mom == "rowscaled":
        m = _normal((rows, cols), seed_of(w.wid, index, _MOM, salt), device, w.mom_sd) * rs
    else:
        m = _normal((rows, cols), seed_of(w.wid, index, _MOM, salt), device, w.mom_sd)
    wt = None
    if w.weights:
        wt = _normal((rows, cols), seed_of(w.wid, index, _WEIGHT, salt), device, w.weight_sd).to(w.weight_dtype)
    return g, m, wt


def make_batch(name: str, device, indices=None, salt: int = 0):
    """Lists (grads, moms, weights) for the chosen matrices of a workload."""
    w = WORKLOADS[name]
    idx = range(len(w.shapes)) if indices is None else indices
    grads, moms, weights = [], [], []
    for i in idx:
        g, m, wt = make_matrix(w, i, device, salt)
        grads.append(g)
        moms.append(m)
        weights.append(wt)
    return grads, moms, (weights if w.weights else None)


def custom_matrix(shape, seed, device, grad_dtype=torch.float32, grad_sd=1.0, mom_sd=1.0,
                  weight_dtype=torch.float32, weight_sd=0.02, rowscaled=True):
    """A single seeded (G, M, W) triple of any shape (tests of odd shapes)."""
    rows, cols = shape
    rs = row_scales(rows, seed * 4 + 0, device) if rowscaled else torch.ones((rows, 1), device=device)
    g = (_normal((rows, cols), seed * 4 + 1, device, grad_sd) * rs).to(grad_dtype)
    m = _normal((rows, cols), seed * 4 + 2, device, mom_sd)
    wt = _normal((rows, cols), seed * 4 + 3, device, weight_sd).to(weight_dtype)
    return g, m, wt


def counted_ns_flops(rows: int, cols: int, ns_steps: int = 12, passes: int = 1) -> float:
    """4 s^2 L + 2 s^3 per Newton-Schulz iteration (s <= L), times iterations and passes."""
    s, L = min(rows, cols), max(rows, cols)
    return float(passes * ns_steps * (4.0 * s * s * L + 2.0 * s ** 3))
