"""Seeded synthetic inputs for the block-scaled quantization path.

This module only draws random numbers and stores them as bf16; it holds no
quantization, scaling or GEMM arithmetic, so both the HIP path and the CPU
oracle can take their inputs from it without sharing any of the method.

Shapes and value distributions follow the workloads described on the pages:
activations are N(0,1) with a 0.1 % fraction of entries multiplied by 50
(outliers), optionally with a per-row magnitude drawn log-uniformly; expert
weights are N(0, 0.02); router logits are N(0,1) plus a per-expert bias that
skews the tokens-per-expert counts (Zipf popularity).  Model shapes are those
of Qwen3-30B-A3B (hidden 2048, expert intermediate 768, 128 experts, top-8) and
DeepSeek-V3 (hidden 7168, expert projections 7168x2048, 256 routed + 1 shared
expert, top-8) [hackernews.jp "4ビットの教訓", footnote 5;
alphasignal.ai "LMSYS Drops Miles", Results on Qwen3-30B-A3B].

Host generators use numpy's PCG64 with a fixed draw order; the device
generators (for tensors of several GB, where a host draw would take minutes)
use torch's seeded CUDA generator.  Both are deterministic for a given seed and
shape.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits_from_f32",
    "f32_from_bf16_bits",
    "activations",
    "weights",
    "fp32_matrix",
    "zipf_bias",
    "route_topk",
    "device_activations",
    "device_weights",
    "CONFIG_SEED_BASE",
]

CONFIG_SEED_BASE = 20261201


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Store float32 values as bf16 bit patterns (round to nearest even).

    This is only the storage conversion of the synthetic draws into the
    path's input dtype; inputs are finite by construction.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (b.astype(np.uint64) + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def activations(seed: int, rows: int, cols: int, *, outlier_frac: float = 1e-3,
                outlier_mult: float = 50.0, row_log10_range: tuple | None = None,
                std: float = 1.0) -> np.ndarray:
    """bf16 bits [rows, cols]: N(0, std) * row magnitude * (outlier_mult on outliers).

    Draw order: normals, outlier uniforms, then (optional) row magnitudes.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    z = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(std)
    if outlier_frac > 0:
        mask = rng.random((rows, cols), dtype=np.float32) < outlier_frac
        z = np.where(mask, z * np.float32(outlier_mult), z)
    if row_log10_range is not None:
        lo, hi = row_log10_range
        mag = np.power(np.float32(10.0), rng.uniform(lo, hi, size=(rows, 1)).astype(np.float32))
        z = z * mag.astype(np.float32)
    return bf16_bits_from_f32(z.astype(np.float32))


def weights(seed: int, experts: int, rows: int, cols: int, std: float = 0.02) -> np.ndarray:
    """bf16 bits [experts * rows, cols] of N(0, std), drawn expert by expert."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = np.empty((experts * rows, cols), dtype=np.uint16)
    for e in range(experts):
        w = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(std)
        out[e * rows:(e + 1) * rows] = bf16_bits_from_f32(w)
    return out


def fp32_matrix(seed: int, rows: int, cols: int, std: float = 1.0) -> np.ndarray:
    """float32 [rows, cols] of N(0, std) (e.g. a synthetic gate/up GEMM output)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(std)


def zipf_bias(seed: int, experts: int, exponent: float = 1.1, uniform_mix: float = 0.0) -> np.ndarray:
    """Per-expert router bias giving Zipf-skewed expert popularity.

    Popularity p_e is proportional to rank_e ** -exponent, with the ranks a
    seeded permutation of 1..E; the bias is ln(uniform_mix / E + (1 -
    uniform_mix) * p_e).  uniform_mix = 0 gives a pure Zipf load, 0.5 the
    "uniform plus Zipf" load.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    ranks = rng.permutation(experts) + 1
    p = ranks.astype(np.float64) ** (-exponent)
    p /= p.sum()
    mix = uniform_mix / experts + (1.0 - uniform_mix) * p
    return np.log(mix).astype(np.float32)


def route_topk(seed: int, tokens: int, experts: int, topk: int, bias: np.ndarray,
               shared_expert: bool = False):
    """Synthetic top-k routing: returns (group_offsets int64 [G+1], src int32 [R]).

    Logits are N(0,1) + bias (float32).  Each token takes its top-k experts
    (ties to the lower expert id).  Grouped rows are ordered by expert, then by
    token id; src[r] is the token of grouped row r.  With shared_expert, an
    extra last group holds every token in order.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    logits = rng.standard_normal((tokens, experts), dtype=np.float32) + bias[None, :].astype(np.float32)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :topk]
    tok = np.repeat(np.arange(tokens, dtype=np.int64), topk)
    exp = order.reshape(-1).astype(np.int64)
    perm = np.lexsort((tok, exp))
    src = tok[perm].astype(np.int32)
    counts = np.bincount(exp, minlength=experts).astype(np.int64)
    if shared_expert:
        src = np.concatenate([src, np.arange(tokens, dtype=np.int32)])
        counts = np.concatenate([counts, np.array([tokens], dtype=np.int64)])
    offsets = np.zeros(counts.size + 1, dtype=np.int64)
    np.cumsum(counts, out=offsets[1:])
    return offsets, src


# ---------------------------------------------------------------------------
# Device-side generators (torch, seeded CUDA generator) for multi-GB tensors.
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def device_activations(seed: int, rows: int, cols: int, device="cuda", *, outlier_frac=1e-3,
                       outlier_mult=50.0, row_log10_range=None, std=1.0):
    """bf16 tensor [rows, cols] on the device with the same recipe as activations()."""
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    z = torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32) * std
    if outlier_frac > 0:
        mask = torch.rand((rows, cols), generator=g, device=device) < outlier_frac
        z = torch.where(mask, z * outlier_mult, z)
    if row_log10_range is not None:
        lo, hi = row_log10_range
        u = torch.rand((rows, 1), generator=g, device=device) * (hi - lo) + lo
        z = z * torch.pow(10.0, u)
    return z.to(torch.bfloat16)


def device_weights(seed: int, experts: int, rows: int, cols: int, device="cuda", std=0.02,
                   chunk_experts: int = 8):
    """bf16 tensor [experts * rows, cols] of N(0, std) on the device."""
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = torch.empty((experts * rows, cols), dtype=torch.bfloat16, device=device)
    for e0 in range(0, experts, chunk_experts):
        e1 = min(experts, e0 + chunk_experts)
        z = torch.randn(((e1 - e0) * rows, cols), generator=g, device=device, dtype=torch.float32)
        out[e0 * rows:e1 * rows] = (z * std).to(torch.bfloat16)
    return out
