"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module only draws random numbers and converts storage formats (fp32 <->
bf16/fp16 bit patterns). It contains none of the quantizer's arithmetic: no
scales, distances, codebooks, encodings or error measures.

The pages measure on trained Mixture-of-Experts expert weights (Kimi-Linear,
Kimi K3, DeepSeek-V4.1-Flash, GLM-5.3-Flash), which are not available here.
The generators below stand in for them with the expert shape the pages imply
(2048 x 7168 per w1 matrix) and heavy-tailed, per-row-scaled entries.

Recipes (numpy PCG64 unless a torch device generator is requested):
  * gaussian_rows(rows, cols, seed): w_ij = z_ij * exp(0.5 * g_i), g, z ~ N(0,1);
    the row factors g are drawn first, then z in row-major order.
  * student_t_rows(rows, cols, seed): w_ij = 0.02 * exp(0.3 * g_i) * t_ij,
    t ~ Student-t(nu=5); row factors first, then t row-major; stored as bf16
    (round-to-nearest-even from fp32).
  * expert seed for expert e of configuration c: 1000 * c + e.
"""
from __future__ import annotations

import numpy as np

EXPERT_ROWS = 2048
EXPERT_COLS = 7168


def expert_seed(cfg: int, expert: int) -> int:
    return 1000 * int(cfg) + int(expert)


# ---------------------------------------------------------------- formats --
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


# ---------------------------------------------------------------- weights --
def gaussian_rows(rows: int, cols: int, seed: int = 0, row_sigma: float = 0.5) -> np.ndarray:
    """fp32 [rows, cols]: N(0,1) entries times a per-row lognormal(0, row_sigma) factor."""
    rng = np.random.Generator(np.random.PCG64(seed))
    g = rng.standard_normal(rows)
    z = rng.standard_normal((rows, cols))
    return (z * np.exp(row_sigma * g)[:, None]).astype(np.float32)


def student_t_rows_f32(rows: int, cols: int, seed: int, nu: float = 5.0,
                       scale: float = 0.02, row_sigma: float = 0.3) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    g = rng.standard_normal(rows)
    t = rng.standard_t(nu, (rows, cols))
    return (scale * np.exp(row_sigma * g)[:, None] * t).astype(np.float32)


def student_t_rows_bf16(rows: int, cols: int, seed: int, **kw) -> np.ndarray:
    """bf16 bit patterns (uint16) of the Student-t expert recipe."""
    return f32_to_bf16_bits(student_t_rows_f32(rows, cols, seed, **kw))


def student_t_expert_torch(seed: int, rows: int = EXPERT_ROWS, cols: int = EXPERT_COLS,
                           device="cuda", nu: float = 5.0, scale: float = 0.02,
                           row_sigma: float = 0.3, out=None):
    """Same recipe drawn with torch's generator on `device` (used for the large,
    full-layer workloads, where numpy would take minutes). Returns bf16 [rows, cols]
    (written into `out` when given)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    g = torch.randn(rows, device=device, generator=gen, dtype=torch.float32)
    z = torch.randn(rows, cols, device=device, generator=gen, dtype=torch.float32)
    # Student-t(nu) = z / sqrt(chi2_nu / nu), chi2_nu = 2 * Gamma(nu / 2, 1)
    conc = torch.full((rows, cols), nu / 2.0, device=device, dtype=torch.float32)
    gam = torch._standard_gamma(conc, generator=gen)
    t = z / torch.sqrt(2.0 * gam / nu)
    w = (scale * torch.exp(row_sigma * g))[:, None] * t
    if out is None:
        return w.to(torch.bfloat16)
    out.copy_(w.to(torch.bfloat16))
    return out


# ------------------------------------------------------ sampling / routing --
def sample_experts(n_total: int, n_sample: int, seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.sort(rng.choice(n_total, size=n_sample, replace=False)).astype(np.int64)


def forgy_init(n_vectors: int, k: int, stages: int, seed: int) -> np.ndarray:
    """int64 [stages, k]: for each stage, k distinct training-vector indices drawn
    uniformly without replacement (the Lloyd initial centroids)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = np.empty((stages, k), dtype=np.int64)
    for t in range(stages):
        out[t] = rng.choice(n_vectors, size=k, replace=False)
    return out


def activations_f16(ntok: int, cols: int, seed: int) -> np.ndarray:
    """fp16 bit patterns [ntok, cols] of x ~ N(0, 1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal((ntok, cols)).astype(np.float16).view(np.uint16)


def routing(ntok: int, n_experts: int, topk: int, seed: int) -> np.ndarray:
    """int32 [ntok, topk]: per token, topk distinct experts uniform without replacement."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.stack([rng.choice(n_experts, size=topk, replace=False) for _ in range(ntok)]
                    ).astype(np.int32).reshape(ntok, topk)
