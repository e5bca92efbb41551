"""Seeded synthetic workloads: shapes, ALiBi scales and Q/K/V generators.

This module holds only input recipes (no part of the estimator): both the
oracle-based tests and the GPU benchmark draw their inputs from here.

Workload shapes follow the attention layers the Positional-LSH pages evaluate
on ("Positional LSH: Binary Block Matrix Approximation for Attention with
Linear Biases", Key results / experimental validation: Qwen3-0.6B trained from
scratch with s = 10, 20; Mistral-7B fine-tuned, 8k -> 16k length
extrapolation).  Trained weights and activations are not available, so seeded
Gaussians of the same shapes stand in for them.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch


def alibi_sigmas(heads: int) -> List[float]:
    """sigma_h = 1 / m_h with the geometric ALiBi slopes m_h = 2^(-8h/H),
    h = 1..H (head index 0 takes h = 1)."""
    return [float(2.0 ** (8.0 * h / heads)) for h in range(1, heads + 1)]


@dataclass
class Workload:
    name: str
    batch: int
    heads: int
    kv_heads: int
    n: int
    d: int
    dtype: str            # "f32" or "bf16"
    causal: bool
    sigma: List[float]
    s: int
    heavy_tail: bool = False
    input_seed: int = 0
    hash_seed: int = 0
    note: str = ""

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def esz(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def describe(self) -> dict:
        return {"workload": self.name, "batch": self.batch, "heads": self.heads,
                "kv_heads": self.kv_heads, "n": self.n, "d": self.d,
                "dtype": self.dtype, "causal": self.causal, "s": self.s,
                "sigma_min": min(self.sigma), "sigma_max": max(self.sigma),
                "heavy_tail_keys": self.heavy_tail}


def long_context_s(n: int) -> int:
    """s = ceil(4 ln n) for the long-context scaling runs."""
    return int(math.ceil(4.0 * math.log(n)))


def workloads() -> List[Workload]:
    """Every workload, in order: tiny fp32, per-head slopes, Qwen3-0.6B-shaped,
    Mistral-7B-shaped (n = 16384), long-context scaling."""
    out = [
        Workload("tiny-f32-n512", 1, 1, 1, 512, 64, "f32", False, [16.0], 8,
                 note="CPU-checkable fp32 case"),
        Workload("slopes-n4096", 2, 8, 8, 4096, 64, "bf16", False, alibi_sigmas(8), 16),
    ]
    for s in (10, 20):
        out.append(Workload(f"qwen3-0.6b-n8192-s{s}", 4, 16, 8, 8192, 128, "bf16", True,
                            alibi_sigmas(16), s))
    for s in (10, 20, 40):
        out.append(Workload(f"mistral-7b-n16384-s{s}", 1, 32, 8, 16384, 128, "bf16", True,
                            alibi_sigmas(32), s, heavy_tail=True))
    for n in (65536, 131072, 524288):
        out.append(Workload(f"long-n{n}", 1, 8, 8, n, 128, "bf16", True, [64.0] * 8,
                            long_context_s(n)))
    return out


def get(name: str) -> Workload:
    for w in workloads():
        if w.name == name:
            return w
    raise KeyError(name)


def make_qkv(w: Workload, seed: Optional[int] = None, scale_v: bool = False):
    """Q [B,H,n,d], K and V [B,Hkv,n,d] on the CPU, in the workload dtype.

    Recipe: fp32 N(0,1) drawn in the order Q, K, V from a seeded
    torch.Generator; Q and K multiplied by d^(-1/4) (so q.k ~ N(0,1); V stays
    N(0,1) unless scale_v); heavy-tail workloads multiply K at a seeded choice
    of floor(0.05 n) positions per (batch, kv-head) by 4; finally cast with
    round-to-nearest-even to the workload dtype."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.input_seed if seed is None else seed)
    B, H, Hkv, n, d = w.batch, w.heads, w.kv_heads, w.n, w.d
    scale = d ** -0.25
    q = torch.randn((B, H, n, d), generator=g, dtype=torch.float32).mul_(scale)
    k = torch.randn((B, Hkv, n, d), generator=g, dtype=torch.float32).mul_(scale)
    v = torch.randn((B, Hkv, n, d), generator=g, dtype=torch.float32)
    if scale_v:
        v.mul_(scale)
    if w.heavy_tail:
        m = int(math.floor(0.05 * n))
        for b in range(B):
            for hk in range(Hkv):
                idx = torch.randperm(n, generator=g)[:m]
                k[b, hk, idx] *= 4.0
    dt = w.torch_dtype
    return q.to(dt), k.to(dt), v.to(dt)


def sample_rows(n: int, count: int, seed: int = 1234) -> np.ndarray:
    """`count` distinct query rows in [0, n), sorted, from a seeded generator;
    always includes the first and last row (edge blocks)."""
    rng = np.random.default_rng(seed)
    count = min(count, n)
    rows = rng.choice(n, size=count, replace=False)
    rows[0] = 0
    if count > 1:
        rows[1] = n - 1
    return np.unique(rows)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of the values the GPU sees."""
    return t.detach().to("cpu").to(torch.float64).numpy()
