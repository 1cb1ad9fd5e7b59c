"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the
bench.

Nothing here computes any step of the bucketing method: it only draws numbers.
Every tensor (replica r, micro-step t, variable v) has its own seed, so any one
of them can be regenerated on its own.

Seed recipe: ``seed = cfg * 10**9 + t * 10**7 + r * 10**4 + v``. A whole
replica's set of step gradients drawn as one flat buffer (``flat_step``) takes
the variable slot ``FLAT_V`` = 9999, which no model here reaches.
Values: N(0, sigma) with sigma = 1e-3 (the standard deviation), drawn in fp32
with ``torch.randn`` from ``torch.Generator(device).manual_seed(seed)`` and
scaled by sigma. The CPU and the GPU generators produce different streams for
the same seed, so a consumer that compares two implementations always hands both
the same generated buffers (host arrays, or a host snapshot of device buffers).
"""
from __future__ import annotations

import math
from typing import List, Sequence

import numpy as np
import torch

SIGMA = 1e-3


def seed_of(cfg: int, r: int, v: int, t: int = 0) -> int:
    if not (0 <= v < 10**4 and 0 <= r < 10**3 and 0 <= t < 100):
        raise ValueError("seed fields out of range")
    return cfg * 10**9 + t * 10**7 + r * 10**4 + v


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(seed: int, numel: int, device="cpu", sigma: float = SIGMA,
           out: torch.Tensor | None = None) -> torch.Tensor:
    """fp32 N(0, sigma) of ``numel`` elements (flat). With ``out`` the values
    are written into that fp32 tensor (any shape with ``numel`` elements)."""
    g = _gen(seed, device)
    if out is None:
        x = torch.randn(numel, generator=g, device=device, dtype=torch.float32)
        return x.mul_(sigma)
    flat = out.view(-1)
    if flat.numel() != numel or out.dtype != torch.float32:
        raise ValueError("out must be fp32 with numel elements")
    torch.randn(numel, generator=g, device=out.device, dtype=torch.float32, out=flat)
    return flat.mul_(sigma)


FLAT_V = 9999


def flat_step(cfg: int, r: int, t: int, numel: int, device="cpu", dtype=torch.bfloat16) -> torch.Tensor:
    """Every variable's step gradient of replica r at micro-step t as one flat
    N(0, sigma) draw of ``numel`` (the model's total) elements, rounded to
    ``dtype``; variable v is the slice at the prefix sum of the numels before
    it. Three device dispatches per (r, t) instead of three per tensor."""
    x = normal(seed_of(cfg, r, FLAT_V, t), numel, device)
    return x if dtype == torch.float32 else x.to(dtype)


def flat_views(flat: torch.Tensor, numels: Sequence[int]) -> List[torch.Tensor]:
    """Per-variable views (flat slices) of one flat_step buffer."""
    out, off = [], 0
    for n in numels:
        out.append(flat[off:off + n])
        off += n
    return out


def normal_bf16(seed: int, numel: int, device="cpu", sigma: float = SIGMA) -> torch.Tensor:
    """N(0, sigma) drawn in fp32, then rounded to bf16 (round to nearest even)."""
    return normal(seed, numel, device, sigma).to(torch.bfloat16)


def grad_set(cfg: int, numels: Sequence[int], R: int, t: int = 0, device="cpu") -> List[List[torch.Tensor]]:
    """R replicas x P variables of fp32 N(0, 1e-3) gradients, flat tensors."""
    return [[normal(seed_of(cfg, r, v, t), n, device) for v, n in enumerate(numels)]
            for r in range(R)]


def to_numpy(sets: List[List[torch.Tensor]]) -> List[List[np.ndarray]]:
    return [[x.detach().to("cpu").numpy().copy() for x in row] for row in sets]


# ---- nn.Linear(10, 10) example inputs -------------------------------------

def linear10_init(r: int):
    """Rank r's own initial (W [10,10], b [10]) from seed 1000 + r, uniform in
    (-1/sqrt(10), 1/sqrt(10)) as nn.Linear's default initialisation bound."""
    g = _gen(1000 + r, "cpu")
    k = 1.0 / math.sqrt(10.0)
    W = torch.empty(10, 10, dtype=torch.float32).uniform_(-k, k, generator=g)
    b = torch.empty(10, dtype=torch.float32).uniform_(-k, k, generator=g)
    return W, b


def linear10_batch(r: int) -> torch.Tensor:
    """Rank r's input batch randn(20, 10) from seed 2000 + r."""
    return torch.randn(20, 10, generator=_gen(2000 + r, "cpu"), dtype=torch.float32)


# ---- small random cases for tests -------------------------------------------

def random_numels(seed: int, P: int, lo: int = 1, hi: int = 5000) -> List[int]:
    rng = np.random.default_rng(seed)
    return [int(x) for x in rng.integers(lo, hi + 1, size=P)]


def dyadic(seed: int, shape, lim: int = 1 << 10, scale_exp: int = -12) -> np.ndarray:
    """fp32 values k * 2**scale_exp with integer k uniform in [-lim, lim]."""
    rng = np.random.default_rng(seed)
    k = rng.integers(-lim, lim + 1, size=shape)
    return (k.astype(np.float64) * 2.0 ** scale_exp).astype(np.float32)


def permutation(seed: int, n: int) -> List[int]:
    rng = np.random.default_rng(seed)
    return [int(x) for x in rng.permutation(n)]
