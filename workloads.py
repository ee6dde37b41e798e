"""Seeded synthetic workloads for C = ReLU(A @ B) with fp16 A[M,K], B[K,N].

This module only draws inputs. It holds none of the method's arithmetic (no
product, no activation, no rounding of results), so both the CPU oracle and the
HIP path can be fed from it without sharing any code of the computation.

The workloads follow the TileLang GEMM example ("Writing high-performance
kernels in TileLang", section "Escribamos un GEMM"): square fp16 problems drawn
from a standard normal, plus a ragged shape (exercising the ceil-divided grid of
that example) and a skinny decode-like shape.

Recipe (every workload): a CPU ``torch.Generator`` seeded with ``seed`` draws A
first and then B in float32, the float32 values are scaled (normal) or mapped
(uniform) and then cast to float16 with round-to-nearest-even. Both sides read
the same fp16 bytes.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dist: str          # "normal" or "uniform" (also "intsmall", "ones")
    scale: float       # standard deviation (normal) or half-width (uniform)
    seed: int = 0

    @property
    def flops(self) -> int:
        """Multiply-adds counted as two operations each: 2*M*N*K."""
        return 2 * self.M * self.N * self.K

    @property
    def min_bytes(self) -> int:
        """Each fp16 operand read once and C written once: 2*(MK + KN + MN)."""
        return 2 * (self.M * self.K + self.K * self.N + self.M * self.N)


# The five workloads. Sizes, distributions and seed as named in each entry.
SQUARE_256 = Workload("gemm_relu_f16_256x256x256_normal", 256, 256, 256, "normal", 1.0)
SQUARE_1024 = Workload("gemm_relu_f16_1024x1024x1024_normal", 1024, 1024, 1024, "normal", 1.0)
SQUARE_4096 = Workload("gemm_relu_f16_4096x4096x4096_normal", 4096, 4096, 4096, "normal", 1.0)
RAGGED = Workload("gemm_relu_f16_1000x1016x1000_uniform", 1000, 1016, 1000, "uniform", 1.0)
SKINNY = Workload("gemm_relu_f16_16x8192x8192_normal0.02", 16, 8192, 8192, "normal", 0.02)

ALL = (SQUARE_256, SQUARE_1024, SQUARE_4096, RAGGED, SKINNY)


def n_shard(w: Workload, ways: int) -> Workload:
    """One GPU's share of `w` when C's columns are split `ways` ways: each GPU
    holds a replica of A and the column panel B[:, N_g] and writes C[:, N_g],
    with no exchange between GPUs (the ReLU is element-wise). Same
    distribution and seed; the shape is M x N/ways x K."""
    if ways < 1 or w.N % ways:
        raise ValueError(f"{w.name}: N = {w.N} does not split {ways} ways")
    n = w.N // ways
    name = w.name.replace(f"_{w.M}x{w.N}x{w.K}_", f"_{w.M}x{n}x{w.K}_") + f"_nsplit{ways}"
    return Workload(name, w.M, n, w.K, w.dist, w.scale, w.seed)


def with_dist(w: Workload, dist: str) -> Workload:
    """The same shape and seed with inputs drawn from `dist` (an ablation of
    the input values: the time of a product depends on its operands' bit
    activity through the power the chip draws). The name records the change."""
    if dist == w.dist:
        return w
    return Workload(f"{w.name}_inputs-{dist}", w.M, w.N, w.K, dist, 1.0, w.seed)


# One GPU's share of the headline square problem and of the skinny one under
# 2-, 4- and 8-way column splits.
SHARDS = tuple(n_shard(w, ways) for w in (SQUARE_4096, SKINNY) for ways in (2, 4, 8))
BY_NAME = {w.name: w for w in ALL + SHARDS}


def _draw(gen: torch.Generator, shape, dist: str, scale: float) -> torch.Tensor:
    if dist == "normal":
        x = torch.randn(shape, generator=gen, dtype=torch.float32)
        if scale != 1.0:
            x = x * scale
    elif dist == "uniform":
        # torch.rand is [0, 1); mapped to [-scale, scale)
        x = torch.rand(shape, generator=gen, dtype=torch.float32) * (2.0 * scale) - scale
    elif dist == "intsmall":
        # integers in {-2,...,2}: every partial sum of K <= 4096 such products
        # stays below 2**24 and is therefore exact in fp32 in any order
        x = torch.randint(-2, 3, shape, generator=gen).to(torch.float32)
    elif dist == "ones":
        # every element equal to `scale`: operands whose bits never change
        x = torch.full(shape, float(scale), dtype=torch.float32)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return x.to(torch.float16)


def make_inputs(M: int, N: int, K: int, dist: str = "normal", scale: float = 1.0,
                seed: int = 0) -> tuple[torch.Tensor, torch.Tensor]:
    """CPU fp16 tensors A[M,K], B[K,N], contiguous row-major. A is drawn first."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    a = _draw(gen, (M, K), dist, scale).contiguous()
    b = _draw(gen, (K, N), dist, scale).contiguous()
    return a, b


def workload_inputs(w: Workload) -> tuple[torch.Tensor, torch.Tensor]:
    return make_inputs(w.M, w.N, w.K, w.dist, w.scale, w.seed)


def as_u16(t: torch.Tensor) -> np.ndarray:
    """The raw fp16 bit patterns of a CPU fp16 tensor as a uint16 numpy array."""
    assert t.dtype == torch.float16 and t.device.type == "cpu"
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def from_u16(x: np.ndarray) -> torch.Tensor:
    """CPU fp16 tensor holding the given uint16 bit patterns."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint16).view(np.int16)).view(torch.float16)
