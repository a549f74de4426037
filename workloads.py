"""Seeded synthetic inputs for SGEMM, shared by the tests, the benchmark and
the oracle.  This module draws numbers and lays them out in memory; it holds
none of the product's arithmetic.

Distributions (all drawn in float32 on the CPU with ``torch.Generator``):

* ``uniform``  -- i.i.d. uniform on [-1, 1), made as ``2*U - 1`` with U the
  float32 uniform on [0, 1).  Both steps are exact in binary32, so every value
  lies in [-1, 1 - 2^-23] and is a multiple of 2^-23.
* ``normal``   -- i.i.d. N(0, std^2): float32 standard normals times ``std``.
* ``integer``  -- i.i.d. uniform on {-4, ..., 4}.  With |entries| <= 4 every
  partial sum of a product is an integer of magnitude <= 16 K, exact in fp32
  for K <= 2^20, so any summation order gives the same bits.

The pages generate synthetic random matrices only (``torch.randn`` with a fixed
seed in "GEMM from naive to tiled", section 十一.2); there is no public dataset
behind any workload here.

Memory layout: row-major with an explicit leading dimension ``ld >= cols``.
The gap ``[cols, ld)`` of every row is filled with a sentinel (NaN by
default), so a kernel that reads padding poisons its result.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def draw(rows: int, cols: int, kind: str, seed: int, std: float = 1.0) -> torch.Tensor:
    """A contiguous (rows, cols) float32 CPU tensor of the given distribution."""
    g = _gen(seed)
    if kind == "uniform":
        u = torch.rand((rows, cols), generator=g, dtype=torch.float32)
        return u * 2.0 - 1.0
    if kind == "normal":
        x = torch.randn((rows, cols), generator=g, dtype=torch.float32)
        return x * float(std) if std != 1.0 else x
    if kind == "integer":
        return torch.randint(-4, 5, (rows, cols), generator=g, dtype=torch.int32).to(torch.float32)
    raise ValueError(f"unknown distribution {kind!r}")


def with_ld(x: torch.Tensor, ld: int, pad_value: float = float("nan")) -> torch.Tensor:
    """Copy ``x`` (rows, cols) into a (rows, ld) buffer whose gap holds ``pad_value``;
    returns the (rows, cols) view with row stride ``ld``."""
    rows, cols = x.shape
    if ld < cols:
        raise ValueError(f"ld={ld} < cols={cols}")
    if ld == cols:
        return x.contiguous()
    buf = torch.full((rows, ld), pad_value, dtype=torch.float32)
    buf[:, :cols] = x
    return buf[:, :cols]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One SGEMM problem: shapes, leading dimensions and input recipe."""
    name: str
    M: int
    N: int
    K: int
    lda: int
    ldb: int
    ldc: int
    a_kind: str
    b_kind: str
    a_std: float = 1.0
    b_std: float = 1.0
    seed_base: int = 0

    def a(self, kind: Optional[str] = None) -> torch.Tensor:
        return with_ld(draw(self.M, self.K, kind or self.a_kind, self.seed_base + 0, self.a_std), self.lda)

    def b(self, kind: Optional[str] = None) -> torch.Tensor:
        return with_ld(draw(self.K, self.N, kind or self.b_kind, self.seed_base + 1, self.b_std), self.ldb)

    def with_integers(self) -> "Workload":
        return dataclasses.replace(self, name=self.name + "_int", a_kind="integer", b_kind="integer")


def _make(cid: int, name: str, M: int, N: int, K: int, dist: str,
          lda: Optional[int] = None, ldb: Optional[int] = None, ldc: Optional[int] = None) -> Workload:
    if dist == "uniform":
        a_kind = b_kind = "uniform"
        a_std = b_std = 1.0
    elif dist == "linear":
        a_kind = b_kind = "normal"
        a_std, b_std = 1.0, 1.0 / math.sqrt(K)
    else:
        raise ValueError(dist)
    return Workload(name=name, M=M, N=N, K=K, lda=lda or K, ldb=ldb or N, ldc=ldc or N,
                    a_kind=a_kind, b_kind=b_kind, a_std=a_std, b_std=b_std, seed_base=1000 * cid)


# The benchmark configurations.  Seeds are 1000*id (+0 for A, +1 for B).
CONFIGS = {
    w.name: w for w in [
        _make(0, "sgemm_256", 256, 256, 256, "uniform"),
        _make(1, "sgemm_4096", 4096, 4096, 4096, "uniform"),
        # odd leading dimensions: rows start on 4-byte boundaries only
        _make(2, "ragged_4097x3001x2049", 4097, 3001, 2049, "uniform"),
        _make(3, "linear_8192x4096x11008", 8192, 11008, 4096, "linear"),
        _make(4, "linear_skinny_16x4096x11008", 16, 11008, 4096, "linear"),
        _make(5, "longk_512x512x65536", 512, 512, 65536, "uniform"),
    ]
}
