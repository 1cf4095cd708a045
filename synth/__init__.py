"""Seeded synthetic inputs for bidirectional linear attention.

This module is shared by the oracle tests, the GPU parity tests and the
benchmark. It holds none of the method's arithmetic: it only draws seeded
normal samples and rounds them to a storage format, so that the CPU oracle and
the GPU kernels consume exactly the same quantised values.

Storage formats (numpy side):
  "f32"  -> numpy.float32
  "f16"  -> numpy.float16 (round-to-nearest-even cast by numpy)
  "bf16" -> numpy.uint16 holding bfloat16 bit patterns (round-to-nearest-even)

The workloads mirror the shapes the FBi-LA page benchmarks (B8-H16-D64 over a
sweep of sequence lengths, "Benchmarks" section of the FBi-LA README) plus a
wide-head and a long-sequence case; the pages name no dataset, so every tensor
is a seeded normal draw.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

DTYPES = ("f32", "f16", "bf16")
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the bits.

    Inputs are finite normal draws, so no NaN handling is needed.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def to_storage(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round a float32 array to the storage format named by ``dtype``."""
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "f16":
        return x32.astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(f"unknown dtype {dtype!r}")


def normal(shape, seed: int, sigma: float, dtype: str) -> np.ndarray:
    """Seeded N(0, sigma^2) draw in float32, then rounded to ``dtype`` storage."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return to_storage(x, dtype)


@dataclass(frozen=True)
class Workload:
    """One synthetic problem: Q and K [B, H, T, D], V and dO [B, H, T, Dv]
    (Dv = 0 stands for Dv = D), dtype, distribution, mode."""

    name: str
    B: int
    H: int
    T: int
    D: int
    dtype: str
    sigma: float = 1.0
    simple: bool = False
    eps: float = 1e-6
    bwd: bool = True
    seed: int = 0
    Dv: int = 0
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def dv(self) -> int:
        """Head size of V, O, dO and dV."""
        return self.Dv or self.D

    @property
    def shape(self):
        """Shape of Q, K, dQ, dK."""
        return (self.B, self.H, self.T, self.D)

    @property
    def shape_v(self):
        """Shape of V, O, dO, dV."""
        return (self.B, self.H, self.T, self.dv)

    @property
    def numel(self) -> int:
        """Elements of one Q-side tensor."""
        return self.B * self.H * self.T * self.D

    @property
    def numel_v(self) -> int:
        """Elements of one V-side tensor."""
        return self.B * self.H * self.T * self.dv

    @property
    def elem_bytes(self) -> int:
        return ELEM_BYTES[self.dtype]


def make_inputs(w: Workload, with_grad: bool | None = None) -> dict:
    """Q, K, V (and dO when the workload has a backward) in storage format.

    Seeds are w.seed + 0..3 for Q, K, V, dO. dO is always N(0, 1).
    """
    with_grad = w.bwd if with_grad is None else with_grad
    out = {
        "q": normal(w.shape, w.seed + 0, w.sigma, w.dtype),
        "k": normal(w.shape, w.seed + 1, w.sigma, w.dtype),
        "v": normal(w.shape_v, w.seed + 2, w.sigma, w.dtype),
    }
    if with_grad:
        out["do"] = normal(w.shape_v, w.seed + 3, 1.0, w.dtype)
    return out


# The five workloads: a tiny fp32 case, the B8-H16-D64 forward at T=4096, the
# headline B8-H16-T16384-D64 fp16 forward+backward, a D=128 bf16 case and a
# long-sequence simple-mode case. Seed base = 1000 * position.
WORKLOADS = {
    "B1-H2-T128-D64-f32": Workload("B1-H2-T128-D64-f32", 1, 2, 128, 64, "f32",
                                   bwd=False, seed=1000),
    "B8-H16-T4096-D64-f16": Workload("B8-H16-T4096-D64-f16", 8, 16, 4096, 64, "f16",
                                     bwd=False, seed=2000),
    "B8-H16-T16384-D64-f16": Workload("B8-H16-T16384-D64-f16", 8, 16, 16384, 64, "f16",
                                      bwd=True, seed=3000),
    "B8-H32-T8192-D128-bf16": Workload("B8-H32-T8192-D128-bf16", 8, 32, 8192, 128, "bf16",
                                       sigma=0.5, bwd=True, seed=4000),
    "B2-H8-T262144-D64-bf16-simple": Workload("B2-H8-T262144-D64-bf16-simple", 2, 8, 262144, 64,
                                              "bf16", simple=True, bwd=True, seed=5000),
}

HEADLINE = "B8-H16-T16384-D64-f16"


# Measurement shapes for the other head sizes: the headline's batch, heads,
# length and dtype with D (of Q, K) and Dv (of V) changed. Seed base 6000 + 100 i.
HEAD_SIZE_WORKLOADS = {
    w.name: w for w in (
        Workload("B8-H16-T16384-D32-f16", 8, 16, 16384, 32, "f16", seed=6000),
        Workload("B8-H16-T16384-D96-f16", 8, 16, 16384, 96, "f16", seed=6100),
        Workload("B8-H16-T16384-D128-f16", 8, 16, 16384, 128, "f16", seed=6200),
        Workload("B8-H16-T16384-D64-Dv128-f16", 8, 16, 16384, 64, "f16", seed=6300, Dv=128),
        Workload("B8-H16-T16384-D128-Dv64-f16", 8, 16, 16384, 128, "f16", seed=6400, Dv=64),
        Workload("B8-H16-T16384-D32-Dv128-f16", 8, 16, 16384, 32, "f16", seed=6500, Dv=128),
        # head size 256: the headline's bytes per tensor (T D per head) at a quarter of its length
        Workload("B8-H16-T4096-D256-f16", 8, 16, 4096, 256, "f16", seed=6600),
        # the headline shape with fp32 elements (fp32 MFMA throughout)
        Workload("B8-H16-T16384-D64-f32", 8, 16, 16384, 64, "f32", seed=6700),
    )
}
