"""Helpers shared by the GPU tests: host<->device conversion and the error metric.

Error metric (the pages state no tolerance; the method's statement fixes
max relative error 5e-3 for f16/f32 inputs and 2e-2 for bf16): per output
tensor X against the oracle R, err = max|X - R| / max|R| (normwise, infinity
norm). Elementwise |X - R| / |R| is ill-posed here: outputs have sign changes
and many near-zero entries, and a 16-bit result cannot be relatively accurate
there.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

TOL = {"f32": 5e-3, "f16": 5e-3, "bf16": 2e-2}
# fp32 inputs run fp32 MFMA: hold them to a much tighter bar as well.
TIGHT = {"f32": 1e-5}
TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def to_device(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Storage array (synth format) to a device tensor with the same bits."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device)


def to_storage(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Device tensor back to the synth storage format (bit-exact)."""
    t = t.detach().cpu()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def decode(t: torch.Tensor, dtype: str) -> np.ndarray:
    return oracle.decode(to_storage(t, dtype), dtype)


def max_rel_err(x: np.ndarray, ref: np.ndarray) -> float:
    scale = float(np.max(np.abs(ref)))
    if scale == 0.0:
        return float(np.max(np.abs(x)))
    return float(np.max(np.abs(np.asarray(x, dtype=np.float64) - ref)) / scale)


def split_state(state: torch.Tensor, B: int, H: int, D: int, Dv: int | None = None):
    """fp32 state buffer -> (S [B,H,D,Dv], z [B,H,D]) as float64 numpy."""
    Dv = D if Dv is None else Dv
    s = state.detach().cpu().numpy().astype(np.float64)
    n = B * H
    return s[: n * D * Dv].reshape(B, H, D, Dv), s[n * D * Dv: n * D * Dv + n * D].reshape(B, H, D)


def bytes_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))
