"""Helpers shared by the GPU tests: move stored inputs to the device, call
the library through its binding, and measure parity against the oracle."""
from __future__ import annotations

import numpy as np
import torch

from sketch_attention_soft_amd import inputs as I

# parity bar: max over heads of the relative Frobenius error
TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 2e-2}


def to_device(a: np.ndarray, dtype: str, dev="cuda") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    if dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.float16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def to_host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def _heads(a: np.ndarray) -> np.ndarray:
    return a.reshape(-1, *a.shape[-2:]) if a.ndim >= 3 else a[None]


def head_relf(x: np.ndarray, ref: np.ndarray, floor_ref: np.ndarray | None = None,
              floor: float = 1e-3) -> float:
    """max over leading (b, h) of ||x - ref||_F / ||ref||_F.

    With floor_ref, the denominator of a head is max(||ref||, floor *
    ||floor_ref||): dQ and dK of a head vanish exactly when every query sees
    a single key (N = 1), and are then compared on the scale of its dV.
    """
    worst = 0.0
    fr = _heads(floor_ref) if floor_ref is not None else None
    for h, (a, b) in enumerate(zip(_heads(x), _heads(ref))):
        nb = np.linalg.norm(b)
        if fr is not None:
            nb = max(nb, floor * np.linalg.norm(fr[h]))
        worst = max(worst, np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))
    return worst


def device_inputs(x: dict, dtype: str) -> dict:
    out = {"W": torch.from_numpy(x["W"]).cuda()}
    for n in ("q", "k", "v", "do"):
        if n in x:
            out[n] = to_device(x[n], dtype)
    return out


def host_inputs(x: dict, dtype: str) -> dict:
    out = {"W": x["W"].astype(np.float64)}
    for n in ("q", "k", "v", "do"):
        if n in x:
            out[n] = I.to_f64(x[n], dtype)
    return out
