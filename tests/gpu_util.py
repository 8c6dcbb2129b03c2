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


# per-row gate: a row is compared with its reference relative to its own norm,
# floored at ROW_FLOOR times the root mean square row norm of its head; the
# bar is ten times the Frobenius bar, so rounding passes and a row that is
# wholly wrong (error ~ 1) does not
ROW_TOL = {k: 10 * v for k, v in TOL.items()}
ROW_FLOOR = 0.05
# dQ and dK rows are differences of nearly equal terms for some rows (a query
# whose keys carry similar values: early causal rows above all), so their
# rounding is measured against a quarter of the head's RMS row norm; a row
# that is wholly wrong still scores about 1 or more
GRAD_FLOOR = 0.25


def row_errors(x: np.ndarray, ref: np.ndarray, floor: float = ROW_FLOOR,
               vanishing: tuple = ()) -> np.ndarray:
    """Per-row relative errors ||x_i - ref_i|| / max(||ref_i||, floor rms_h),
    rows over the last axis, rms_h over the rows of each leading (b, h).

    vanishing: row indices (within every head) whose exact value is zero for
    any input -- the causal dQ of row 0, whose output o_0 = v_0 does not
    depend on q_0 -- so that the computed row is rounding noise; they are
    measured on the head's scale (floor 1)."""
    xs, rs = _heads(x), _heads(ref)
    out = []
    for a, b in zip(xs, rs):
        a = a.reshape(a.shape[0], -1) if a.ndim > 1 else a[:, None]
        b = b.reshape(b.shape[0], -1) if b.ndim > 1 else b[:, None]
        nb = np.linalg.norm(b, axis=1)
        rms = np.sqrt(np.mean(nb * nb)) if nb.size else 0.0
        fl = np.full(nb.shape, floor * rms)
        for i in vanishing:
            if i < fl.size:
                fl[i] = rms
        den = np.maximum(nb, fl)
        den[den == 0] = 1.0
        out.append(np.linalg.norm(a - b, axis=1) / den)
    return np.concatenate(out) if out else np.zeros(0)


def row_report(name: str, e: np.ndarray) -> str:
    if e.size == 0:
        return f"rows_{name}: none"
    return (f"rows_{name}: max={e.max():.2e} (row {int(np.argmax(e))}) "
            f"p99={np.percentile(e, 99):.2e} median={np.median(e):.2e}")
