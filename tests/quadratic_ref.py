"""Brute-force O(N^2) closed forms used to pin the oracle (small N only).

Independent of the oracle's code: written from the closed form of the soft
RACE kernel and from the sharpened angular kernel, not from the streaming
algorithm.

Closed form of the soft kernel.  The corner softmax of one table factorises
over hyperplanes, softmax_r((1/tau) <z, c_r>) = prod_p sigmoid(2 c_rp z_p / tau),
and sigmoid(2y) = (1 + tanh y)/2, so with t = tanh(z / tau)

    kappa(q, k) = sum_l sum_r phi_lr(q) phi_lr(k) = sum_l prod_p (1 + t_lp(q) t_lp(k)) / 2

and the RACE readout of the pages' ratio estimator is the kernel-weighted
average o_i = sum_j kappa_ij v_j / sum_j kappa_ij over the visible keys j.
"""
from __future__ import annotations

import numpy as np


def normalise(x: np.ndarray) -> np.ndarray:
    n = np.sqrt((x * x).sum(-1, keepdims=True))
    return x / np.maximum(n, 1e-12)


def t_features(x: np.ndarray, W: np.ndarray, tau: float) -> np.ndarray:
    """t[n, L, P] = tanh(tanh(W x_hat) / tau)."""
    u = np.einsum("lpd,nd->nlp", W, normalise(x))
    return np.tanh(np.tanh(u) / tau)


def soft_kernel(q: np.ndarray, k: np.ndarray, W: np.ndarray, tau: float) -> np.ndarray:
    """kappa[i, j] for rows q[i], k[j]."""
    tq, tk = t_features(q, W, tau), t_features(k, W, tau)
    f = (1.0 + tq[:, None, :, :] * tk[None, :, :, :]) / 2.0  # [Nq, Nk, L, P]
    return f.prod(-1).sum(-1)


def kernel_attention(kappa: np.ndarray, v: np.ndarray, causal: bool):
    """(o, den) of the kernel-weighted average; causal keeps j <= i."""
    if causal:
        kappa = np.tril(kappa)
    den = kappa.sum(1)
    return kappa @ v / den[:, None], den


def soft_race_attention(q, k, v, W, tau, causal):
    return kernel_attention(soft_kernel(q, k, W, tau), v, causal)


def angular_attention(q, k, v, gamma, causal=False):
    """Sharpened angular kernel (1 - acos(q_hat . k_hat)/pi)^gamma attention."""
    c = np.clip(normalise(q) @ normalise(k).T, -1.0, 1.0)
    return kernel_attention((1.0 - np.arccos(c) / np.pi) ** gamma, v, causal)
