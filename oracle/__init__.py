"""fp64 CPU oracle for RACE attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or executes anything here, and this
package never imports the product.

The arithmetic lives in ``race_oracle.c`` (plain C, fp64, OpenMP over
independent elements only); this module marshals numpy arrays to it.  The
steps it follows are listed, with their sources, in that file's header:
normalise, project on W[L][P][d], tanh, corner softmax at temperature tau,
bucket sums A and B, ratio readout, causal running sums, and the exact
backward of all of it.

Every function takes float arrays of any precision and computes in fp64 on
exactly the values given (a bf16 or fp32 input is widened without rounding).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "race_oracle.c")
_LIB = os.path.join(_HERE, "librace_oracle.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile race_oracle.c into librace_oracle.so next to it (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O3", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared",
             "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        i64, c_int, c_dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.race_oracle_threads.argtypes = [c_int]
        lib.race_oracle_threads.restype = c_int
        lib.race_oracle_hash.argtypes = [dp, i64, c_int, dp, c_int, c_int, c_dbl, c_int, dp, dp]
        lib.race_oracle_hash.restype = c_int
        lib.race_oracle_forward.argtypes = [dp, dp, dp, dp, c_int, c_int, c_dbl, c_int, c_int,
                                            i64, i64, c_int, dp, dp]
        lib.race_oracle_forward.restype = c_int
        lib.race_oracle_forward_backward.argtypes = [dp, dp, dp, dp, dp, c_int, c_int, c_dbl,
                                                     c_int, i64, i64, c_int, dp, dp, dp, dp, dp]
        lib.race_oracle_forward_backward.restype = c_int
        lib.race_oracle_forward_backward_w.argtypes = lib.race_oracle_forward_backward.argtypes + [dp]
        lib.race_oracle_forward_backward_w.restype = c_int
        lib.race_oracle_stream_forward.argtypes = [dp, dp, dp, dp, c_int, c_int, c_dbl, i64, c_int,
                                                   dp, dp, dp]
        lib.race_oracle_stream_forward.restype = c_int
        lib.race_oracle_stream_backward.argtypes = [dp, dp, dp, dp, dp, dp, dp, c_int, c_int,
                                                    c_dbl, i64, c_int, dp, dp, dp, dp, dp]
        lib.race_oracle_stream_backward.restype = c_int
        lib.race_oracle_block_sums.argtypes = [dp, dp, c_int, i64, c_int, dp, c_int, c_int, c_dbl,
                                               dp]
        lib.race_oracle_block_sums.restype = c_int
        _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def threads(n: int = 0) -> int:
    """Set the OpenMP thread count (n > 0) and return the count in use."""
    return int(_load().race_oracle_threads(int(n)))


def _check(err: int, what: str) -> None:
    if err == 1:
        raise ValueError(f"oracle {what}: invalid arguments")
    if err == 2:
        raise MemoryError(f"oracle {what}: out of host memory")
    if err:
        raise RuntimeError(f"oracle {what}: error {err}")


def soft_hash(x, W, tau: float, hard: bool = False):
    """Soft (or hard) bucket assignment of the rows of x[n, d].

    Returns (phi[n, L, R], z[n, L, P]) with z = tanh(W x_hat) and phi the
    softmax over the R = 2^P corners of the logits (1/tau) <z_l, c_r>.
    """
    x = _f64(x)
    W = _f64(W)
    L, P, d = W.shape
    n = x.shape[0]
    assert x.shape == (n, d)
    R = 1 << P
    phi = np.empty((n, L, R))
    z = np.empty((n, L, P))
    _check(_load().race_oracle_hash(_ptr(x), n, d, _ptr(W), L, P, float(tau), int(hard),
                                    _ptr(phi), _ptr(z)), "hash")
    return phi, z


def forward(q, k, v, W, tau: float, causal: bool, hard: bool = False):
    """RACE attention forward on [..., N, d] inputs; returns (o, den) in fp64.

    den is the readout denominator sum_l phi_l(q)^T A_l of every row.
    """
    q, k, v, W = _f64(q), _f64(k), _f64(v), _f64(W)
    assert q.shape == k.shape == v.shape and q.ndim >= 2
    N, d = q.shape[-2:]
    BH = int(np.prod(q.shape[:-2], dtype=np.int64))
    L, P, dw = W.shape
    assert dw == d
    o = np.empty(q.shape)
    den = np.empty(q.shape[:-1])
    _check(_load().race_oracle_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(W), L, P, float(tau),
                                       int(causal), int(hard), BH, N, d, _ptr(o), _ptr(den)),
           "forward")
    return o, den


def forward_backward(q, k, v, g, W, tau: float, causal: bool, with_dw: bool = False):
    """Forward plus the exact backward for upstream gradient g = dL/do.

    Returns (o, den, dq, dk, dv), all fp64, and with with_dw also dW [L, P, d],
    the gradient of the projection (summed over every head and over the rows of
    q and k).  The backward uses this call's own forward results only.
    """
    q, k, v, g, W = _f64(q), _f64(k), _f64(v), _f64(g), _f64(W)
    assert q.shape == k.shape == v.shape == g.shape and q.ndim >= 2
    N, d = q.shape[-2:]
    BH = int(np.prod(q.shape[:-2], dtype=np.int64))
    L, P, dw = W.shape
    assert dw == d
    o = np.empty(q.shape)
    den = np.empty(q.shape[:-1])
    dq = np.empty(q.shape)
    dk = np.empty(q.shape)
    dv = np.empty(q.shape)
    dW = np.empty((L, P, d)) if with_dw else None
    _check(_load().race_oracle_forward_backward_w(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(W), L, P, float(tau), int(causal), BH, N, d,
        _ptr(o), _ptr(den), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dW) if with_dw else None),
        "forward_backward")
    return (o, den, dq, dk, dv, dW) if with_dw else (o, den, dq, dk, dv)


def bucket_sums(k, v, W, tau: float):
    """Per-table bucket sums of the keys of one head ([zh] §2.2 bucket
    aggregation): A[l, r] = sum_j phi_lr(k_j) and B[l, r, :] = sum_j
    phi_lr(k_j) v_j, returned together as AB[l, r, :d] = B and AB[l, r, d] = A
    (fp64, k and v [N, d])."""
    k, v = _f64(k), _f64(v)
    phi, _ = soft_hash(k, W, tau)                      # [N, L, R]
    yv = np.concatenate([v, np.ones((v.shape[0], 1))], axis=1)
    return np.einsum("jlr,jc->lrc", phi, yv)


def walsh_state(k, v, W, tau: float):
    """The streaming state of one head after the keys k (values v), in the
    Walsh basis of each table: S[R l + s, :] = 2^(-P/2) sum_r chi_s(r) AB[l, r, :]
    with chi_s(r) = prod_{p in s} c_rp and AB from bucket_sums (R = 2^P; the
    scale is 1/4 for P = 4).  Since the corner weights are
    phi_lr = prod_p (1 + c_rp t_lp) / 2 (pin P-2), 2^(-P/2) sum_r chi_s(r) phi_lr
    = 2^(-P/2) prod_{p in s} t_lp: S is the sum over the keys of those
    products times [v | 1].  Returns [L * R, d + 1] fp64.

    The readout of step 7 ([zh] §2.2) from it, sum_l phi_l(q)^T AB_l, equals
    psi(q) S with psi_{R l + s}(q) = 2^(-P/2) sum_r chi_s(r) phi_lr(q), because
    sum_s chi_s(r) chi_s(r') = R [r == r']."""
    AB = bucket_sums(k, v, W, tau)                     # [L, R, d + 1]
    L, R, C = AB.shape
    P = R.bit_length() - 1
    r = np.arange(R)
    c = np.where(((r[:, None] >> np.arange(P)[None, :]) & 1) == 1, 1.0, -1.0)   # [R, P]
    s_bits = ((np.arange(R)[:, None] >> np.arange(P)[None, :]) & 1) == 1        # [S, P]
    chi = np.prod(np.where(s_bits[:, None, :], c[None, :, :], 1.0), axis=2)     # [S, R]
    return (2.0 ** (-P / 2) * np.einsum("sr,lrc->lsc", chi, AB)).reshape(L * R, C)


# ---------------------------------------------------------------------------
# Causal streaming over consecutive blocks of one head (the running sums of
# [zh] §2.3 handed from block to block), for sequences too long to hold at
# once.  States are fp64 [d + 1, L R]: row c < d holds the bucket sums B of
# value column c, row d the key mass A (features f = R l + r in table-major
# order), i.e. the transpose of bucket_sums(...).reshape(L R, d + 1).

def new_stream_state(L: int, P: int, d: int) -> np.ndarray:
    """The empty state (no keys / no queries yet)."""
    return np.zeros((d + 1, L << P))


def stream_forward(q, k, v, W, tau: float, state: np.ndarray):
    """Causal forward of one block [n, d] of a head continuing a sequence:
    state holds the sums of every earlier key and is advanced in place
    through the block's last key.  Returns (o, den) of the block's rows."""
    q, k, v, W = _f64(q), _f64(k), _f64(v), _f64(W)
    n, d = q.shape
    L, P, dw = W.shape
    assert k.shape == v.shape == (n, d) and dw == d
    assert state.dtype == np.float64 and state.shape == (d + 1, L << P) and state.flags.c_contiguous
    o = np.empty((n, d))
    den = np.empty(n)
    _check(_load().race_oracle_stream_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(W), L, P,
                                              float(tau), n, d, _ptr(state), _ptr(o), _ptr(den)),
           "stream_forward")
    return o, den


def stream_backward(q, k, v, g, o, den, W, tau: float, key_state: np.ndarray,
                    grad_state: np.ndarray):
    """Causal backward of one block, given the block's own (o, den) from
    stream_forward and g = dL/do.  key_state: the sums of the keys before the
    block (advanced in place through the block); grad_state: the gradient
    sums sum_i phi(q_i) [g_i/m_i | -(g_i . o_i)/m_i]^T of the queries after
    the block (extended in place by the block's queries).  Returns (dq, dk,
    dv) of the block's rows."""
    q, k, v, g, o, den, W = (_f64(a) for a in (q, k, v, g, o, den, W))
    n, d = q.shape
    L, P, dw = W.shape
    assert k.shape == v.shape == g.shape == o.shape == (n, d) and den.shape == (n,) and dw == d
    for st in (key_state, grad_state):
        assert st.dtype == np.float64 and st.shape == (d + 1, L << P) and st.flags.c_contiguous
    dq, dk, dv = np.empty((n, d)), np.empty((n, d)), np.empty((n, d))
    _check(_load().race_oracle_stream_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(o), _ptr(den), _ptr(W), L, P, float(tau), n, d,
        _ptr(key_state), _ptr(grad_state), _ptr(dq), _ptr(dk), _ptr(dv)), "stream_backward")
    return dq, dk, dv


def block_sums(x, y, W, tau: float, state: np.ndarray) -> np.ndarray:
    """state [C, L R] += sum_j phi(x_j) y_j^T over the rows of x [n, d] and
    y [n, C], in row order; returns state.  With y = [v | 1]: a block's
    bucket sums ([zh] §2.2)."""
    x, y, W = _f64(x), _f64(y), _f64(W)
    n, d = x.shape
    L, P, dw = W.shape
    C = y.shape[1]
    assert y.shape == (n, C) and dw == d
    assert state.dtype == np.float64 and state.shape == (C, L << P) and state.flags.c_contiguous
    _check(_load().race_oracle_block_sums(_ptr(x), _ptr(y), C, n, d, _ptr(W), L, P, float(tau),
                                          _ptr(state)), "block_sums")
    return state


def ratio_gradients(g, o, den) -> np.ndarray:
    """D_i = [g_i / m_i | -(g_i . o_i) / m_i] of the ratio readout o = n / m
    (the values the gradient sums carry)."""
    g, o, den = _f64(g), _f64(o), _f64(den)
    return np.concatenate([g / den[:, None], (-(g * o).sum(axis=1) / den)[:, None]], axis=1)
