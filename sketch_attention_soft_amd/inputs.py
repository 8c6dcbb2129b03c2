"""Seeded synthetic inputs for RACE attention workloads.

This module is shared by the tests, the benchmark and the smoke check, and it
feeds both the HIP path and the oracle the same bytes.  It holds none of the
method's arithmetic: only random draws, the per-row L2 normalisation that the
input recipe applies to Q and K, rounding to the storage dtype, and bf16 / fp16
bit conversions.

Recipe (one counter-based Philox stream per tensor, fixed order W, Q, K, V,
dO; rows generated in blocks of ``ROWS_PER_BLOCK`` so that any block can be
reproduced on its own):

* every tensor is drawn i.i.d. N(0, 1) in fp32;
* rows of Q and K are L2-normalised in fp64, rounded to fp32, and for bf16
  or fp16 workloads rounded again to that type with round-to-nearest-even;
* V and dO are rounded to the storage dtype the same way;
* W[L, P, d] stays fp32;
* the counter of block b of stream s is (0, b, 0, 0) under key
  seed * 16 + s, so generation is identical on every machine.

Un-normalised rows (``row_scale=True``, a test recipe, not a workload's):
after the normalisation each row of Q and K is multiplied by 10**(6u - 3),
u ~ U(0, 1), a log-uniform factor in [1e-3, 1e3], and with probability 1/64
by zero instead; u and the zero draw come from the stream ``STREAM_SCALE +
s`` of the same block, so the rows' directions are those of the normalised
recipe.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROWS_PER_BLOCK = 1 << 16

STREAM_W, STREAM_Q, STREAM_K, STREAM_V, STREAM_DO = range(5)
STREAM_SCALE = 8  # + the stream of the scaled tensor (Q or K)
ZERO_ROW_P = 1.0 / 64


@dataclasses.dataclass(frozen=True)
class Workload:
    """One RACE attention workload: shapes, hyper-parameters and passes."""
    name: str
    B: int
    H: int
    N: int
    d: int
    L: int
    P: int
    tau: float
    causal: bool
    dtype: str  # "f32", "bf16" or "f16": storage type of Q, K, V, O, dO, dQ, dK, dV
    backward: bool
    chunk: int  # 0: the library chooses
    seed: int

    @property
    def tokens(self) -> int:
        return self.B * self.H * self.N


# The five workloads this library is specified and measured on.
WORKLOADS = {
    "noncausal_fwd_n1k_f32": Workload("noncausal_fwd_n1k_f32", 1, 1, 1024, 64, 8, 4, 1.0,
                                      False, "f32", False, 0, 1001),
    "causal_h8_n64k_f32": Workload("causal_h8_n64k_f32", 1, 8, 65536, 64, 32, 4, 1.0,
                                   True, "f32", True, 256, 1002),
    "causal_b4h16_n16k_bf16": Workload("causal_b4h16_n16k_bf16", 4, 16, 16384, 64, 64, 4, 0.5,
                                       True, "bf16", True, 0, 1003),
    "causal_n4m_bf16": Workload("causal_n4m_bf16", 1, 1, 4194304, 64, 32, 4, 1.0,
                                True, "bf16", True, 0, 1004),
    "causal_n75m_bf16": Workload("causal_n75m_bf16", 1, 1, 75_000_000, 64, 16, 4, 1.0,
                                 True, "bf16", True, 0, 1005),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round-to-nearest-even); returns uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to fp32 exactly."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of a stored tensor (fp32 array, bf16 or fp16 bits)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    if dtype == "f16":
        return np.ascontiguousarray(a, dtype=np.uint16).view(np.float16).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _gen(seed: int, stream: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=seed * 16 + stream,
                                                counter=[0, block, 0, 0]))


def _rows(seed: int, stream: int, r0: int, r1: int, d: int, normalise: bool,
          scale: bool = False) -> np.ndarray:
    """fp32 rows [r0, r1) of a stream (blocks are drawn whole, then sliced)."""
    out = np.empty((r1 - r0, d), dtype=np.float32)
    b0, b1 = r0 // ROWS_PER_BLOCK, (r1 - 1) // ROWS_PER_BLOCK
    for b in range(b0, b1 + 1):
        blk = _gen(seed, stream, b).standard_normal((ROWS_PER_BLOCK, d), dtype=np.float32)
        if normalise:
            x = blk.astype(np.float64)
            x /= np.sqrt((x * x).sum(axis=1, keepdims=True))
            if scale:
                gs = _gen(seed, STREAM_SCALE + stream, b)
                f = 10.0 ** (6.0 * gs.random(ROWS_PER_BLOCK) - 3.0)
                f[gs.random(ROWS_PER_BLOCK) < ZERO_ROW_P] = 0.0
                x *= f[:, None]
            blk = x.astype(np.float32)
        lo = max(r0, b * ROWS_PER_BLOCK)
        hi = min(r1, (b + 1) * ROWS_PER_BLOCK)
        out[lo - r0:hi - r0] = blk[lo - b * ROWS_PER_BLOCK:hi - b * ROWS_PER_BLOCK]
    return out


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f16":  # IEEE half, round-to-nearest-even (numpy's cast)
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)
    return x


def stream_rows(seed: int, stream: int, r0: int, r1: int, d: int, dtype: str) -> np.ndarray:
    """Rows [r0, r1) of one stream in storage form (Q and K normalised): for a
    single-head workload, rows r0..r1 of that tensor, without drawing the rest."""
    return _store(_rows(seed, stream, r0, r1, d, stream in (STREAM_Q, STREAM_K)), dtype)


def make_w(seed: int, L: int, P: int, d: int) -> np.ndarray:
    """Projection tensor W[L, P, d], fp32 N(0, 1)."""
    return _gen(seed, STREAM_W, 0).standard_normal((L, P, d), dtype=np.float32)


def make_tensor(seed: int, stream: int, BH: int, N: int, d: int, dtype: str,
                n_rows: int | None = None, threads: int = 8, row_scale: bool = False) -> np.ndarray:
    """Rows of one input tensor [BH, n_rows, d] in storage form.

    Head h of a [BH, N, d] tensor occupies stream rows [h*N, (h+1)*N); only the
    first ``n_rows`` (default N) rows of each head are produced, so a prefix of
    a long workload is bit-identical to the same rows of the full tensor.
    row_scale: Q and K rows scaled as the module docstring describes.
    """
    n = N if n_rows is None else n_rows
    normalise = stream in (STREAM_Q, STREAM_K)
    scale = row_scale and normalise
    out = np.empty((BH, n, d), dtype=np.uint16 if dtype in ("bf16", "f16") else np.float32)
    jobs = []
    for h in range(BH):
        for r in range(0, n, ROWS_PER_BLOCK):
            jobs.append((h, r, min(n, r + ROWS_PER_BLOCK)))

    def work(job):
        h, r0, r1 = job
        out[h, r0:r1] = _store(_rows(seed, stream, h * N + r0, h * N + r1, d, normalise, scale),
                               dtype)

    if len(jobs) > 1 and threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, jobs))
    else:
        for j in jobs:
            work(j)
    return out


def make_inputs(B: int, H: int, N: int, d: int, L: int, P: int, dtype: str, seed: int,
                with_grad: bool = True, n_rows: int | None = None,
                row_scale: bool = False) -> dict:
    """All inputs of a workload in storage form: W (fp32) and q, k, v[, do].
    row_scale: un-normalised Q and K rows (module docstring)."""
    BH = B * H
    n = N if n_rows is None else n_rows
    res = {"W": make_w(seed, L, P, d)}
    for name, s in (("q", STREAM_Q), ("k", STREAM_K), ("v", STREAM_V)):
        res[name] = make_tensor(seed, s, BH, N, d, dtype, n,
                                row_scale=row_scale).reshape(B, H, n, d)
    if with_grad:
        res["do"] = make_tensor(seed, STREAM_DO, BH, N, d, dtype, n).reshape(B, H, n, d)
    return res


def workload_inputs(w: Workload, n_rows: int | None = None, with_grad: bool | None = None):
    """Inputs of a named workload (optionally only the first n_rows per head)."""
    wg = w.backward if with_grad is None else with_grad
    return make_inputs(w.B, w.H, w.N, w.d, w.L, w.P, w.dtype, w.seed, wg, n_rows)
