#!/usr/bin/env python3
"""Write the oracle's expected values at sampled rows of a full workload.

Runs the fp64 oracle (``oracle/``) on every row of the named workload's
seeded inputs and stores, for a fixed set of sampled rows, o, den, dq, dk
and dv together with a digest of the input bytes, so that a GPU test can
regenerate the same inputs, run the library at full size and compare the
sampled rows.  Calls nothing but the oracle and the input generator.

Usage: python tests/golden/make_workload_golden.py causal_n4m_bf16
"""
from __future__ import annotations

import hashlib
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from sketch_attention_soft_amd import inputs as I  # noqa: E402

N_SAMPLE = 256


def sample_rows(N: int, seed: int) -> np.ndarray:
    """First 32 and last 32 rows plus 192 spread over the sequence."""
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(32, N - 32), N_SAMPLE - 64, replace=False)
    return np.unique(np.concatenate([np.arange(32), mid, np.arange(N - 32, N)]))


def input_digest(x: dict) -> str:
    h = hashlib.sha256()
    for k in ("W", "q", "k", "v", "do"):
        if k in x:
            h.update(np.ascontiguousarray(x[k]).tobytes())
    return h.hexdigest()


def main(name: str) -> None:
    w = I.WORKLOADS[name]
    assert w.B * w.H == 1, "sampled goldens are for single-head workloads"
    t0 = time.time()
    x = I.workload_inputs(w)
    digest = input_digest(x)
    q, k, v = (I.to_f64(x[n], w.dtype) for n in ("q", "k", "v"))
    g = I.to_f64(x["do"], w.dtype)
    print(f"inputs {time.time() - t0:.1f}s, oracle threads {oracle.threads()}", flush=True)
    t0 = time.time()
    o, den, dq, dk, dv = oracle.forward_backward(q, k, v, g, x["W"], w.tau, w.causal)
    print(f"oracle fwd+bwd {time.time() - t0:.1f}s", flush=True)
    rows = sample_rows(w.N, w.seed)
    out = os.path.join(HERE, f"{name}_rows.npz")
    np.savez_compressed(out, rows=rows, digest=np.array(digest), o=o[0, 0, rows],
                        den=den[0, 0, rows], dq=dq[0, 0, rows], dk=dk[0, 0, rows],
                        dv=dv[0, 0, rows],
                        sum_dv=dv[0, 0].sum(0), sum_g=g[0, 0].sum(0))
    print("wrote", out, os.path.getsize(out), "bytes")


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else "causal_n4m_bf16")
