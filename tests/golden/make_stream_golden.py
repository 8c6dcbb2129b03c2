#!/usr/bin/env python3
"""Write the oracle's expected values at rows sampled over a whole sequence
too long to hold at once (the causal 75,000,000-token workload).

The sequence is streamed through the fp64 oracle in the input generator's
blocks of 65,536 rows (oracle.stream_forward / stream_backward, pinned bit
for bit against the one-shot oracle by P-15 and P-16):

1. forward over every block in order, carrying the key sums from block to
   block; for every block the gradient sums of its queries,
   sum_i phi(q_i) [g_i/m_i | -(g_i . o_i)/m_i]^T (oracle.block_sums), are
   kept, and for the sampled blocks also the key sums before them and their
   o, den;
2. the gradient sums after each sampled block (the sum of the later blocks'
   sums), then the backward of the sampled blocks.

Stored: o, den, dq, dk, dv at the sampled rows (fp64), the sum of dO over
all rows, and a SHA-256 digest of W and of the sampled blocks' input
bytes.  Calls nothing but the oracle and the input generator.

Usage: python tests/golden/make_stream_golden.py [causal_n75m_bf16]
(about 15 minutes on 8 cores).
"""
from __future__ import annotations

import hashlib
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from sketch_attention_soft_amd import inputs as I  # noqa: E402

BLOCK = I.ROWS_PER_BLOCK
STREAMS = (("q", I.STREAM_Q), ("k", I.STREAM_K), ("v", I.STREAM_V), ("do", I.STREAM_DO))


def sampled_blocks(N: int) -> list:
    """Blocks whose rows are sampled: the first two, the ones around rows
    2^24 and 2^25 (element offsets 2^30 and 2^31 at d = 64, where 32-bit
    offsets would wrap), four spread further on, and the last two."""
    nb = -(-N // BLOCK)
    want = [0, 1, 255, 256, 511, 512, 513, nb // 2 + 3, (2 * nb) // 3, (5 * nb) // 6, nb - 2, nb - 1]
    return sorted({b for b in want if 0 <= b < nb})


def sample_rows(N: int, seed: int) -> np.ndarray:
    """In every sampled block: its first 4 and last 4 rows and 14 others at
    random; and the last 16 rows of the sequence (about 280 rows)."""
    rng = np.random.default_rng(seed)
    rows = []
    for b in sampled_blocks(N):
        r0, r1 = b * BLOCK, min(N, (b + 1) * BLOCK)
        rows += list(range(r0, r0 + 4)) + list(range(r1 - 4, r1))
        rows += list(rng.choice(np.arange(r0 + 4, r1 - 4), 14, replace=False))
    rows += list(range(N - 16, N))
    return np.unique(np.array(rows, dtype=np.int64))


def block_inputs(w, b: int, pool: ThreadPoolExecutor) -> dict:
    r0, r1 = b * BLOCK, min(w.N, (b + 1) * BLOCK)
    futs = {n: pool.submit(I.stream_rows, w.seed, s, r0, r1, w.d, w.dtype) for n, s in STREAMS}
    return {n: f.result() for n, f in futs.items()}


def compute(w, log=print) -> dict:
    """Stream every row of the single-head causal workload w through the
    oracle; returns the sampled rows' values and the digest (see above)."""
    assert w.B * w.H == 1 and w.causal and w.backward
    N, d, L, P, tau = w.N, w.d, w.L, w.P, w.tau
    W = I.make_w(w.seed, L, P, d)
    Wd = W.astype(np.float64)
    nb = -(-N // BLOCK)
    sblocks = set(sampled_blocks(N))
    log(f"{w.name}: {nb} blocks, sampled {sorted(sblocks)}, oracle threads {oracle.threads()}")
    digest = hashlib.sha256(np.ascontiguousarray(W).tobytes())
    state = oracle.new_stream_state(L, P, d)
    gsums = [None] * nb
    keep = {}
    sum_g = np.zeros(d)
    t0 = time.time()
    with ThreadPoolExecutor(4) as gen, ThreadPoolExecutor(1) as pre:
        nxt = pre.submit(block_inputs, w, 0, gen)
        for b in range(nb):
            raw = nxt.result()
            if b + 1 < nb:
                nxt = pre.submit(block_inputs, w, b + 1, gen)
            x = {n: I.to_f64(raw[n], w.dtype) for n in raw}
            before = state.copy() if b in sblocks else None
            o, den = oracle.stream_forward(x["q"], x["k"], x["v"], Wd, tau, state)
            D = oracle.ratio_gradients(x["do"], o, den)
            gsums[b] = oracle.block_sums(x["q"], D, Wd, tau, oracle.new_stream_state(L, P, d))
            sum_g += x["do"].sum(axis=0)
            if b in sblocks:
                for n in ("q", "k", "v", "do"):
                    digest.update(np.ascontiguousarray(raw[n]).tobytes())
                keep[b] = (before, o, den)
            if b % 64 == 0 or b == nb - 1:
                log(f"  forward block {b + 1}/{nb}  {time.time() - t0:.0f}s")
    # gradient sums of the queries after each block, from the end
    after = [None] * nb
    acc = oracle.new_stream_state(L, P, d)
    for b in range(nb - 1, -1, -1):
        after[b] = acc.copy()
        acc += gsums[b]
    rows = sample_rows(N, w.seed)
    res = {n: np.empty((rows.size, d)) for n in ("o", "dq", "dk", "dv")}
    res["den"] = np.empty(rows.size)
    with ThreadPoolExecutor(4) as gen:
        for b in sorted(sblocks):
            r0, r1 = b * BLOCK, min(N, (b + 1) * BLOCK)
            x = {n: I.to_f64(a, w.dtype) for n, a in block_inputs(w, b, gen).items()}
            before, o, den = keep[b]
            dq, dk, dv = oracle.stream_backward(x["q"], x["k"], x["v"], x["do"], o, den, Wd, tau,
                                                before.copy(), after[b].copy())
            sel = (rows >= r0) & (rows < r1)
            loc = rows[sel] - r0
            for n, a in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv)):
                res[n][sel] = a[loc]
            res["den"][sel] = den[loc]
            log(f"  backward of block {b} done  {time.time() - t0:.0f}s")
    res.update(rows=rows, digest=np.array(digest.hexdigest()),
               blocks=np.array(sorted(sblocks), dtype=np.int64), block_rows=BLOCK, sum_g=sum_g)
    return res


def main(name: str) -> None:
    res = compute(I.WORKLOADS[name], log=lambda m: print(m, flush=True))
    out = os.path.join(HERE, f"{name}_rows.npz")
    np.savez_compressed(out, **res)
    print("wrote", out, os.path.getsize(out), "bytes")


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else "causal_n75m_bf16")
