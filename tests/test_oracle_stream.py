"""Pins of the oracle's block-streaming entry points (causal running sums
carried from block to block, gist.science/zh/paper/2510.04008, technical
summary §2.3), which let a sequence too long to hold at once be checked
block by block.

P-15: chaining oracle.stream_forward over consecutive blocks gives the
one-shot causal oracle.forward bit for bit (every sum runs in the same token
order), and the independent quadratic closed form (tests/quadratic_ref.py)
to rounding; the state after the last block is the sequence's bucket sums
(oracle.bucket_sums, block_sums).
P-16: oracle.stream_backward over the blocks in reverse, each given the key
sums before it and the gradient sums after it, gives the one-shot
oracle.forward_backward; the gradient sums of a block are block_sums of its
queries with values ratio_gradients, so states assembled from per-block sums
(as a script over 75M rows does) give the same gradients to rounding.
"""
import numpy as np
import pytest

import oracle
from sketch_attention_soft_amd import inputs as I
from tests import quadratic_ref as Q


def _head(N, d, L, P, dtype, seed, row_scale=False):
    x = I.make_inputs(1, 1, N, d, L, P, dtype, seed, row_scale=row_scale)
    return {n: I.to_f64(x[n], dtype)[0, 0] for n in ("q", "k", "v", "do")}, x["W"].astype(np.float64)


def _blocks(N, sizes):
    edges = [0]
    for s in sizes:
        edges.append(min(N, edges[-1] + s))
    edges[-1] = N
    return list(zip(edges[:-1], edges[1:]))


CASES = [
    # N, d, L, P, tau, block sizes (the last block takes the rest)
    (700, 16, 3, 4, 1.0, (1, 255, 100, 344)),
    (5000, 64, 8, 4, 0.5, (2048, 2049, 903)),
    (333, 8, 2, 2, 0.7, (333,)),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "N%d_d%d_L%d_P%d" % c[:4])
@pytest.mark.parametrize("row_scale", [False, True], ids=["unit", "scaled"])
def test_p15_stream_forward_equals_one_shot(case, row_scale):
    N, d, L, P, tau, sizes = case
    x, W = _head(N, d, L, P, "f32", 70 + N, row_scale)
    st = oracle.new_stream_state(L, P, d)
    o = np.empty((N, d))
    den = np.empty(N)
    for a, b in _blocks(N, sizes):
        o[a:b], den[a:b] = oracle.stream_forward(x["q"][a:b], x["k"][a:b], x["v"][a:b], W, tau, st)
    ro, rden = oracle.forward(x["q"], x["k"], x["v"], W, tau, True)
    assert np.array_equal(o, ro) and np.array_equal(den, rden)
    if N <= 1000:
        qo, qden = Q.soft_race_attention(x["q"], x["k"], x["v"], W, tau, True)
        assert np.abs(o - qo).max() <= 1e-12 * np.abs(qo).max()
        assert np.abs(den / qden - 1).max() <= 1e-12
    # the final state: every key's bucket sums
    AB = oracle.bucket_sums(x["k"], x["v"], W, tau)               # [L, R, d + 1]
    assert np.allclose(st, AB.reshape(L << P, d + 1).T, rtol=1e-12, atol=1e-9)
    y = np.concatenate([x["v"], np.ones((N, 1))], axis=1)
    bs = oracle.block_sums(x["k"], y, W, tau, oracle.new_stream_state(L, P, d))
    assert np.array_equal(bs, st)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "N%d_d%d_L%d_P%d" % c[:4])
@pytest.mark.parametrize("row_scale", [False, True], ids=["unit", "scaled"])
def test_p16_stream_backward_equals_one_shot(case, row_scale):
    N, d, L, P, tau, sizes = case
    x, W = _head(N, d, L, P, "f32", 90 + N, row_scale)
    blocks = _blocks(N, sizes)
    # forward, keeping the key sums before each block
    st = oracle.new_stream_state(L, P, d)
    before, o, den = [], np.empty((N, d)), np.empty(N)
    for a, b in blocks:
        before.append(st.copy())
        o[a:b], den[a:b] = oracle.stream_forward(x["q"][a:b], x["k"][a:b], x["v"][a:b], W, tau, st)
    ref = oracle.forward_backward(x["q"], x["k"], x["v"], x["do"], W, tau, True)
    # reverse chain: each block gets the gradient sums of the queries after it
    G = oracle.new_stream_state(L, P, d)
    grads = np.empty((3, N, d))
    for (a, b), S in reversed(list(zip(blocks, before))):
        S = S.copy()
        g = oracle.stream_backward(x["q"][a:b], x["k"][a:b], x["v"][a:b], x["do"][a:b], o[a:b],
                                   den[a:b], W, tau, S, G)
        grads[:, a:b] = g
    for i, n in enumerate(("dq", "dk", "dv")):
        assert np.array_equal(grads[i], ref[2 + i]), n
    # gradient states from per-block sums, as a long-sequence script builds them
    D = oracle.ratio_gradients(x["do"], o, den)
    sums = [oracle.block_sums(x["q"][a:b], D[a:b], W, tau, oracle.new_stream_state(L, P, d))
            for a, b in blocks]
    for j, ((a, b), S) in enumerate(zip(blocks, before)):
        Gs = sum(sums[j + 1:], oracle.new_stream_state(L, P, d))
        got = oracle.stream_backward(x["q"][a:b], x["k"][a:b], x["v"][a:b], x["do"][a:b],
                                     o[a:b], den[a:b], W, tau, S.copy(), Gs)
        for i, n in enumerate(("dq", "dk", "dv")):
            r = ref[2 + i][a:b]
            assert np.abs(got[i] - r).max() <= 1e-10 * max(np.abs(r).max(), 1e-30), n
    # and the summed gradient state is the whole sequence's
    assert np.allclose(G, sum(sums), rtol=1e-12, atol=1e-12)


def test_stream_rejects_bad_shapes():
    x, W = _head(10, 8, 2, 4, "f32", 5)
    with pytest.raises(AssertionError):
        oracle.stream_forward(x["q"], x["k"], x["v"], W, 1.0, np.zeros((8, 32)))
    with pytest.raises(ValueError):
        oracle.stream_forward(x["q"], x["k"], x["v"], W, -1.0, oracle.new_stream_state(2, 4, 8))


def test_stream_golden_script_matches_the_one_shot_oracle():
    """tests/golden/make_stream_golden.py's assembly (per-block gradient sums,
    suffixes, the backward of sampled blocks) on a sequence of four
    generator blocks, every block sampled, against the one-shot oracle."""
    import dataclasses
    import importlib.util
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                        "make_stream_golden.py")
    spec = importlib.util.spec_from_file_location("make_stream_golden", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    w = dataclasses.replace(I.WORKLOADS["causal_n75m_bf16"], N=3 * I.ROWS_PER_BLOCK + 1000, L=2,
                            d=16, name="small")
    assert mod.sampled_blocks(w.N) == [0, 1, 2, 3]
    res = mod.compute(w, log=lambda m: None)
    x = I.workload_inputs(w)
    h = {n: I.to_f64(x[n], w.dtype)[0, 0] for n in ("q", "k", "v", "do")}
    ref = oracle.forward_backward(h["q"], h["k"], h["v"], h["do"], x["W"], w.tau, True)
    rows = res["rows"]
    assert rows.size > 80 and rows.max() == w.N - 1
    for i, n in enumerate(("o", "den", "dq", "dk", "dv")):
        r = ref[i][rows]
        err = np.abs(res[n] - r).max() / np.abs(r).max()
        assert err <= 1e-12, (n, err)
    assert np.allclose(res["sum_g"], h["do"].sum(0), rtol=1e-12, atol=1e-9)
