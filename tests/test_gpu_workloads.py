"""Parity at the five workloads' full sizes, in the configuration bench.py times.

* non-causal forward, N = 1024, fp32: every output against the live oracle;
* causal fwd+bwd, 8 heads x 65536, fp32, segments of 256 tokens: every
  output of every head against the live oracle;
* causal fwd+bwd, 4 x 16 heads x 16384, bf16, L = 64: every output of a
  sample of heads against the live oracle, gradient identities on all heads;
* causal fwd+bwd, N = 4,194,304, bf16: sampled rows against oracle values
  written by tests/golden/make_workload_golden.py (inputs checked by digest),
  gradient identities over the whole sequence;
* causal fwd+bwd, N = 75,000,000, bf16, L = 16: o, den, dq, dk, dv at
  about 280 rows sampled over the whole sequence (past element offset 2^31
  and up to the last row) against values that
  tests/golden/make_stream_golden.py streamed through the oracle, gradient
  identities over all rows; and two forward invariants over all rows:
  perturbing token j leaves every output before j bitwise unchanged, and
  constant values (powers of two) come out exactly.

Bar: relative Frobenius error 1e-4 (fp32) / 2e-2 (bf16), per head or over
the sampled rows.
"""
import hashlib
import os

import numpy as np
import pytest
import torch

import oracle
from sketch_attention_soft_amd import binding
from sketch_attention_soft_amd import inputs as I
from tests.gpu_util import (GRAD_FLOOR, ROW_FLOOR, ROW_TOL, TOL, device_inputs, head_relf,
                            host_inputs, row_errors, row_report, to_host64)

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _relf(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def _run(w, dx):
    """forward + backward as bench.py times them (the backward reads the
    forward's saved state)."""
    print(f"[workload] {w.name}: B={w.B} H={w.H} N={w.N} L={w.L} {w.dtype}", flush=True)
    sv = binding.new_saved(dx["q"], dx["W"], w.causal, w.chunk) if w.backward else None
    o, den = binding.forward(dx["q"], dx["k"], dx["v"], dx["W"], w.tau, w.causal, w.chunk,
                             saved=sv)
    res = {"o": o, "den": den}
    if w.backward:
        dq, dk, dv = binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"],
                                      w.tau, w.causal, w.chunk, saved=sv)
        res.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    del sv
    return res


def _identities(res, dx, tol, rows=1 << 22):
    """Gradient identities that hold at any size (per head, fp64 on the GPU,
    in slices of rows): sum_j dv_j = sum_i dO_i and <dq_i, q_i> = <dk_j, k_j> = 0."""
    N = dx["q"].shape[-2]
    sdv = sg = 0.0
    cos = {"dq": 0.0, "dk": 0.0}
    for r0 in range(0, N, rows):
        sl = slice(r0, min(N, r0 + rows))
        sdv = sdv + res["dv"][..., sl, :].double().sum(-2)
        sg = sg + dx["do"][..., sl, :].double().sum(-2)
        for gr, x in (("dq", "q"), ("dk", "k")):
            a, b = res[gr][..., sl, :].double(), dx[x][..., sl, :].double()
            c = (a * b).sum(-1).abs() / (a.norm(dim=-1) * b.norm(dim=-1) + 1e-30)
            cos[gr] += c.sum().item()
    err = ((sdv - sg).norm(dim=-1) / sg.norm(dim=-1)).max().item()
    print(f"  sum dv vs sum dO: {err:.2e}")
    assert err <= tol
    cnt = dx["q"].numel() // dx["q"].shape[-1]
    for gr in cos:
        c = cos[gr] / cnt
        print(f"  mean |<{gr}, x>| / norms: {c:.2e}")
        assert c <= tol


def test_noncausal_fwd_n1k_f32():
    w = I.WORKLOADS["noncausal_fwd_n1k_f32"]
    x = I.workload_inputs(w)
    res = _run(w, device_inputs(x, w.dtype))
    hx = host_inputs(x, w.dtype)
    ro, rden = oracle.forward(hx["q"], hx["k"], hx["v"], hx["W"], w.tau, w.causal)
    e = head_relf(to_host64(res["o"]), ro)
    print(f"  rel_o={e:.2e}")
    assert e <= TOL[w.dtype]
    np.testing.assert_allclose(to_host64(res["den"]), rden, rtol=TOL[w.dtype])


@pytest.mark.timeout(600)
def test_causal_h8_n64k_f32():
    w = I.WORKLOADS["causal_h8_n64k_f32"]
    x = I.workload_inputs(w)
    dx = device_inputs(x, w.dtype)
    res = _run(w, dx)
    hx = host_inputs(x, w.dtype)
    ref = dict(zip(("o", "den", "dq", "dk", "dv"),
                   oracle.forward_backward(hx["q"], hx["k"], hx["v"], hx["do"], hx["W"], w.tau,
                                           w.causal)))
    for n in ("o", "dq", "dk", "dv"):
        e = head_relf(to_host64(res[n]), ref[n])
        print(f"  rel_{n}={e:.2e}")
        assert e <= TOL[w.dtype], (n, e)
    _identities(res, dx, 1e-4)


@pytest.mark.timeout(600)
def test_causal_b4h16_n16k_bf16():
    w = I.WORKLOADS["causal_b4h16_n16k_bf16"]
    x = I.workload_inputs(w)
    dx = device_inputs(x, w.dtype)
    res = _run(w, dx)
    hx = host_inputs(x, w.dtype)
    heads = [(0, 0), (1, 5), (2, 10), (3, 15)]
    for b, h in heads:
        ref = dict(zip(("o", "den", "dq", "dk", "dv"),
                       oracle.forward_backward(hx["q"][b, h], hx["k"][b, h], hx["v"][b, h],
                                               hx["do"][b, h], hx["W"], w.tau, w.causal)))
        for n in ("o", "dq", "dk", "dv"):
            e = _relf(to_host64(res[n][b, h]), ref[n])
            print(f"  head ({b},{h}) rel_{n}={e:.2e}")
            assert e <= TOL[w.dtype], (b, h, n, e)
    _identities(res, dx, 2e-2)


@pytest.mark.timeout(600)
def test_causal_n4m_bf16():
    w = I.WORKLOADS["causal_n4m_bf16"]
    path = os.path.join(GOLDEN, f"{w.name}_rows.npz")
    gold = np.load(path)
    x = I.workload_inputs(w)
    h = hashlib.sha256()
    for k in ("W", "q", "k", "v", "do"):
        h.update(np.ascontiguousarray(x[k]).tobytes())
    assert h.hexdigest() == str(gold["digest"]), "input generator drifted from the stored values"
    dx = device_inputs(x, w.dtype)
    del x
    res = _run(w, dx)
    rows = torch.from_numpy(gold["rows"]).cuda()
    for n in ("o", "dq", "dk", "dv"):
        got = res[n][0, 0].index_select(0, rows).double().cpu().numpy()
        e = _relf(got, gold[n])
        print(f"  sampled rel_{n}={e:.2e}")
        assert e <= TOL[w.dtype], (n, e)
    got = res["den"][0, 0].index_select(0, rows).double().cpu().numpy()
    assert _relf(got, gold["den"]) <= TOL[w.dtype]
    _identities(res, dx, 2e-2)


@pytest.fixture(scope="module")
def n75m():
    """The 75M-token workload's inputs on the device (about 40 GB), shared by
    the tests below."""
    w = I.WORKLOADS["causal_n75m_bf16"]
    print(f"[workload] {w.name}: generating inputs", flush=True)
    x = I.workload_inputs(w)
    dx = device_inputs(x, w.dtype)
    del x
    yield w, dx
    del dx
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_causal_n75m_bf16(n75m):
    w, dx = n75m
    gold = np.load(os.path.join(GOLDEN, f"{w.name}_rows.npz"))
    # the sampled blocks' inputs, regenerated alone, are those on the device
    # and those the stored values were computed from
    h = hashlib.sha256(np.ascontiguousarray(I.make_w(w.seed, w.L, w.P, w.d)).tobytes())
    B = int(gold["block_rows"])
    for b in gold["blocks"]:
        r0, r1 = int(b) * B, min(w.N, (int(b) + 1) * B)
        for n, st in (("q", I.STREAM_Q), ("k", I.STREAM_K), ("v", I.STREAM_V),
                      ("do", I.STREAM_DO)):
            raw = I.stream_rows(w.seed, st, r0, r1, w.d, w.dtype)
            h.update(np.ascontiguousarray(raw).tobytes())
            dev = dx[n][0, 0, r0:r1].view(torch.int16).cpu().numpy().view(np.uint16)
            assert np.array_equal(dev, raw), (n, int(b))
    assert h.hexdigest() == str(gold["digest"]), "input generator drifted from the stored values"
    res = _run(w, dx)
    rows = torch.from_numpy(gold["rows"]).cuda()
    print(f"  {rows.numel()} sampled rows, last {int(gold['rows'][-1])}", flush=True)
    for n in ("o", "dq", "dk", "dv"):
        got = res[n][0, 0].index_select(0, rows).double().cpu().numpy()
        e = _relf(got, gold[n])
        e_row = row_errors(got, gold[n], GRAD_FLOOR if n in ("dq", "dk") else ROW_FLOOR)
        print(f"  sampled rel_{n}={e:.2e} " + row_report(n, e_row))
        assert e <= TOL[w.dtype], (n, e)
        assert e_row.max() <= ROW_TOL[w.dtype], (n, e_row.max())
    got = res["den"][0, 0].index_select(0, rows).double().cpu().numpy()
    e_den = np.abs(got / gold["den"] - 1).max()
    print(f"  sampled den: max rel {e_den:.2e}")
    assert e_den <= TOL[w.dtype]
    _identities(res, dx, 2e-2)


@pytest.mark.timeout(900)
def test_causal_n75m_perturbation(n75m):
    """Perturbing token j (its query, key and value) changes no output before
    j: o and den of rows i < j are bitwise the same over 75M rows."""
    w, dx = n75m
    j = 60_000_017
    o1, den1 = binding.forward(dx["q"], dx["k"], dx["v"], dx["W"], w.tau, True, w.chunk)
    q, k, v = (dx[n].clone() for n in ("q", "k", "v"))
    q[0, 0, j] = -q[0, 0, j]
    k[0, 0, j] = k[0, 0, j + 1]
    v[0, 0, j] = 4.0
    o2, den2 = binding.forward(q, k, v, dx["W"], w.tau, True, w.chunk)
    torch.cuda.synchronize()
    same_o = torch.equal(o1[0, 0, :j], o2[0, 0, :j])
    same_den = torch.equal(den1[0, 0, :j], den2[0, 0, :j])
    changed = int((o1[0, 0, j:] != o2[0, 0, j:]).any(dim=-1).sum().item())
    print(f"  rows < {j}: o bitwise {same_o}, den bitwise {same_den}; rows >= j changed: {changed}")
    assert same_o and same_den
    assert not torch.equal(o1[0, 0, j], o2[0, 0, j])
    del q, k, v, o1, o2, den1, den2


@pytest.mark.timeout(900)
def test_causal_n75m_constant_values(n75m):
    """Constant values come out exactly: with v_j = c for every row (c_col = a
    signed power of two, so that n = c m holds bit for bit), o_i = c on all
    75M rows."""
    w, dx = n75m
    col = torch.arange(w.d, device="cuda")
    c = torch.where(col % 2 == 0, 1.0, -1.0) * torch.exp2((col % 9 - 4).float())
    v = c.to(torch.bfloat16).expand(1, 1, w.N, w.d).contiguous()
    o, den = binding.forward(dx["q"], dx["k"], v, dx["W"], w.tau, True, w.chunk)
    torch.cuda.synchronize()
    bad = int((o[0, 0] != v[0, 0]).any(dim=-1).sum().item())
    print(f"  rows differing from the constant: {bad}")
    assert bad == 0
    assert bool(torch.isfinite(den).all()) and bool((den > 0).all())
    del v, o, den
