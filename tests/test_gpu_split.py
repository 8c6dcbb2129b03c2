"""More than 32 tables: passes over tables 0..31, 32..63, ... (up to
L = 128, four passes) of the fused kernels (16-bit rows) or of the unfused
fp32 kernels, the first storing fp32 partial sums, the middle ones adding to
them and the last adding them before the ratio, dV and the normalisation
backward.

The readout and its gradients are sums over tables until those last steps
(pages: "RACE Attention: A Strictly Linear-Time Attention for Long-Sequence
Training", gist.science/zh/paper/2510.04008, technical summary §2.2: n and m
sum the tables' bucket statistics), so splitting the tables changes only the
order of the sums.  Bar: the parity bar of the storage type, against the
fp64 oracle on the same inputs, per head (relative Frobenius) and per row
(tests/gpu_util.row_errors).
"""
import numpy as np
import pytest
import torch

import oracle
from sketch_attention_soft_amd import binding
from sketch_attention_soft_amd import inputs as I
from tests.gpu_util import (GRAD_FLOOR, ROW_FLOOR, ROW_TOL, TOL, device_inputs, head_relf,
                            host_inputs, row_errors, row_report, to_host64)

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, B, H, N, L, P, tau, chunk
    ("bf16", 1, 2, 1000, 64, 4, 1.0, 0),
    ("f16", 1, 1, 4133, 64, 4, 0.5, 256),
    ("bf16", 2, 1, 257, 33, 4, 1.0, 64),
    ("f16", 1, 2, 700, 48, 3, 1.0, 0),
    ("bf16", 1, 1, 1, 40, 4, 1.0, 0),
    ("bf16", 1, 1, 2100, 128, 4, 0.5, 0),
    ("f16", 1, 2, 600, 96, 4, 1.0, 64),
    ("bf16", 2, 1, 333, 65, 4, 1.0, 0),
    ("bf16", 1, 1, 1500, 100, 2, 1.0, 128),
]


@pytest.mark.parametrize("saved", [False, True], ids=["recompute", "saved"])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s_B%dH%dN%dL%dP%d_tau%g_ch%d" % c)
def test_split_tables(case, causal, saved):
    dtype, B, H, N, L, P, tau, chunk = case
    x = I.make_inputs(B, H, N, 64, L, P, dtype, 2100 + N + L + P + causal, with_grad=True)
    dx, hx = device_inputs(x, dtype), host_inputs(x, dtype)
    print(f"[case] split {dtype} B={B} H={H} N={N} L={L} P={P} causal={causal} saved={saved}",
          flush=True)
    sv = binding.new_saved(dx["q"], dx["W"], causal, chunk) if saved else None
    o, den = binding.forward(dx["q"], dx["k"], dx["v"], dx["W"], tau, causal, chunk, saved=sv)
    dq, dk, dv = binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], tau,
                                  causal, chunk, saved=sv)
    torch.cuda.synchronize()
    ref = dict(zip(("o", "den", "dq", "dk", "dv"),
                   oracle.forward_backward(hx["q"], hx["k"], hx["v"], hx["do"], hx["W"], tau,
                                           causal)))
    got = {"o": o, "den": den, "dq": dq, "dk": dk, "dv": dv}
    for n in got:
        g = to_host64(got[n])
        assert np.all(np.isfinite(g)), n
        # dQ and dK floored on dV's scale; N = 1: every query sees only its own
        # key, the exact dQ and dK are zero and the computed ones rounding noise
        fr = ref["dv"] if n in ("dq", "dk") else None
        e = head_relf(g, ref[n], floor_ref=fr, floor=1.0 if N == 1 else 1e-3)
        print(f"  rel_{n}={e:.2e}")
        assert e <= TOL[dtype], (n, e)
    _row_gate(got, ref, dtype, N, causal)


def _row_gate(got, ref, dtype, N, causal):
    """Per-row errors (dQ, dK: skipped at N = 1, where they vanish exactly;
    causal dQ row 0 is exactly zero and measured on the head's scale)."""
    for n in ("o", "dv") + (("dq", "dk") if N > 1 else ()):
        e_row = row_errors(to_host64(got[n]), ref[n], GRAD_FLOOR if n in ("dq", "dk") else ROW_FLOOR,
                           vanishing=(0,) if n == "dq" and causal else ())
        print("  " + row_report(n, e_row))
        assert e_row.max() <= ROW_TOL[dtype], (n, e_row.max())


F32_CASES = [
    # B, H, N, L, tau, chunk: two passes (the second full or of 8 tables),
    # four passes (first, two middle, last), one token
    (1, 2, 1000, 64, 1.0, 0),
    (2, 1, 700, 40, 0.5, 64),
    (1, 1, 1300, 128, 1.0, 256),
    (1, 1, 1, 65, 1.0, 0),
]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
@pytest.mark.parametrize("case", F32_CASES, ids=lambda c: "f32_B%dH%dN%dL%d_tau%g_ch%d" % c)
def test_split_tables_f32(case, causal):
    """fp32 rows with L > 32: passes of the unfused fp32 kernels, the fp32
    bar (1e-4)."""
    B, H, N, L, tau, chunk = case
    x = I.make_inputs(B, H, N, 64, L, 4, "f32", 2300 + N + L + causal, with_grad=True)
    dx, hx = device_inputs(x, "f32"), host_inputs(x, "f32")
    print(f"[case] split f32 B={B} H={H} N={N} L={L} causal={causal}", flush=True)
    o, den = binding.forward(dx["q"], dx["k"], dx["v"], dx["W"], tau, causal, chunk)
    dq, dk, dv = binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], tau,
                                  causal, chunk)
    torch.cuda.synchronize()
    ref = dict(zip(("o", "den", "dq", "dk", "dv"),
                   oracle.forward_backward(hx["q"], hx["k"], hx["v"], hx["do"], hx["W"], tau,
                                           causal)))
    got = {"o": o, "den": den, "dq": dq, "dk": dk, "dv": dv}
    for n in got:
        g = to_host64(got[n])
        assert np.all(np.isfinite(g)), n
        fr = ref["dv"] if n in ("dq", "dk") else None
        e = head_relf(g, ref[n], floor_ref=fr, floor=1.0 if N == 1 else 1e-3)
        print(f"  rel_{n}={e:.2e}")
        assert e <= TOL["f32"], (n, e)
    _row_gate(got, ref, "f32", N, causal)
    with pytest.raises(binding.RaceError):  # no dW on fp32 rows
        binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], tau, causal, chunk,
                         dw=True)


def test_split_f32_padded_and_hard():
    """fp32, L = 64: a right-padded batch against the oracle on each sequence,
    and the hard forward (t = +-1 on the unfused kernels) against the
    oracle's hard mode."""
    H, N, L, tau, lens = 1, 600, 64, 1.0, (600, 250)
    B = len(lens)
    x = I.make_inputs(B, H, N, 64, L, 4, "f32", 2395, with_grad=True)
    dx, hx = device_inputs(x, "f32"), host_inputs(x, "f32")
    print("[case] split f32 padded + hard", flush=True)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o, den = binding.forward_padded(dx["q"], dx["k"], dx["v"], dx["W"], sl, tau, True)
    dq, dk, dv = binding.backward_padded(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], sl,
                                         tau, True)
    oh, denh = binding.forward_hard(dx["q"], dx["k"], dx["v"], dx["W"], True)
    torch.cuda.synchronize()
    for b, n_b in enumerate(lens):
        sub = {k_: hx[k_][b:b + 1, :, :n_b] for k_ in ("q", "k", "v", "do")}
        ref = oracle.forward_backward(sub["q"], sub["k"], sub["v"], sub["do"], hx["W"], tau, True)
        for t, r in zip((o, den, dq, dk, dv), ref):
            assert head_relf(to_host64(t)[b:b + 1, :, :n_b], r) <= TOL["f32"]
        assert not torch.any(o[b, :, n_b:])
    ro, rden = oracle.forward(hx["q"], hx["k"], hx["v"], hx["W"], 1.0, True, hard=True)
    d = to_host64(denh)
    assert np.array_equal(d, np.round(d)) and np.mean(d == rden) >= 0.999
    ok = d == rden
    assert head_relf(np.where(ok[..., None], to_host64(oh), 0.0), np.where(ok[..., None], ro, 0.0)) <= TOL["f32"]


@pytest.mark.parametrize("L", [64, 100])
def test_split_dw_and_hard(L):
    B, H, N, tau = 1, 2, 900, 1.0
    x = I.make_inputs(B, H, N, 64, L, 4, "bf16", 2190 + L, with_grad=True)
    dx, hx = device_inputs(x, "bf16"), host_inputs(x, "bf16")
    print(f"[case] split dW + hard L={L}", flush=True)
    o, den = binding.forward(dx["q"], dx["k"], dx["v"], dx["W"], tau, True)
    *_, dW = binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], tau, True,
                              dw=True)
    oh, denh = binding.forward_hard(dx["q"], dx["k"], dx["v"], dx["W"], True)
    torch.cuda.synchronize()
    ref = oracle.forward_backward(hx["q"], hx["k"], hx["v"], hx["do"], hx["W"], tau, True,
                                  with_dw=True)
    err = np.linalg.norm(to_host64(dW) - ref[5]) / np.linalg.norm(ref[5])
    print(f"  dW rel err {err:.2e}")
    assert err <= TOL["bf16"]
    ro, rden = oracle.forward(hx["q"], hx["k"], hx["v"], hx["W"], 1.0, True, hard=True)
    hit = (rden > 0) & (to_host64(denh) > 0)
    assert np.mean(hit) > 0.99
    assert head_relf(np.where(hit[..., None], to_host64(oh), 0.0),
                     np.where(hit[..., None], ro, 0.0)) <= TOL["bf16"]


def test_split_padded_batch():
    H, N, L, tau, lens = 1, 600, 64, 1.0, (600, 250)
    B = len(lens)
    x = I.make_inputs(B, H, N, 64, L, 4, "bf16", 2195, with_grad=True)
    dx, hx = device_inputs(x, "bf16"), host_inputs(x, "bf16")
    print("[case] split padded", flush=True)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o, den = binding.forward_padded(dx["q"], dx["k"], dx["v"], dx["W"], sl, tau, True)
    dq, dk, dv = binding.backward_padded(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], sl,
                                         tau, True)
    torch.cuda.synchronize()
    for b, n_b in enumerate(lens):
        sub = {k_: hx[k_][b:b + 1, :, :n_b] for k_ in ("q", "k", "v", "do")}
        ref = oracle.forward_backward(sub["q"], sub["k"], sub["v"], sub["do"], hx["W"], tau, True)
        for t, r in zip((o, den, dq, dk, dv), ref):
            assert head_relf(to_host64(t)[b:b + 1, :, :n_b], r) <= TOL["bf16"]
        assert not torch.any(o[b, :, n_b:])
