"""Parity of the HIP path (through the C ABI) against the fp64 oracle.

Small and medium shapes that span several segments, sub-chunks and a ragged
tail, both dtypes, causal and non-causal, every table count the library
dispatches on (1, 2, 4 or 8 waves), and explicit segment lengths.  Bar: max
over heads of the relative Frobenius error, 1e-4 for fp32 inputs and 2e-2 for
bf16 inputs (fp32 accumulation).
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
    # B, H, N, L, tau, chunk
    (1, 1, 1, 8, 1.0, 0),
    (1, 1, 15, 8, 1.0, 0),
    (1, 2, 100, 5, 0.5, 16),
    (2, 1, 257, 16, 1.0, 64),
    (1, 1, 1000, 3, 1.0, 0),
    (1, 1, 4133, 32, 1.0, 256),
    (1, 2, 2048, 32, 0.5, 0),
    (1, 1, 1500, 64, 0.5, 128),
]


def _ids(c):
    return "B%dH%dN%dL%d_tau%g_ch%d" % c


def _run(dtype, causal, B, H, N, L, tau, chunk, backward, saved=False):
    seed = 7 + N + 31 * L + (1 if causal else 0)
    x = I.make_inputs(B, H, N, 64, L, 4, dtype, seed, with_grad=backward)
    dx, hx = device_inputs(x, dtype), host_inputs(x, dtype)
    print(f"[case] {dtype} causal={causal} B={B} H={H} N={N} L={L} tau={tau} chunk={chunk}",
          flush=True)
    sv = binding.new_saved(dx["q"], dx["W"], causal, chunk) if saved else None
    o, den = binding.forward(dx["q"], dx["k"], dx["v"], dx["W"], tau, causal, chunk, saved=sv)
    torch.cuda.synchronize()
    res = {"o": to_host64(o), "den": to_host64(den)}
    if backward:
        dq, dk, dv = binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], tau,
                                      causal, chunk, saved=sv)
        torch.cuda.synchronize()
        res.update(dq=to_host64(dq), dk=to_host64(dk), dv=to_host64(dv))
        ref = oracle.forward_backward(hx["q"], hx["k"], hx["v"], hx["do"], hx["W"], tau, causal)
        refd = dict(zip(("o", "den", "dq", "dk", "dv"), ref))
    else:
        ro, rden = oracle.forward(hx["q"], hx["k"], hx["v"], hx["W"], tau, causal)
        refd = {"o": ro, "den": rden}
    return res, refd


@pytest.mark.parametrize("case", CASES, ids=_ids)
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_parity(dtype, causal, case):
    res, ref = _run(dtype, causal, *case, backward=False)
    tol = TOL[dtype]
    e_o = head_relf(res["o"], ref["o"])
    e_den = np.abs(res["den"] - ref["den"]).max() / np.abs(ref["den"]).max()
    e_row = row_errors(res["o"], ref["o"])
    print(f"  rel_o={e_o:.3e} rel_den={e_den:.3e} " + row_report("o", e_row))
    assert np.all(np.isfinite(res["o"]))
    assert e_o <= tol, e_o
    assert e_den <= tol, e_den
    assert e_row.max() <= ROW_TOL[dtype], e_row.max()


@pytest.mark.parametrize("case", CASES, ids=_ids)
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("saved", [False, True], ids=["recompute", "saved"])
def test_backward_parity(dtype, causal, case, saved):
    """saved: the backward reads the forward's saved state (as bench.py times it)."""
    res, ref = _run(dtype, causal, *case, backward=True, saved=saved)
    tol = TOL[dtype]
    # N = 1: every query sees only its own key, so o = v and the exact dQ, dK
    # are zero; the computed values are rounding noise, measured on dV's scale.
    floor = 1.0 if case[2] == 1 else 1e-3
    errs = {n: head_relf(res[n], ref[n], ref["dv"] if n in ("dq", "dk") else None, floor)
            for n in ("o", "dq", "dk", "dv")}
    print("  " + " ".join(f"rel_{n}={e:.3e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert np.all(np.isfinite(res[n])), n
        assert e <= tol, (n, e)
    # per-row gate (dQ, dK: skipped at N = 1, where they vanish exactly)
    for n in ("o", "dv") + (("dq", "dk") if case[2] > 1 else ()):
        e_row = row_errors(res[n], ref[n], GRAD_FLOOR if n in ("dq", "dk") else ROW_FLOOR,
                           vanishing=(0,) if n == "dq" and causal else ())
        print("  " + row_report(n, e_row))
        assert e_row.max() <= ROW_TOL[dtype], (n, e_row.max())
