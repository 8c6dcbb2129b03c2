"""fp16 rows (RACE_F16) against the fp64 oracle: forward, backward (with and
without the saved state), the projection gradient, the hard-hash forward and
the streaming decode.

The method is the same for every storage type (pages: "RACE Attention: A
Strictly Linear-Time Attention for Long-Sequence Training",
gist.science/zh/paper/2510.04008, technical summary §2.2-§2.3); fp16 rows are
read exactly, multiplied as bf16 on the matrix cores with fp32 sums, as bf16
rows are, and the outputs are rounded to fp16.  The oracle takes the exact
fp64 values of the stored fp16 inputs.  Bar: 2e-2 relative Frobenius, the bar
of the bf16 path, whose operand rounding this path shares.
"""
import numpy as np
import pytest
import torch

import oracle
from sketch_attention_soft_amd import binding
from sketch_attention_soft_amd import inputs as I
from tests.gpu_util import TOL, device_inputs, head_relf, host_inputs, to_host64

pytestmark = pytest.mark.gpu

CASES = [
    # B, H, N, L, tau, chunk
    (1, 1, 1, 8, 1.0, 0),
    (1, 2, 100, 5, 0.5, 16),
    (2, 1, 257, 16, 1.0, 64),
    (1, 1, 4133, 32, 1.0, 256),
    (1, 2, 2048, 32, 0.5, 0),
]


def _inputs(B, H, N, L, seed, grad=True):
    x = I.make_inputs(B, H, N, 64, L, 4, "f16", seed, with_grad=grad)
    return device_inputs(x, "f16"), host_inputs(x, "f16")


@pytest.mark.parametrize("saved", [False, True], ids=["recompute", "saved"])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dH%dN%dL%d_tau%g_ch%d" % c)
def test_f16_forward_backward(case, causal, saved):
    B, H, N, L, tau, chunk = case
    dx, hx = _inputs(B, H, N, L, 1500 + N + L + causal)
    print(f"[case] f16 B={B} H={H} N={N} L={L} causal={causal} saved={saved}", flush=True)
    sv = binding.new_saved(dx["q"], dx["W"], causal, chunk) if saved else None
    o, den = binding.forward(dx["q"], dx["k"], dx["v"], dx["W"], tau, causal, chunk, saved=sv)
    dq, dk, dv = binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], tau,
                                  causal, chunk, saved=sv)
    torch.cuda.synchronize()
    assert o.dtype == torch.float16 and dq.dtype == torch.float16
    ref = dict(zip(("o", "den", "dq", "dk", "dv"),
                   oracle.forward_backward(hx["q"], hx["k"], hx["v"], hx["do"], hx["W"], tau,
                                           causal)))
    got = {"o": o, "den": den, "dq": dq, "dk": dk, "dv": dv}
    for n in ("o", "den", "dq", "dk", "dv"):
        g = to_host64(got[n])
        assert np.all(np.isfinite(g)), n
        # dQ and dK floored on dV's scale; N = 1: every query sees only its own
        # key, the exact dQ and dK are zero and the computed ones rounding noise
        fr = ref["dv"] if n in ("dq", "dk") else None
        e = head_relf(g, ref[n], floor_ref=fr, floor=1.0 if N == 1 else 1e-3)
        print(f"  rel_{n}={e:.2e}")
        assert e <= TOL["f16"], (n, e)


def test_f16_dw():
    B, H, N, L, tau = 1, 2, 1000, 32, 1.0
    dx, hx = _inputs(B, H, N, L, 1601)
    print("[case] f16 dW", flush=True)
    o, den = binding.forward(dx["q"], dx["k"], dx["v"], dx["W"], tau, True)
    dq, dk, dv, dW = binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], tau,
                                      True, dw=True)
    torch.cuda.synchronize()
    ref = oracle.forward_backward(hx["q"], hx["k"], hx["v"], hx["do"], hx["W"], tau, True,
                                  with_dw=True)
    err = np.linalg.norm(to_host64(dW) - ref[5]) / np.linalg.norm(ref[5])
    print(f"  dW rel err {err:.2e}")
    assert err <= TOL["f16"]
    assert head_relf(to_host64(dq), ref[2]) <= TOL["f16"]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
def test_f16_hard_forward(causal):
    """fp16 rows with L = 8 run on the bucket ids: every sign of W x is
    decided on the exact product of the stored fp16 row, so the oracle takes
    the same exact values.  Only a projection within fp32 rounding of zero can
    put a row in another bucket; counts must agree on nearly every row, and a
    row that meets no key (count 0) has o = 0 on both sides."""
    B, H, N, L = 1, 2, 1000, 8
    x = I.make_inputs(B, H, N, 64, L, 4, "f16", 1602, with_grad=False)
    dx, hx = device_inputs(x, "f16"), host_inputs(x, "f16")
    print(f"[case] f16 hard causal={causal}", flush=True)
    o, den = binding.forward_hard(dx["q"], dx["k"], dx["v"], dx["W"], causal)
    torch.cuda.synchronize()
    ro, rden = oracle.forward(hx["q"], hx["k"], hx["v"], hx["W"], 1.0, causal, hard=True)
    d, og = to_host64(den), to_host64(o)
    assert np.all(np.isfinite(og))
    assert np.mean(d == rden) >= 0.999
    assert np.all(og[d == 0] == 0.0)
    assert head_relf(og, ro) <= TOL["f16"]
    assert head_relf(d, rden) <= TOL["f16"]


@pytest.mark.parametrize("L", [8, 32, 64])
def test_f16_decode_and_readout(L):
    B, H, N, tau = 1, 2, 300, 1.0
    dx, hx = _inputs(B, H, N, L, 1603 + L, grad=False)
    print(f"[case] f16 decode L={L}", flush=True)
    st = binding.new_state(B, H, 64, L, 4, dx["q"].device)
    o, den = binding.decode(st, dx["q"], dx["k"], dx["v"], dx["W"], tau)
    ro2, rden2 = binding.state_readout(st, dx["q"], dx["W"], tau)
    torch.cuda.synchronize()
    ro, rden = oracle.forward(hx["q"], hx["k"], hx["v"], hx["W"], tau, True)
    assert o.dtype == torch.float16
    assert head_relf(to_host64(o), ro) <= TOL["f16"]
    assert head_relf(to_host64(den), rden) <= TOL["f16"]
    nro, nrden = oracle.forward(hx["q"], hx["k"], hx["v"], hx["W"], tau, False)
    assert head_relf(to_host64(ro2), nro) <= TOL["f16"]
    assert head_relf(to_host64(rden2), nrden) <= TOL["f16"]
