"""Heads of d = 128 against the fp64 oracle (pinned at d = 128 by the
quadratic closed form, P-3, and by finite differences, P-9).

Pages: "RACE Attention: A Strictly Linear-Time Attention for Long-Sequence
Training", gist.science/zh/paper/2510.04008, technical summary §2.2 (the
method on rows of any width d; its cost O(L N R d)).  The library hashes each
128-element row once and runs the fused kernels on value columns 0..63 and
64..127; the gradient's two passes meet in du, and the tail (dx_hat = du W,
the normalisation backward) runs over the whole row.  Bars: the Frobenius
bar of the storage type per head and ten times it per row, on unit, scaled
and zero rows.
"""
import numpy as np
import pytest
import torch

import oracle
from sketch_attention_soft_amd import binding
from sketch_attention_soft_amd import inputs as I
from tests.gpu_util import ROW_TOL, TOL, device_inputs, host_inputs, to_host64
from tests.test_gpu_unnormalised import _compare, _row_norms

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, B, H, N, L, P, tau, causal, chunk, row_scale
    ("bf16", 1, 2, 4133, 32, 4, 1.0, True, 256, False),
    ("bf16", 2, 1, 1000, 8, 4, 0.5, False, 0, True),
    ("bf16", 1, 1, 2600, 16, 3, 1.0, True, 0, True),
    ("bf16", 1, 1, 1500, 5, 4, 0.25, True, 64, False),  # direct squash in the fused kernels' layout
    ("f16", 1, 2, 1800, 32, 4, 1.0, True, 0, True),
    ("f16", 1, 1, 700, 12, 2, 1.0, False, 32, False),
    ("bf16", 1, 1, 1, 8, 4, 1.0, True, 0, False),       # one token
    ("bf16", 1, 1, 37, 8, 4, 1.0, True, 0, False),      # a ragged chunk
]


def _ids(c):
    return "%s_B%dH%dN%dL%dP%d_tau%g_c%d_ch%d_rs%d" % c


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_headdim128_forward_backward(case):
    dtype, B, H, N, L, P, tau, causal, chunk, row_scale = case
    seed = 12800 + N + 3 * L + P
    x = I.make_inputs(B, H, N, 128, L, P, dtype, seed, with_grad=True, row_scale=row_scale)
    dx, hx = device_inputs(x, dtype), host_inputs(x, dtype)
    print(f"[case] d=128 {dtype} B={B} H={H} N={N} L={L} P={P} tau={tau} causal={causal} "
          f"chunk={chunk} row_scale={row_scale}", flush=True)
    o, den = binding.forward(dx["q"], dx["k"], dx["v"], dx["W"], tau, causal, chunk)
    dq, dk, dv = binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], tau,
                                  causal, chunk)
    torch.cuda.synchronize()
    ref = oracle.forward_backward(hx["q"], hx["k"], hx["v"], hx["do"], hx["W"], tau, causal)
    _compare("o", to_host64(o), ref[0], dtype)
    e_den = np.abs(to_host64(den) - ref[1]) / ref[1]
    print(f"  den: max rel {e_den.max():.2e}")
    assert e_den.max() <= ROW_TOL[dtype]
    if N == 1:
        for g in (dq, dk):
            assert np.linalg.norm(to_host64(g)) <= 2 * TOL[dtype] * np.linalg.norm(ref[4])
    else:
        _compare("dq", to_host64(dq), ref[2], dtype, _row_norms(hx["q"]),
                 vanishing=(0,) if causal else ())
        _compare("dk", to_host64(dk), ref[3], dtype, _row_norms(hx["k"]))
    _compare("dv", to_host64(dv), ref[4], dtype)


@pytest.mark.parametrize("causal", [True, False])
def test_headdim128_saved_features(causal):
    """With the forward's saved buffer the backward reads the hash features
    instead of rehashing: the same gradients, bit for bit."""
    B, H, N, L, tau = 1, 2, 1300, 16, 1.0
    x = I.make_inputs(B, H, N, 128, L, 4, "bf16", 12870 + causal, with_grad=True)
    dx = device_inputs(x, "bf16")
    print(f"[case] d=128 saved causal={causal}", flush=True)
    sv = binding.new_saved(dx["q"], dx["W"], causal, 0)
    assert sv is not None
    o, den = binding.forward(dx["q"], dx["k"], dx["v"], dx["W"], tau, causal, saved=sv)
    a = binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], tau, causal, saved=sv)
    b = binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], tau, causal)
    torch.cuda.synchronize()
    for u, w in zip(a, b):
        assert torch.equal(u, w)


def test_headdim128_autograd():
    """The autograd wrapper (forward with a saved buffer, then the backward)
    on d = 128 heads."""
    B, H, N, L, tau = 1, 1, 900, 8, 1.0
    x = I.make_inputs(B, H, N, 128, L, 4, "bf16", 12899, with_grad=True)
    dx, hx = device_inputs(x, "bf16"), host_inputs(x, "bf16")
    print("[case] d=128 autograd", flush=True)
    q, k, v = (dx[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    o = binding.RaceAttention.apply(q, k, v, dx["W"], tau, True, 0)
    o.backward(dx["do"])
    torch.cuda.synchronize()
    ref = oracle.forward_backward(hx["q"], hx["k"], hx["v"], hx["do"], hx["W"], tau, True)
    _compare("o", to_host64(o), ref[0], "bf16")
    _compare("dq", to_host64(q.grad), ref[2], "bf16", _row_norms(hx["q"]), vanishing=(0,))
    _compare("dk", to_host64(k.grad), ref[3], "bf16", _row_norms(hx["k"]))
    _compare("dv", to_host64(v.grad), ref[4], "bf16")
