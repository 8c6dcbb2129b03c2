"""Tables of P = 5 and 6 hyperplanes (32 and 64 soft buckets) on the fused
16-bit kernels against the fp64 oracle, whose soft assignment is the plain
softmax over the 2^P corners for any P (pinned at P = 5, 6 by the quadratic
closed form, P-3, and by finite differences, P-9).

Pages: "RACE Attention: A Strictly Linear-Time Attention for Long-Sequence
Training", gist.science/zh/paper/2510.04008, technical summary §2.2 (P
hyperplanes per table, 2^P corners) and §3 (L, P as the method's
hyper-parameters).  The kernels take a table of 2^P features as 2^(P-4)
virtual tables of 16 (the features of hyperplanes 0..3 times those of 4, 5),
whose kernels add up to the table's.  Bars: the Frobenius bar of the storage
type per head and ten times it per row (tests/gpu_util), on un-normalised and
zero rows as well as unit ones.
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
    # dtype, P, B, H, N, L, tau, causal, chunk, row_scale, saved, dw
    ("bf16", 5, 1, 2, 4133, 8, 1.0, True, 256, False, True, True),     # 16 virtual tables
    ("bf16", 6, 1, 1, 2600, 8, 1.0, True, 0, True, False, True),       # 32: one pass
    ("bf16", 6, 2, 1, 1000, 3, 0.5, False, 0, False, True, True),
    ("bf16", 6, 1, 1, 1500, 4, 0.25, True, 64, True, True, False),     # direct squash
    ("f16", 5, 1, 2, 1500, 5, 1.0, True, 64, True, True, True),
    ("f16", 6, 1, 1, 1, 4, 1.0, True, 0, False, False, False),         # one token
    ("bf16", 5, 1, 1, 2000, 24, 1.0, True, 0, False, True, True),      # 48: two passes
    ("bf16", 6, 1, 1, 1200, 12, 0.5, True, 0, True, False, True),
    ("f16", 6, 1, 1, 700, 33, 1.0, False, 0, False, True, False),      # 132: five passes
]


def _ids(c):
    return "%s_P%d_B%dH%dN%dL%d_tau%g_c%d_ch%d_rs%d_sv%d_dw%d" % c


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_planes56_forward_backward(case):
    dtype, P, B, H, N, L, tau, causal, chunk, row_scale, saved, dw = case
    seed = 5600 + 11 * P + N + L
    x = I.make_inputs(B, H, N, 64, L, P, dtype, seed, with_grad=True, row_scale=row_scale)
    dx, hx = device_inputs(x, dtype), host_inputs(x, dtype)
    assert dx["W"].shape == (L, P, 64)
    print(f"[case] P={P} {dtype} B={B} H={H} N={N} L={L} tau={tau} causal={causal} "
          f"chunk={chunk} row_scale={row_scale} saved={saved} dw={dw}", flush=True)
    sv = binding.new_saved(dx["q"], dx["W"], causal, chunk) if saved else None
    o, den = binding.forward(dx["q"], dx["k"], dx["v"], dx["W"], tau, causal, chunk, saved=sv)
    grads = binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], tau, causal,
                             chunk, saved=sv, dw=dw)
    torch.cuda.synchronize()
    ref = oracle.forward_backward(hx["q"], hx["k"], hx["v"], hx["do"], hx["W"], tau, causal,
                                  with_dw=dw)
    _compare("o", to_host64(o), ref[0], dtype)
    e_den = np.abs(to_host64(den) - ref[1]) / ref[1]
    print(f"  den: max rel {e_den.max():.2e}")
    assert e_den.max() <= ROW_TOL[dtype]
    if N == 1:
        # one token: o = v and the exact dQ, dK vanish (rounding noise on dV's scale)
        for g in grads[:2]:
            assert np.linalg.norm(to_host64(g)) <= 2 * TOL[dtype] * np.linalg.norm(ref[4])
    else:
        _compare("dq", to_host64(grads[0]), ref[2], dtype, _row_norms(hx["q"]),
                 vanishing=(0,) if causal else ())
        _compare("dk", to_host64(grads[1]), ref[3], dtype, _row_norms(hx["k"]))
    _compare("dv", to_host64(grads[2]), ref[4], dtype)
    if dw:
        e = np.linalg.norm(to_host64(grads[3]) - ref[5]) / np.linalg.norm(ref[5])
        print(f"  rel_dW={e:.2e}")
        assert e <= TOL[dtype]


def test_planes56_recomputed_equals_saved():
    """The backward from the forward's saved state and the one that re-hashes
    give the same gradients (up to the order of bf16 roundings)."""
    B, H, N, L, P, tau = 1, 1, 3000, 6, 6, 1.0
    x = I.make_inputs(B, H, N, 64, L, P, "bf16", 5690, with_grad=True)
    dx = device_inputs(x, "bf16")
    print("[case] P=6 saved vs recomputed", flush=True)
    sv = binding.new_saved(dx["q"], dx["W"], True, 0)
    o, den = binding.forward(dx["q"], dx["k"], dx["v"], dx["W"], tau, True, saved=sv)
    a = binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], tau, True, saved=sv)
    b = binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], tau, True)
    torch.cuda.synchronize()
    for u, w in zip(a, b):
        u, w = to_host64(u), to_host64(w)
        assert np.linalg.norm(u - w) <= 1e-2 * np.linalg.norm(w)
