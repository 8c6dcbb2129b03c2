"""Hard-hash forward (race_attn_forward_hard) against the oracle's hard mode.

Pages (title "RACE Attention: A Strictly Linear-Time Attention for
Long-Sequence Training", gist.science/zh/paper/2510.04008, technical summary
§2.2 and §3): soft hashing replaces the one-bucket-per-table assignment of the
original RACE sketch; with tau -> 0 the corner softmax becomes that hard
assignment, and the bucket sums are true counts.  The oracle's hard mode is
pinned by the SimHash collision rate (P-4) and the convergence to angular
attention (P-7).  Bar: the parity bar; with fp32 inputs den, a sum of
collision counts, must be an exact integer.
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
    # dtype, B, H, N, L, causal, chunk
    ("bf16", 1, 2, 1000, 8, True, 0),
    ("bf16", 1, 1, 4133, 32, True, 256),
    ("bf16", 2, 1, 333, 5, False, 0),
    ("bf16", 1, 1, 1500, 64, True, 128),
    ("f32", 1, 2, 777, 16, True, 0),
    ("f32", 1, 1, 500, 32, False, 64),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s_B%dH%dN%dL%d_c%d_ch%d" % c)
def test_hard_forward_matches_the_oracle(case):
    dtype, B, H, N, L, causal, chunk = case
    x = I.make_inputs(B, H, N, 64, L, 4, dtype, 1300 + N + L, with_grad=False)
    dx, hx = device_inputs(x, dtype), host_inputs(x, dtype)
    print(f"[case] hard {dtype} B={B} H={H} N={N} L={L} causal={causal}", flush=True)
    o, den = binding.forward_hard(dx["q"], dx["k"], dx["v"], dx["W"], causal, chunk)
    torch.cuda.synchronize()
    ro, rden = oracle.forward(hx["q"], hx["k"], hx["v"], hx["W"], 1.0, causal, hard=True)
    d = to_host64(den)
    if dtype == "f32":
        # den counts (table, key) collisions: with fp32 states an exact integer,
        # equal to the oracle's count (a bucket decided by a projection within
        # fp32 rounding of zero would be the only exception)
        assert np.array_equal(d, np.round(d))
        assert np.mean(d == rden) >= 0.999
    # (bf16: the state is read as bf16 MFMA operands, so counts above 256 are
    # rounded to 8 bits; the parity bar covers that)
    assert head_relf(to_host64(o), ro) <= TOL[dtype]
    assert head_relf(d, rden) <= TOL[dtype]


def test_hard_forward_first_row_and_self_collisions():
    """Causal row 0 sees only its own key, which collides with its query in
    every table when q = k: o_0 = v_0 and den_0 = L."""
    B, H, N, L = 1, 1, 64, 32
    x = I.make_inputs(B, H, N, 64, L, 4, "bf16", 77, with_grad=False)
    dx = device_inputs(x, "bf16")
    o, den = binding.forward_hard(dx["k"], dx["k"], dx["v"], dx["W"], True)
    torch.cuda.synchronize()
    assert torch.equal(den[0, 0, 0], torch.tensor(float(L), device=den.device))
    assert torch.allclose(o[0, 0, 0].float(), dx["v"][0, 0, 0].float(), rtol=1e-2, atol=1e-3)
    # with q = k every row collides with its own key in all L tables
    assert torch.all(den[0, 0] >= L)
