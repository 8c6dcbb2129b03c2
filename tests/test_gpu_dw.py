"""The projection gradient dW (race_attn_backward_dw, learned hyperplanes)
against the fp64 oracle (its dW is pinned by finite differences, P-14).

dW = sum over the rows x of Q and K of dLoss/du (x / max(|x|, 1e-12))^T with
u = W x_hat: the chain rule of the backward continued to the projection of
the pages' step 1 (gist.science/zh/paper/2510.04008, technical summary §2.2).
Bar: the bf16 parity bar, 2e-2 relative Frobenius.
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
    # B, H, N, L, tau, causal, chunk
    (1, 1, 257, 8, 1.0, True, 0),
    (2, 1, 333, 5, 0.5, True, 64),
    (1, 2, 1000, 32, 1.0, True, 0),
    (1, 1, 700, 16, 0.7, False, 0),
    (1, 1, 4133, 32, 1.0, True, 256),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dH%dN%dL%d_tau%g_c%d_ch%d" % c)
def test_dw_matches_the_oracle(case):
    B, H, N, L, tau, causal, chunk = case
    x = I.make_inputs(B, H, N, 64, L, 4, "bf16", 900 + N + L, with_grad=True)
    dx, hx = device_inputs(x, "bf16"), host_inputs(x, "bf16")
    print(f"[case] dW B={B} H={H} N={N} L={L} causal={causal}", flush=True)
    o, den = binding.forward(dx["q"], dx["k"], dx["v"], dx["W"], tau, causal, chunk)
    dq, dk, dv, dW = binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], tau,
                                      causal, chunk, dw=True)
    rq, rk, rv = binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], tau,
                                  causal, chunk)
    torch.cuda.synchronize()
    # asking for dW leaves the other gradients as they are
    assert torch.equal(dq, rq) and torch.equal(dk, rk) and torch.equal(dv, rv)
    ref = oracle.forward_backward(hx["q"], hx["k"], hx["v"], hx["do"], hx["W"], tau, causal,
                                  with_dw=True)
    err = np.linalg.norm(to_host64(dW) - ref[5]) / np.linalg.norm(ref[5])
    print(f"  dW rel err {err:.2e}")
    assert err <= TOL["bf16"]


def test_dw_with_saved_state_and_autograd():
    B, H, N, L, tau = 1, 2, 900, 32, 1.0
    x = I.make_inputs(B, H, N, 64, L, 4, "bf16", 950, with_grad=True)
    dx, hx = device_inputs(x, "bf16"), host_inputs(x, "bf16")
    print("[case] dW autograd", flush=True)
    layer = binding.RaceAttentionLayer(d=64, L=L, P=4, tau=tau, causal=True,
                                       learn_projection=True).cuda()
    with torch.no_grad():
        layer.W.copy_(dx["W"])
    q, k, v = (dx[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    o = layer(q, k, v)
    o.backward(dx["do"])
    torch.cuda.synchronize()
    assert layer.W.grad is not None and layer.W.grad.shape == (L, 4, 64)
    ref = oracle.forward_backward(hx["q"], hx["k"], hx["v"], hx["do"], hx["W"], tau, True,
                                  with_dw=True)
    err = np.linalg.norm(to_host64(layer.W.grad) - ref[5]) / np.linalg.norm(ref[5])
    assert err <= TOL["bf16"]
    for a, r in ((q.grad, ref[2]), (k.grad, ref[3]), (v.grad, ref[4])):
        assert head_relf(to_host64(a), r) <= TOL["bf16"]
    # a fixed projection (the default) gets no gradient and no dW work
    fixed = binding.RaceAttentionLayer(d=64, L=L, P=4, tau=tau).cuda()
    o2 = fixed(q.detach().clone().requires_grad_(True), k, v)
    o2.sum().backward()
    assert not fixed.W.requires_grad and fixed.W.grad is None


def test_dw_unsupported_configurations_raise():
    x = I.make_inputs(1, 1, 64, 64, 8, 4, "f32", 3, with_grad=True)
    dx = device_inputs(x, "f32")
    o, den = binding.forward(dx["q"], dx["k"], dx["v"], dx["W"], 1.0, True)
    with pytest.raises(binding.RaceError):
        binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], 1.0, True, dw=True)
