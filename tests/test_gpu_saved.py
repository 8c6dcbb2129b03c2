"""The forward's saved state (key-side segment sums and the fp16 hash
features of Q and K): a backward that reads it agrees with one that
recomputes it, through the C ABI and through the autograd wrapper.  The
forward output is unchanged by saving; the gradients agree to rounding (the
hash features are computed by different kernels), far inside the parity bar.
"""
import pytest
import torch

from sketch_attention_soft_amd import binding
from sketch_attention_soft_amd import inputs as I
from tests.gpu_util import device_inputs


def _relf(a, b):
    a, b = a.double(), b.double()
    return ((a - b).norm() / b.norm().clamp_min(1e-30)).item()

pytestmark = pytest.mark.gpu

CASES = [
    # B, H, N, L, tau, chunk, causal
    (1, 1, 1, 8, 1.0, 0, True),
    (1, 2, 1000, 16, 0.5, 64, True),
    (2, 1, 4133, 32, 1.0, 0, True),
    (1, 1, 3000, 32, 1.0, 256, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dH%dN%dL%d_tau%g_ch%d_c%d" % c)
def test_backward_with_saved_state_is_identical(case):
    B, H, N, L, tau, chunk, causal = case
    x = I.make_inputs(B, H, N, 64, L, 4, "bf16", 11 + N, with_grad=True)
    dx = device_inputs(x, "bf16")
    print(f"[case] B={B} H={H} N={N} L={L} causal={causal}", flush=True)
    saved = binding.new_saved(dx["q"], dx["W"], causal, chunk)
    assert saved is not None and saved.data_ptr() % 256 == 0
    o, den = binding.forward(dx["q"], dx["k"], dx["v"], dx["W"], tau, causal, chunk, saved=saved)
    o2, den2 = binding.forward(dx["q"], dx["k"], dx["v"], dx["W"], tau, causal, chunk)
    ref = binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], tau, causal,
                           chunk)
    got = binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], tau, causal,
                           chunk, saved=saved)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(den, den2)
    for a, b in zip(got, ref):
        e = _relf(a, b)
        print(f"  saved vs recomputed: {e:.2e}")
        assert e <= 1e-2


F32_CASES = [
    # B, H, N, L, tau, chunk, causal
    (1, 1, 1, 8, 1.0, 0, True),
    (1, 2, 1000, 16, 0.5, 64, True),
    (2, 1, 4133, 32, 1.0, 0, True),
    (1, 1, 3000, 32, 1.0, 256, False),
    (1, 2, 777, 40, 1.0, 0, True),  # two table passes, each with its saved rows
]


@pytest.mark.parametrize("case", F32_CASES, ids=lambda c: "B%dH%dN%dL%d_tau%g_ch%d_c%d" % c)
def test_f32_saved_hash_rows_are_bitwise_the_recomputed_ones(case):
    """fp32 rows save t and dt/du' of Q and K: the forward hashes them with the
    same arithmetic the backward would, so outputs and gradients are bitwise
    those without the saved buffer."""
    B, H, N, L, tau, chunk, causal = case
    x = I.make_inputs(B, H, N, 64, L, 4, "f32", 23 + N, with_grad=True)
    dx = device_inputs(x, "f32")
    print(f"[case] f32 B={B} H={H} N={N} L={L} causal={causal}", flush=True)
    saved = binding.new_saved(dx["q"], dx["W"], causal, chunk)
    assert saved is not None and saved.numel() == binding.saved_bytes(B, H, N, 64, L, 4, causal, chunk,
                                                                        torch.float32)
    o, den = binding.forward(dx["q"], dx["k"], dx["v"], dx["W"], tau, causal, chunk, saved=saved)
    o2, den2 = binding.forward(dx["q"], dx["k"], dx["v"], dx["W"], tau, causal, chunk)
    ref = binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], tau, causal, chunk)
    got = binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], tau, causal, chunk,
                           saved=saved)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(den, den2)
    for a, b in zip(got, ref):
        assert torch.equal(a, b)


def test_autograd_wrapper_matches_binding():
    x = I.make_inputs(1, 2, 777, 64, 32, 4, "bf16", 5, with_grad=True)
    dx = device_inputs(x, "bf16")
    q, k, v = (dx[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    o = binding.RaceAttention.apply(q, k, v, dx["W"], 1.0, True, 0)
    o.backward(dx["do"])
    ro, rden = binding.forward(dx["q"], dx["k"], dx["v"], dx["W"], 1.0, True)
    rq, rk, rv = binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], ro, rden, dx["do"], 1.0,
                                  True)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), ro)
    for a, b in ((q.grad, rq), (k.grad, rk), (v.grad, rv)):
        assert _relf(a, b) <= 1e-2
