"""Right-padded batches (race_attn_forward_padded / race_attn_backward_padded)
against the fp64 oracle run on each sequence alone.

A batch of sequences of different lengths, padded to a common N, is the
method applied to each sequence on its own rows (pages: "RACE Attention: A
Strictly Linear-Time Attention for Long-Sequence Training",
gist.science/zh/paper/2510.04008, technical summary §2.2-§2.3: the sketch of a
sequence sums its own keys only).  So batch b's outputs on rows < seqlens[b]
must equal the oracle's on the truncated inputs, in causal and non-causal
mode, and the padding rows must stay zero.  Bar: the parity bar of the
storage type; dW is the sum over the sequences of the oracle's dW.
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
    # dtype, H, N, L, lens, chunk
    ("bf16", 2, 1000, 16, (1000, 617, 1, 0), 64),
    ("bf16", 1, 4133, 32, (4133, 2500, 33), 0),
    ("f16", 2, 300, 8, (300, 31, 129), 0),
    ("f32", 1, 777, 32, (777, 400), 256),
    ("bf16", 1, 600, 64, (600, 250), 128),
]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s_H%dN%dL%d_%s_ch%d" % (
    c[0], c[1], c[2], c[3], "-".join(map(str, c[4])), c[5]))
def test_padded_batches(case, causal):
    dtype, H, N, L, lens, chunk = case
    B, tau = len(lens), 0.8
    x = I.make_inputs(B, H, N, 64, L, 4, dtype, 1900 + N + L + causal, with_grad=True)
    dx, hx = device_inputs(x, dtype), host_inputs(x, dtype)
    print(f"[case] padded {dtype} H={H} N={N} L={L} lens={lens} causal={causal}", flush=True)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o, den = binding.forward_padded(dx["q"], dx["k"], dx["v"], dx["W"], sl, tau, causal, chunk)
    dq, dk, dv = binding.backward_padded(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], sl,
                                         tau, causal, chunk)
    torch.cuda.synchronize()
    got = {n: to_host64(t) for n, t in zip(("o", "den", "dq", "dk", "dv"), (o, den, dq, dk, dv))}
    for b, n_b in enumerate(lens):
        for n in got:
            assert not np.any(got[n][b, :, n_b:]), (b, n)  # padding rows untouched (zeros)
        if n_b == 0:
            continue
        sub = {k_: hx[k_][b:b + 1, :, :n_b] for k_ in ("q", "k", "v", "do")}
        ref = dict(zip(("o", "den", "dq", "dk", "dv"),
                       oracle.forward_backward(sub["q"], sub["k"], sub["v"], sub["do"], hx["W"],
                                               tau, causal)))
        for n in got:
            g = got[n][b:b + 1, :, :n_b]
            assert np.all(np.isfinite(g)), (b, n)
            fr = ref["dv"] if n in ("dq", "dk") else None
            e = head_relf(g, ref[n], floor_ref=fr, floor=1.0 if n_b == 1 else 1e-3)
            print(f"  b={b} len={n_b} rel_{n}={e:.2e}")
            assert e <= TOL[dtype], (b, n, e)


def test_padded_full_lengths_match_the_dense_entry_points():
    """seqlens = N everywhere gives the dense results bit for bit."""
    B, H, N, L, tau = 2, 2, 1500, 32, 1.0
    x = I.make_inputs(B, H, N, 64, L, 4, "bf16", 1950, with_grad=True)
    dx = device_inputs(x, "bf16")
    print("[case] padded = dense", flush=True)
    sl = torch.full((B,), N, dtype=torch.int32, device="cuda")
    o, den = binding.forward(dx["q"], dx["k"], dx["v"], dx["W"], tau, True)
    g = binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], tau, True, dw=True)
    # chunk 0: the dense entry points' segments
    op, denp = binding.forward_padded(dx["q"], dx["k"], dx["v"], dx["W"], sl, tau, True, 0)
    gp = binding.backward_padded(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], sl, tau,
                                 True, 0, dw=True)
    torch.cuda.synchronize()
    assert torch.equal(o, op) and torch.equal(den, denp)
    for a, b in zip(g, gp):
        assert torch.equal(a, b)


def test_padded_dw_is_the_sum_over_sequences():
    H, N, L, tau, lens = 2, 800, 16, 1.0, (800, 333, 0)
    B = len(lens)
    x = I.make_inputs(B, H, N, 64, L, 4, "bf16", 1960, with_grad=True)
    dx, hx = device_inputs(x, "bf16"), host_inputs(x, "bf16")
    print("[case] padded dW", flush=True)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o, den = binding.forward_padded(dx["q"], dx["k"], dx["v"], dx["W"], sl, tau, True)
    *_, dW = binding.backward_padded(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], sl, tau,
                                     True, dw=True)
    torch.cuda.synchronize()
    ref = np.zeros_like(hx["W"])
    for b, n_b in enumerate(lens):
        if n_b:
            sub = {k_: hx[k_][b:b + 1, :, :n_b] for k_ in ("q", "k", "v", "do")}
            ref += oracle.forward_backward(sub["q"], sub["k"], sub["v"], sub["do"], hx["W"], tau,
                                           True, with_dw=True)[5]
    err = np.linalg.norm(to_host64(dW) - ref) / np.linalg.norm(ref)
    print(f"  dW rel err {err:.2e}")
    assert err <= TOL["bf16"]
