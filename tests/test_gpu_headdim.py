"""Head dimensions other than 64 against the fp64 oracle: d = 32 on the fused
path (bf16 and fp16 rows, L <= 32: forward, backward with and without the
saved state, dW, the hard forward) and any d <= 64 on the streaming state.

The method does not depend on d (pages: "RACE Attention: A Strictly
Linear-Time Attention for Long-Sequence Training",
gist.science/zh/paper/2510.04008, technical summary §2.2: rows are normalised
and projected by W[L][P][d]); the kernels stage d = 32 rows into their 64
columns with zeros, which changes no sum.  Bar: the parity bar of the storage
type (2e-2 for 16-bit rows).
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
    # dtype, B, H, N, L, tau, chunk
    ("bf16", 1, 1, 1, 8, 1.0, 0),
    ("bf16", 1, 2, 100, 5, 0.5, 16),
    ("f16", 2, 1, 257, 16, 1.0, 64),
    ("bf16", 1, 1, 4133, 32, 1.0, 256),
    ("f16", 1, 2, 2048, 32, 0.5, 0),
]


def _inputs(dtype, B, H, N, d, L, seed, grad=True):
    x = I.make_inputs(B, H, N, d, L, 4, dtype, seed, with_grad=grad)
    return device_inputs(x, dtype), host_inputs(x, dtype)


@pytest.mark.parametrize("saved", [False, True], ids=["recompute", "saved"])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s_B%dH%dN%dL%d_tau%g_ch%d" % c)
def test_d32_forward_backward(case, causal, saved):
    dtype, B, H, N, L, tau, chunk = case
    dx, hx = _inputs(dtype, B, H, N, 32, L, 1700 + N + L + causal)
    print(f"[case] d=32 {dtype} B={B} H={H} N={N} L={L} causal={causal} saved={saved}", flush=True)
    sv = binding.new_saved(dx["q"], dx["W"], causal, chunk) if saved else None
    o, den = binding.forward(dx["q"], dx["k"], dx["v"], dx["W"], tau, causal, chunk, saved=sv)
    dq, dk, dv = binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], tau,
                                  causal, chunk, saved=sv)
    torch.cuda.synchronize()
    assert o.shape == (B, H, N, 32) and dq.shape == (B, H, N, 32)
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
        assert e <= TOL[dtype], (n, e)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_d32_dw(dtype):
    B, H, N, L, tau = 1, 2, 1000, 32, 1.0
    dx, hx = _inputs(dtype, B, H, N, 32, L, 1750)
    print(f"[case] d=32 dW {dtype}", flush=True)
    o, den = binding.forward(dx["q"], dx["k"], dx["v"], dx["W"], tau, True)
    dq, dk, dv, dW = binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], tau,
                                      True, dw=True)
    torch.cuda.synchronize()
    assert dW.shape == (L, 4, 32)
    ref = oracle.forward_backward(hx["q"], hx["k"], hx["v"], hx["do"], hx["W"], tau, True,
                                  with_dw=True)
    err = np.linalg.norm(to_host64(dW) - ref[5]) / np.linalg.norm(ref[5])
    print(f"  dW rel err {err:.2e}")
    assert err <= TOL[dtype]


def test_d32_hard_forward():
    B, H, N, L = 1, 2, 1000, 16
    dx, hx = _inputs("bf16", B, H, N, 32, L, 1760, grad=False)
    print("[case] d=32 hard", flush=True)
    o, den = binding.forward_hard(dx["q"], dx["k"], dx["v"], dx["W"], True)
    torch.cuda.synchronize()
    ro, rden = oracle.forward(hx["q"], hx["k"], hx["v"], hx["W"], 1.0, True, hard=True)
    hit = (rden > 0) & (to_host64(den) > 0)
    assert np.mean(hit) > 0.99
    assert head_relf(np.where(hit[..., None], to_host64(o), 0.0),
                     np.where(hit[..., None], ro, 0.0)) <= TOL["bf16"]


def test_d32_agrees_with_zero_padded_d64():
    """d = 32 rows give what d = 64 rows with 32 zero columns (and W with 32
    zero columns) give, on the same kernels: to rounding (the two launches
    differ only in which columns are read from memory)."""
    B, H, N, L, tau = 1, 1, 3000, 32, 1.0
    dx, _ = _inputs("bf16", B, H, N, 32, L, 1770)
    print("[case] d=32 vs padded d=64", flush=True)
    pad = lambda t: torch.nn.functional.pad(t, (0, 32)).contiguous()
    o, den = binding.forward(dx["q"], dx["k"], dx["v"], dx["W"], tau, True)
    dq, dk, dv = binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], tau, True)
    o6, den6 = binding.forward(pad(dx["q"]), pad(dx["k"]), pad(dx["v"]), pad(dx["W"]), tau, True)
    dq6, dk6, dv6 = binding.backward(pad(dx["q"]), pad(dx["k"]), pad(dx["v"]), pad(dx["W"]), o6,
                                     den6, pad(dx["do"]), tau, True)
    torch.cuda.synchronize()
    assert torch.equal(o, o6[..., :32]) and torch.equal(den, den6)
    assert torch.equal(dq, dq6[..., :32]) and torch.equal(dk, dk6[..., :32])
    assert torch.equal(dv, dv6[..., :32])
    assert not torch.any(o6[..., 32:]) and not torch.any(dq6[..., 32:])


@pytest.mark.parametrize("d", [8, 32, 48])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_stream_any_head_dim(dtype, d):
    B, H, N, N0, L, tau = 1, 2, 400, 150, 16, 0.8
    dx, hx = _inputs(dtype, B, H, N, d, L, 1780 + d, grad=False)
    print(f"[case] stream d={d} {dtype}", flush=True)
    st = binding.new_state(B, H, d, L, 4, dx["q"].device)
    assert st.shape == (B, H, 16 * L, d + 1)
    binding.state_add(st, dx["k"][:, :, :N0].contiguous(), dx["v"][:, :, :N0].contiguous(),
                      dx["W"], tau)
    q, k, v = (dx[n][:, :, N0:].contiguous() for n in ("q", "k", "v"))
    o, den = binding.decode(st, q, k, v, dx["W"], tau)
    ro2, rden2 = binding.state_readout(st, dx["q"], dx["W"], tau)
    torch.cuda.synchronize()
    ro, rden = oracle.forward(hx["q"], hx["k"], hx["v"], hx["W"], tau, True)
    assert head_relf(to_host64(o), ro[:, :, N0:]) <= TOL[dtype]
    assert head_relf(to_host64(den), rden[:, :, N0:]) <= TOL[dtype]
    nro, nrden = oracle.forward(hx["q"], hx["k"], hx["v"], hx["W"], tau, False)
    assert head_relf(to_host64(ro2), nro) <= TOL[dtype]
    assert head_relf(to_host64(rden2), nrden) <= TOL[dtype]
    ws = np.stack([np.stack([oracle.walsh_state(hx["k"][b, h], hx["v"][b, h], hx["W"], tau)
                             for h in range(H)]) for b in range(B)])
    assert head_relf(to_host64(st), ws) <= 1e-4
