"""Parity of the streaming state entry points (race_attn_state_add,
race_attn_decode, race_attn_state_readout) against the fp64 oracle.

Pages (title "RACE Attention: A Strictly Linear-Time Attention for
Long-Sequence Training", gist.science/zh/paper/2510.04008, technical summary
§2.3): causal mode keeps running bucket sums and reads them at every step.
So a decode from the empty state must reproduce the causal forward row by row
(pin P-8 of the oracle), a decode after a bulk prefix the rows that follow
it, a readout of a key set's state the non-causal forward over those keys, and
the state itself the oracle's bucket sums in the Walsh basis
(oracle.walsh_state, pin P-13).  Bar: the relative Frobenius error of the
parity tests (1e-4 fp32 inputs, 2e-2 bf16 inputs: the outputs are rounded to
the input type); the state, summed in fp32 either way, to 1e-4.
"""
import numpy as np
import pytest
import torch

import oracle
from sketch_attention_soft_amd import binding
from sketch_attention_soft_amd import inputs as I
from tests.gpu_util import TOL, device_inputs, head_relf, host_inputs, to_host64

pytestmark = pytest.mark.gpu


def _inputs(B, H, N, L, dtype, seed):
    x = I.make_inputs(B, H, N, 64, L, 4, dtype, seed, with_grad=False)
    return device_inputs(x, dtype), host_inputs(x, dtype)


def _oracle_state(hx, N0, tau):
    k, v, W = hx["k"], hx["v"], hx["W"]
    B, H = k.shape[:2]
    return np.stack([np.stack([oracle.walsh_state(k[b, h, :N0], v[b, h, :N0], W, tau)
                               for h in range(H)]) for b in range(B)])


DECODE_CASES = [
    # B, H, N, L, tau
    (1, 1, 1, 8, 1.0),
    (1, 2, 333, 8, 1.0),
    (2, 1, 130, 5, 0.5),
    (1, 1, 257, 32, 1.0),
    (1, 1, 100, 64, 0.7),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "B%dH%dN%dL%d_tau%g" % c)
def test_decode_from_empty_state_is_the_causal_forward(dtype, case):
    B, H, N, L, tau = case
    dx, hx = _inputs(B, H, N, L, dtype, 100 + N + L)
    print(f"[case] decode {dtype} B={B} H={H} N={N} L={L}", flush=True)
    st = binding.new_state(B, H, 64, L, 4, dx["q"].device)
    o, den = binding.decode(st, dx["q"], dx["k"], dx["v"], dx["W"], tau)
    torch.cuda.synchronize()
    ro, rden = oracle.forward(hx["q"], hx["k"], hx["v"], hx["W"], tau, True)
    assert head_relf(to_host64(o), ro) <= TOL[dtype]
    assert head_relf(to_host64(den), rden) <= TOL[dtype]
    # the state after the sequence is the oracle's over all N keys
    assert head_relf(to_host64(st), _oracle_state(hx, N, tau)) <= 1e-4


def test_decode_split_into_calls_is_bitwise_the_same():
    B, H, N, L, tau = 1, 2, 200, 16, 0.8
    dx, _ = _inputs(B, H, N, L, "bf16", 5)
    print("[case] decode split", flush=True)
    s1 = binding.new_state(B, H, 64, L, 4, dx["q"].device)
    o1, d1 = binding.decode(s1, dx["q"], dx["k"], dx["v"], dx["W"], tau)
    s2 = binding.new_state(B, H, 64, L, 4, dx["q"].device)
    parts, a = [], 0
    for t in (1, 7, 64, 3, N - 75):
        sl = slice(a, a + t)
        q, k, v = (dx[n][:, :, sl].contiguous() for n in ("q", "k", "v"))
        parts.append(binding.decode(s2, q, k, v, dx["W"], tau))
        a += t
    torch.cuda.synchronize()
    assert a == N
    assert torch.equal(torch.cat([p[0] for p in parts], 2), o1)
    assert torch.equal(torch.cat([p[1] for p in parts], 2), d1)
    assert torch.equal(s1, s2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_after_bulk_prefix(dtype):
    B, H, N0, T, L, tau = 1, 2, 1000, 37, 32, 1.0
    dx, hx = _inputs(B, H, N0 + T, L, dtype, 77)
    print(f"[case] prefix {dtype} N0={N0} T={T}", flush=True)
    st = binding.new_state(B, H, 64, L, 4, dx["q"].device)
    binding.state_add(st, dx["k"][:, :, :N0].contiguous(), dx["v"][:, :, :N0].contiguous(),
                      dx["W"], tau)
    q, k, v = (dx[n][:, :, N0:].contiguous() for n in ("q", "k", "v"))
    o, den = binding.decode(st, q, k, v, dx["W"], tau)
    torch.cuda.synchronize()
    ro, rden = oracle.forward(hx["q"], hx["k"], hx["v"], hx["W"], tau, True)
    assert head_relf(to_host64(o), ro[:, :, N0:]) <= TOL[dtype]
    assert head_relf(to_host64(den), rden[:, :, N0:]) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("L", [3, 16, 32, 64])
def test_state_add_is_the_oracle_state(dtype, L):
    B, H, N, tau = 2, 1, 3001, 0.6
    dx, hx = _inputs(B, H, N, L, dtype, 200 + L)
    print(f"[case] state_add {dtype} L={L}", flush=True)
    st = binding.new_state(B, H, 64, L, 4, dx["q"].device)
    binding.state_add(st, dx["k"], dx["v"], dx["W"], tau)
    torch.cuda.synchronize()
    assert head_relf(to_host64(st), _oracle_state(hx, N, tau)) <= 1e-4
    # appending in two calls sums the same keys
    s2 = binding.new_state(B, H, 64, L, 4, dx["q"].device)
    a = 1234
    binding.state_add(s2, dx["k"][:, :, :a].contiguous(), dx["v"][:, :, :a].contiguous(),
                      dx["W"], tau)
    binding.state_add(s2, dx["k"][:, :, a:].contiguous(), dx["v"][:, :, a:].contiguous(),
                      dx["W"], tau)
    torch.cuda.synchronize()
    assert head_relf(to_host64(s2), to_host64(st)) <= 1e-5


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_readout_of_a_key_state_is_the_non_causal_forward(dtype):
    B, H, N, L, tau = 1, 3, 700, 8, 1.0
    dx, hx = _inputs(B, H, N, L, dtype, 300)
    print(f"[case] readout {dtype}", flush=True)
    st = binding.new_state(B, H, 64, L, 4, dx["q"].device)
    binding.state_add(st, dx["k"], dx["v"], dx["W"], tau)
    before = st.clone()
    o, den = binding.state_readout(st, dx["q"], dx["W"], tau)
    torch.cuda.synchronize()
    assert torch.equal(st, before)
    ro, rden = oracle.forward(hx["q"], hx["k"], hx["v"], hx["W"], tau, False)
    assert head_relf(to_host64(o), ro) <= TOL[dtype]
    assert head_relf(to_host64(den), rden) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_decode_many_heads_one_token(dtype):
    """The decode shape of inference: 64 heads, one new token each, after a
    2048-token prefix added in bulk (the one-token call runs its own
    instance, with the row, W and state loads overlapped)."""
    B, H, N0, L, tau = 4, 16, 2048, 32, 1.0
    dx, hx = _inputs(B, H, N0 + 1, L, dtype, 400)
    print(f"[case] 64 heads x 1 token {dtype}", flush=True)
    st = binding.new_state(B, H, 64, L, 4, dx["q"].device)
    binding.state_add(st, dx["k"][:, :, :N0].contiguous(), dx["v"][:, :, :N0].contiguous(),
                      dx["W"], tau)
    q, k, v = (dx[n][:, :, N0:].contiguous() for n in ("q", "k", "v"))
    o, den = binding.decode(st, q, k, v, dx["W"], tau)
    torch.cuda.synchronize()
    ro, rden = oracle.forward(hx["q"], hx["k"], hx["v"], hx["W"], tau, True)
    assert head_relf(to_host64(o), ro[:, :, N0:]) <= TOL[dtype]
    assert head_relf(to_host64(den), rden[:, :, N0:]) <= TOL[dtype]


def test_decode_agrees_with_the_forward_kernels():
    B, H, N, L, tau = 1, 1, 4096, 32, 1.0
    dx, _ = _inputs(B, H, N, L, "bf16", 500)
    print("[case] decode vs forward kernels", flush=True)
    st = binding.new_state(B, H, 64, L, 4, dx["q"].device)
    o, den = binding.decode(st, dx["q"], dx["k"], dx["v"], dx["W"], tau)
    fo, fden = binding.forward(dx["q"], dx["k"], dx["v"], dx["W"], tau, True)
    torch.cuda.synchronize()
    assert head_relf(to_host64(o), to_host64(fo)) <= TOL["bf16"]
    assert head_relf(to_host64(den), to_host64(fden)) <= TOL["bf16"]


def test_empty_calls_leave_the_state():
    dx, _ = _inputs(1, 1, 16, 8, "f32", 600)
    st = binding.new_state(1, 1, 64, 8, 4, dx["q"].device)
    binding.state_add(st, dx["k"], dx["v"], dx["W"], 1.0)
    before = st.clone()
    e = dx["q"][:, :, :0].contiguous()
    o, den = binding.decode(st, e, e, e, dx["W"], 1.0)
    binding.state_add(st, e, e, dx["W"], 1.0)
    torch.cuda.synchronize()
    assert o.shape == (1, 1, 0, 64) and den.shape == (1, 1, 0)
    assert torch.equal(st, before)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("L,P,d", [(32, 4, 64), (5, 4, 64), (16, 3, 32)])
def test_fast_state_add(dtype, L, P, d):
    """The bulk add through the fused segment sum gives the oracle's state to
    the bf16 parity bar, the fp32 add's state to the same, and a decode after
    it the oracle's causal rows."""
    B, H, N, N0, tau = 2, 1, 3001, 2900, 0.8
    x = I.make_inputs(B, H, N, d, L, P, dtype, 2300 + L + d, with_grad=False)
    dx, hx = device_inputs(x, dtype), host_inputs(x, dtype)
    print(f"[case] fast state_add {dtype} L={L} P={P} d={d}", flush=True)
    k0, v0 = dx["k"][:, :, :N0].contiguous(), dx["v"][:, :, :N0].contiguous()
    fast = binding.new_state(B, H, d, L, P, dx["q"].device)
    exact = binding.new_state(B, H, d, L, P, dx["q"].device)
    binding.state_add(fast, k0, v0, dx["W"], tau, fast=True)
    binding.state_add(exact, k0, v0, dx["W"], tau)
    q, k, v = (dx[n][:, :, N0:].contiguous() for n in ("q", "k", "v"))
    o, den = binding.decode(fast, q, k, v, dx["W"], tau)
    torch.cuda.synchronize()
    R = 1 << P
    ref = np.stack([np.stack([oracle.walsh_state(hx["k"][b, h, :N0], hx["v"][b, h, :N0], hx["W"], tau)
                              for h in range(H)]) for b in range(B)]).reshape(B, H, L, R, d + 1)
    ex = to_host64(exact).reshape(B, H, L, 16, d + 1)[:, :, :, :R]
    assert head_relf(ex.reshape(B, H, -1, d + 1), ref.reshape(B, H, -1, d + 1)) <= 1e-4
    # the fast state after the prefix is not observed directly (decode moved it
    # on); rebuild it once more for the state comparison
    fast2 = binding.new_state(B, H, d, L, P, dx["q"].device)
    binding.state_add(fast2, k0, v0, dx["W"], tau, fast=True)
    torch.cuda.synchronize()
    fs = to_host64(fast2).reshape(B, H, L, 16, d + 1)
    assert not np.any(fs[:, :, :, R:])
    assert head_relf(fs[:, :, :, :R].reshape(B, H, -1, d + 1), ref.reshape(B, H, -1, d + 1)) <= TOL["bf16"]
    ro, rden = oracle.forward(hx["q"], hx["k"], hx["v"], hx["W"], tau, True)
    assert head_relf(to_host64(o), ro[:, :, N0:]) <= TOL[dtype]
    assert head_relf(to_host64(den), rden[:, :, N0:]) <= TOL[dtype]
