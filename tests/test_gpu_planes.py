"""Fewer hyperplanes per table (P = 1, 2, 3) against the fp64 oracle, whose
soft assignment is the plain softmax over the 2^P corners for any P (pinned
for P = 1 by the logistic closed form, P-12, and for P = 2, 3 by the finite
differences of P-9).

Pages: "RACE Attention: A Strictly Linear-Time Attention for Long-Sequence
Training", gist.science/zh/paper/2510.04008, technical summary §2.2 (P
hyperplanes per table, 2^P corners) and §3 (L, P as the method's
hyper-parameters).  The kernels keep four hyperplanes per table and give the
padding ones t = 0, so each table's kernel is exactly the P-plane corner
product.  Bar: the parity bar of the storage type.
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
    # dtype, P, d, B, H, N, L, tau, chunk
    ("bf16", 1, 64, 1, 2, 333, 8, 1.0, 0),
    ("bf16", 2, 64, 2, 1, 1000, 16, 0.5, 64),
    ("bf16", 3, 64, 1, 1, 4133, 32, 1.0, 256),
    ("f16", 3, 32, 1, 2, 700, 5, 1.0, 0),
    ("f16", 2, 64, 1, 1, 1, 8, 1.0, 0),
]


def _inputs(dtype, B, H, N, d, L, P, seed, grad=True):
    x = I.make_inputs(B, H, N, d, L, P, dtype, seed, with_grad=grad)
    return device_inputs(x, dtype), host_inputs(x, dtype)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s_P%d_d%d_B%dH%dN%dL%d_tau%g_ch%d" % c)
def test_planes_forward_backward(case, causal):
    dtype, P, d, B, H, N, L, tau, chunk = case
    dx, hx = _inputs(dtype, B, H, N, d, L, P, 1800 + 7 * P + N + L + causal)
    print(f"[case] P={P} d={d} {dtype} B={B} H={H} N={N} L={L} causal={causal}", flush=True)
    assert dx["W"].shape == (L, P, d)
    sv = binding.new_saved(dx["q"], dx["W"], causal, chunk)
    o, den = binding.forward(dx["q"], dx["k"], dx["v"], dx["W"], tau, causal, chunk, saved=sv)
    dq, dk, dv = binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], tau,
                                  causal, chunk, saved=sv)
    dq2, dk2, dv2 = binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], tau,
                                     causal, chunk)
    torch.cuda.synchronize()
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
    # the recomputed backward agrees with the one from the saved state
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert head_relf(to_host64(a), to_host64(b), to_host64(dv), 1e-3) <= 1e-2


@pytest.mark.parametrize("P", [1, 3])
def test_planes_dw(P):
    B, H, N, L, tau = 1, 2, 900, 16, 1.0
    dx, hx = _inputs("bf16", B, H, N, 64, L, P, 1850 + P)
    print(f"[case] P={P} dW", flush=True)
    o, den = binding.forward(dx["q"], dx["k"], dx["v"], dx["W"], tau, True)
    dq, dk, dv, dW = binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], tau,
                                      True, dw=True)
    torch.cuda.synchronize()
    assert dW.shape == (L, P, 64)
    ref = oracle.forward_backward(hx["q"], hx["k"], hx["v"], hx["do"], hx["W"], tau, True,
                                  with_dw=True)
    err = np.linalg.norm(to_host64(dW) - ref[5]) / np.linalg.norm(ref[5])
    print(f"  dW rel err {err:.2e}")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("P", [1, 2, 3])
def test_planes_hard_forward(P):
    B, H, N, L = 1, 2, 1000, 8
    dx, hx = _inputs("bf16", B, H, N, 64, L, P, 1870 + P, grad=False)
    print(f"[case] P={P} hard", flush=True)
    o, den = binding.forward_hard(dx["q"], dx["k"], dx["v"], dx["W"], False)
    torch.cuda.synchronize()
    ro, rden = oracle.forward(hx["q"], hx["k"], hx["v"], hx["W"], 1.0, False, hard=True)
    d = to_host64(den)
    # den counts (table, key) collisions over 2^P buckets per table (rounded:
    # the state is read as bf16 operands)
    hit = (rden > 0) & (d > 0)
    assert np.mean(hit) > 0.99
    assert head_relf(np.where(hit[..., None], to_host64(o), 0.0),
                     np.where(hit[..., None], ro, 0.0)) <= TOL["bf16"]
    assert head_relf(d, rden) <= TOL["bf16"]


@pytest.mark.parametrize("P", [2, 4])
def test_gradients_are_deterministic(P):
    """The gradient kernels give the same bits on every call.  (Their first
    chunk reads LDS selection operands that one wave stages; with P <= 2 some
    waves stage only zero W rows and used to reach that read before it was
    written.)"""
    B, H, N, L, tau, chunk = 2, 1, 1000, 16, 0.5, 64
    dx, _ = _inputs("bf16", B, H, N, 64, L, P, 1890 + P)
    print(f"[case] P={P} determinism", flush=True)
    o, den = binding.forward(dx["q"], dx["k"], dx["v"], dx["W"], tau, True, chunk)
    outs = [binding.backward(dx["q"], dx["k"], dx["v"], dx["W"], o, den, dx["do"], tau, True,
                             chunk) for _ in range(3)]
    torch.cuda.synchronize()
    for rep in outs[1:]:
        for a, b in zip(outs[0], rep):
            assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("P", [1, 2, 3])
def test_planes_streaming_state(dtype, P):
    """Streaming state at P < 4: decode from the empty state is the causal
    forward, readout the non-causal one, and the state's rows are the oracle's
    Walsh-basis state (scale 2^(-P/2)), the 16 - 2^P rows per table that
    contain a padding hyperplane being zero."""
    B, H, N, N0, L, tau = 1, 2, 300, 120, 8, 0.9
    R = 1 << P
    dx, hx = _inputs(dtype, B, H, N, 64, L, P, 1990 + P, grad=False)
    print(f"[case] P={P} stream {dtype}", flush=True)
    st = binding.new_state(B, H, 64, L, P, dx["q"].device)
    assert st.shape == (B, H, 16 * L, 65)
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
    s = to_host64(st).reshape(B, H, L, 16, 65)
    assert not np.any(s[:, :, :, R:])
    ws = np.stack([np.stack([oracle.walsh_state(hx["k"][b, h], hx["v"][b, h], hx["W"], tau)
                             for h in range(H)]) for b in range(B)]).reshape(B, H, L, R, 65)
    assert head_relf(s[:, :, :, :R].reshape(B, H, L * R, 65), ws.reshape(B, H, L * R, 65)) <= 1e-4
