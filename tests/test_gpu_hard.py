"""Hard-hash forward (race_attn_forward_hard, _counts) against the oracle's
hard mode.

Pages (title "RACE Attention: A Strictly Linear-Time Attention for
Long-Sequence Training", gist.science/zh/paper/2510.04008, technical summary
§2.2 and §3): soft hashing replaces the one-bucket-per-table assignment of the
original RACE sketch; with tau -> 0 the corner softmax becomes that hard
assignment, and the bucket sums are true counts.  The oracle's hard mode is
pinned by the SimHash collision rate (P-4) and the convergence to angular
attention (P-7).

16-bit rows with L <= 32, P <= 4 (or L 2^(P-4) <= 32 for P = 5, 6: each table
as 2^(P-4) virtual tables of 16 buckets) run on integer bucket ids: every row's int32
count sum_l A_l[r_l(q_i)] must equal the oracle's exactly, except on rows that
a bucket decided within fp32 rounding of zero can reach (a query id that
differs from the oracle's, or, causal, any row after a key id that does);
the number of such ids is reported.  o: the parity bar.  Other shapes (fp32
rows, L > 32) run the soft kernels with t = +-1.
"""
import numpy as np
import pytest
import torch

import oracle
from sketch_attention_soft_amd import binding
from sketch_attention_soft_amd import inputs as I
from tests.gpu_util import TOL, device_inputs, head_relf, host_inputs, to_host64

pytestmark = pytest.mark.gpu

ID_CASES = [
    # dtype, d, B, H, N, L, P, causal, chunk
    ("bf16", 64, 1, 2, 1000, 8, 4, True, 0),
    ("bf16", 64, 1, 1, 4133, 32, 4, True, 256),
    ("bf16", 64, 2, 1, 333, 5, 4, False, 0),
    ("f16", 64, 1, 1, 3000, 16, 4, True, 0),
    ("bf16", 32, 1, 2, 1200, 32, 3, True, 64),
    ("f16", 32, 2, 1, 900, 12, 2, False, 0),
    ("bf16", 64, 1, 1, 70000, 32, 4, True, 0),
    # P = 5, 6: each table as 2, 4 virtual tables of 16 buckets
    ("bf16", 64, 1, 2, 1000, 8, 5, True, 0),
    ("bf16", 64, 1, 1, 3000, 8, 6, True, 64),
    ("f16", 32, 2, 1, 700, 3, 6, False, 0),
    ("bf16", 64, 1, 1, 1500, 16, 5, True, 0),
]
DENSE_CASES = [
    ("bf16", 1, 1, 1500, 64, True, 128),
    ("f32", 1, 2, 777, 16, True, 0),
    ("f32", 1, 1, 500, 32, False, 64),
]


def _oracle_ids(x, W):
    phi, _ = oracle.soft_hash(x.reshape(-1, x.shape[-1]), W, 1.0, hard=True)
    return phi.argmax(axis=-1).reshape(*x.shape[:-1], W.shape[0])


@pytest.mark.parametrize("case", ID_CASES, ids=lambda c: "%s_d%d_B%dH%dN%dL%dP%d_c%d_ch%d" % c)
def test_hard_counts_are_exact(case):
    dtype, d, B, H, N, L, P, causal, chunk = case
    x = I.make_inputs(B, H, N, d, L, P, dtype, 1300 + N + L + d, with_grad=False)
    dx, hx = device_inputs(x, dtype), host_inputs(x, dtype)
    print(f"[case] hard ids {dtype} d={d} B={B} H={H} N={N} L={L} P={P} causal={causal}", flush=True)
    o, den, cnt = binding.forward_hard(dx["q"], dx["k"], dx["v"], dx["W"], causal, chunk, counts=True)
    oh, denh = binding.forward_hard(dx["q"], dx["k"], dx["v"], dx["W"], causal, chunk)
    gq = binding.hash_ids(dx["q"], dx["W"]).cpu().numpy()
    gk = binding.hash_ids(dx["k"], dx["W"]).cpu().numpy()
    torch.cuda.synchronize()
    assert torch.equal(o, oh) and torch.equal(den, denh)
    ro, rden = oracle.forward(hx["q"], hx["k"], hx["v"], hx["W"], 1.0, causal, hard=True)
    c = cnt.cpu().numpy().astype(np.int64)
    # a row that meets no visible key: empty sums, o = 0 (as the oracle)
    og = to_host64(o)
    assert np.all(np.isfinite(og)) and np.all(og[c == 0] == 0.0)
    # rows a near-zero decision can reach
    dq = (gq != _oracle_ids(hx["q"], hx["W"])).any(axis=-1)          # [B, H, N]
    dk = (gk != _oracle_ids(hx["k"], hx["W"])).any(axis=-1)
    ok = ~dq
    for b in range(B):
        for h in range(H):
            if dk[b, h].any():
                if causal:
                    ok[b, h, np.argmax(dk[b, h]):] = False
                else:
                    ok[b, h] = False
    print(f"  query ids differing: {int(dq.sum())}, key ids differing: {int(dk.sum())}; "
          f"rows compared: {int(ok.sum())} of {ok.size}")
    assert ok.mean() > 0.9
    assert np.array_equal(c[ok], rden[ok].astype(np.int64))
    assert np.array_equal(to_host64(den)[ok], rden[ok])
    live = ok & (rden > 0)
    e = np.linalg.norm(og[live] - ro[live]) / np.linalg.norm(ro[live])
    print(f"  rel_o={e:.2e}")
    assert e <= TOL[dtype]
    if not causal:
        # rows that collide with no key at all: den = 0 on both sides
        assert np.array_equal(c == 0, rden == 0)


@pytest.mark.parametrize("case", DENSE_CASES, ids=lambda c: "%s_B%dH%dN%dL%d_c%d_ch%d" % c)
def test_hard_forward_other_shapes(case):
    """fp32 rows and L > 32: the soft kernels with t = +-1."""
    dtype, B, H, N, L, causal, chunk = case
    x = I.make_inputs(B, H, N, 64, L, 4, dtype, 1300 + N + L, with_grad=False)
    dx, hx = device_inputs(x, dtype), host_inputs(x, dtype)
    print(f"[case] hard dense {dtype} B={B} H={H} N={N} L={L} causal={causal}", flush=True)
    o, den = binding.forward_hard(dx["q"], dx["k"], dx["v"], dx["W"], causal, chunk)
    torch.cuda.synchronize()
    ro, rden = oracle.forward(hx["q"], hx["k"], hx["v"], hx["W"], 1.0, causal, hard=True)
    d = to_host64(den)
    if dtype == "f32":
        assert np.array_equal(d, np.round(d))
        assert np.mean(d == rden) >= 0.999
    assert head_relf(to_host64(o), ro) <= TOL[dtype]
    assert head_relf(d, rden) <= TOL[dtype]
    with pytest.raises(binding.RaceError):  # no int32 counts on these shapes
        binding.forward_hard(dx["q"], dx["k"], dx["v"], dx["W"], causal, chunk, counts=True)


def test_hard_forward_first_row_and_self_collisions():
    """Causal row 0 sees only its own key, which collides with its query in
    every table when q = k: o_0 = v_0 and the count is L; every row's count is
    at least L."""
    B, H, N, L = 1, 1, 300, 32
    x = I.make_inputs(B, H, N, 64, L, 4, "bf16", 77, with_grad=False)
    dx = device_inputs(x, "bf16")
    o, den, cnt = binding.forward_hard(dx["k"], dx["k"], dx["v"], dx["W"], True, counts=True)
    torch.cuda.synchronize()
    assert int(cnt[0, 0, 0]) == L and float(den[0, 0, 0]) == float(L)
    assert torch.equal(o[0, 0, 0], dx["v"][0, 0, 0])
    assert torch.all(cnt[0, 0] >= L)
