"""Packed batches (race_attn_forward_varlen / race_attn_backward_varlen):
variable-length sequences back to back in [H, T, d] tensors, delimited by
cu_seqlens.  The method is defined per sequence (gist.science/zh/paper/
2510.04008, technical summary §2.2-2.3: the sketch of one sequence's keys,
read by that sequence's queries), so each sequence is checked against the
oracle on its own rows, and against the right-padded entry points on the
same rows (the same kernels, bitwise).  Bar: the parity bar of the storage
type; per-row gate as tests/gpu_util.row_errors.
"""
import numpy as np
import pytest
import torch

import oracle
from sketch_attention_soft_amd import binding
from sketch_attention_soft_amd import inputs as I
from tests.gpu_util import (GRAD_FLOOR, ROW_FLOOR, ROW_TOL, TOL, device_inputs, head_relf,
                            host_inputs, row_errors, to_host64)

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, d, H, L, P, tau, lengths
    ("bf16", 64, 2, 8, 4, 1.0, (1000, 1, 0, 2500, 777)),
    ("f16", 64, 1, 32, 4, 0.5, (4133, 64, 300)),
    ("bf16", 32, 2, 16, 3, 1.0, (257, 1500)),
    ("bf16", 64, 1, 64, 4, 1.0, (900, 0, 1201)),
    # P = 5, 6: virtual tables (one pass, and two passes of 32)
    ("bf16", 64, 1, 8, 6, 1.0, (700, 1, 1300)),
    ("f16", 64, 2, 12, 5, 0.5, (333, 2000)),
    ("bf16", 64, 1, 12, 6, 1.0, (600, 1111)),
]


def _ids(c):
    return "%s_d%d_H%d_L%d_P%d_tau%g" % c[:6] + "_n" + "-".join(map(str, c[6]))


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_varlen_against_oracle_and_padded(case, causal):
    dtype, d, H, L, P, tau, lens = case
    T = sum(lens)
    B = len(lens)
    cu_h = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    nmax = max(lens)
    x = I.make_inputs(1, H, T, d, L, P, dtype, 5100 + T + L + causal, with_grad=True)
    dx, hx = device_inputs(x, dtype), host_inputs(x, dtype)
    q, k, v, do = (dx[n][0] for n in ("q", "k", "v", "do"))
    cu = torch.from_numpy(cu_h).cuda()
    print(f"[case] varlen {dtype} d={d} H={H} L={L} P={P} causal={causal} lens={lens}", flush=True)
    o, den = binding.forward_varlen(q, k, v, dx["W"], cu, nmax, tau, causal)
    dq, dk, dv, dW = binding.backward_varlen(q, k, v, dx["W"], o, den, do, cu, nmax, tau, causal,
                                            dw=True)
    torch.cuda.synchronize()
    got = {n: to_host64(t) for n, t in (("o", o), ("den", den), ("dq", dq), ("dk", dk), ("dv", dv))}
    dw_ref = np.zeros_like(x["W"], dtype=np.float64)
    for b in range(B):
        s0, s1 = int(cu_h[b]), int(cu_h[b + 1])
        if s1 == s0:
            continue
        sub = {n: hx[n][0, :, s0:s1] for n in ("q", "k", "v", "do")}
        ref = dict(zip(("o", "den", "dq", "dk", "dv", "dW"),
                       oracle.forward_backward(sub["q"], sub["k"], sub["v"], sub["do"], hx["W"],
                                               tau, causal, with_dw=True)))
        dw_ref += ref["dW"]
        for n in ("o", "dq", "dk", "dv"):
            g = got[n][:, s0:s1]
            fr = ref["dv"] if n in ("dq", "dk") else None
            e = head_relf(g, ref[n], floor_ref=fr, floor=1.0 if s1 - s0 == 1 else 1e-3)
            assert np.all(np.isfinite(g)), (b, n)
            # one token: the exact dq, dk vanish and what is measured is
            # rounding noise on dv's scale, which grows with the features
            # (2.0e-2 at P = 6): twice the bar
            bar = 2 * TOL[dtype] if s1 - s0 == 1 and fr is not None else TOL[dtype]
            assert e <= bar, (b, n, e)
            if s1 - s0 > 1:
                er = row_errors(g, ref[n], GRAD_FLOOR if n in ("dq", "dk") else ROW_FLOOR,
                                vanishing=(0,) if n == "dq" and causal else ())
                assert er.max() <= ROW_TOL[dtype], (b, n, er.max())
        assert np.abs(got["den"][:, s0:s1] / ref["den"] - 1).max() <= TOL[dtype]
    e_dw = np.linalg.norm(to_host64(dW) - dw_ref) / np.linalg.norm(dw_ref)
    print(f"  dW rel err {e_dw:.2e}")
    assert e_dw <= TOL[dtype]
    # the padded entry points on the same rows give the same bits
    pad = {n: torch.zeros((B, H, nmax, d), dtype=q.dtype, device="cuda") for n in ("q", "k", "v", "do")}
    for b in range(B):
        s0, s1 = int(cu_h[b]), int(cu_h[b + 1])
        for n, t in (("q", q), ("k", k), ("v", v), ("do", do)):
            pad[n][b, :, :s1 - s0] = t[:, s0:s1]
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    ch = binding.padded_chunk(B, H, nmax)
    po, pden = binding.forward_padded(pad["q"], pad["k"], pad["v"], dx["W"], sl, tau, causal, ch)
    pdq, pdk, pdv = binding.backward_padded(pad["q"], pad["k"], pad["v"], dx["W"], po, pden,
                                            pad["do"], sl, tau, causal, ch)
    torch.cuda.synchronize()
    for b in range(B):
        s0, s1 = int(cu_h[b]), int(cu_h[b + 1])
        for a, p_ in ((o, po), (dq, pdq), (dk, pdk), (dv, pdv)):
            assert torch.equal(a[:, s0:s1], p_[b, :, :s1 - s0]), b
        assert torch.equal(den[:, s0:s1], pden[b, :, :s1 - s0])


def test_varlen_rejects_fp32_and_bad_lengths():
    q = torch.zeros((1, 100, 64), dtype=torch.float32, device="cuda")
    W = torch.zeros((8, 4, 64), dtype=torch.float32, device="cuda")
    cu = torch.tensor([0, 60, 100], dtype=torch.int32, device="cuda")
    with pytest.raises(binding.RaceError) as e:
        binding.forward_varlen(q, q, q, W, cu, 60, 1.0, True)
    assert e.value.code == 3  # RACE_ERR_UNSUPPORTED
    qb = q.to(torch.bfloat16)
    with pytest.raises(binding.RaceError) as e:      # T = 100 > B * max_seqlen = 2 * 40
        binding.forward_varlen(qb, qb, qb, W, cu, 40, 1.0, True)
    assert e.value.code == 2  # RACE_ERR_SHAPE
