"""The plain C entry points race_attn_forward and race_attn_backward, called
through ctypes with device pointers and a caller workspace (no events, no
saved state), against the oracle and against the binding's *_ex calls.

The plain calls run the same plan and kernels as the *_ex calls with null
events and no saved buffer, so the outputs are expected to be bitwise equal;
against the oracle both parity gates apply (per-head Frobenius, per row).
"""
import numpy as np
import pytest
import torch

import oracle
from sketch_attention_soft_amd import binding
from sketch_attention_soft_amd import inputs as I
from tests.gpu_util import (GRAD_FLOOR, ROW_TOL, TOL, device_inputs, head_relf, host_inputs,
                            row_errors, to_host64)

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, B, H, N, L, tau, causal, chunk
    ("bf16", 1, 2, 1500, 8, 1.0, True, 0),
    ("f16", 2, 1, 700, 16, 0.5, False, 0),
    ("f32", 1, 1, 900, 8, 1.0, True, 256),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_plain_entry_points(case):
    dtype, B, H, N, L, tau, causal, chunk = case
    print(f"[case] plain ABI {case}", flush=True)
    x = I.make_inputs(B, H, N, 64, L, 4, dtype, 4242 + N)
    dx = device_inputs(x, dtype)
    q, k, v, do, W = dx["q"], dx["k"], dx["v"], dx["do"], dx["W"]
    code = binding.dtype_code(q.dtype)
    lib = binding.lib()
    stream = torch.cuda.current_stream().cuda_stream

    nf = binding.workspace_bytes(B, H, N, 64, L, 4, causal, chunk, q.dtype, False)
    wsf = torch.empty(max(nf, 1), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    den = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    rc = lib.race_attn_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), W.data_ptr(), L, 4,
                               float(tau), int(causal), B, H, N, 64, code, chunk, o.data_ptr(),
                               den.data_ptr(), wsf.data_ptr(), wsf.numel(), stream)
    assert rc == 0, rc

    nb = binding.workspace_bytes(B, H, N, 64, L, 4, causal, chunk, q.dtype, 1)
    wsb = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    rc = lib.race_attn_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), W.data_ptr(),
                                o.data_ptr(), den.data_ptr(), do.data_ptr(), L, 4, float(tau),
                                int(causal), B, H, N, 64, code, chunk, dq.data_ptr(),
                                dk.data_ptr(), dv.data_ptr(), wsb.data_ptr(), wsb.numel(), stream)
    assert rc == 0, rc

    o2, den2 = binding.forward(q, k, v, W, tau, causal, chunk)
    dq2, dk2, dv2 = binding.backward(q, k, v, W, o2, den2, do, tau, causal, chunk)
    torch.cuda.synchronize()
    same = all(torch.equal(a, b) for a, b in ((o, o2), (den, den2), (dq, dq2), (dk, dk2), (dv, dv2)))
    print(f"  bitwise equal to the *_ex calls: {same}", flush=True)
    assert same

    h = host_inputs(x, dtype)
    ref = oracle.forward_backward(h["q"], h["k"], h["v"], h["do"], h["W"], tau, causal)
    got = {"o": o, "den": den, "dq": dq, "dk": dk, "dv": dv}
    want = dict(zip(("o", "den", "dq", "dk", "dv"), ref[:5]))
    for name in ("o", "den", "dq", "dk", "dv"):
        g = to_host64(got[name])
        e = head_relf(g, want[name])
        floor = GRAD_FLOOR if name in ("dq", "dk") else 0.05
        vanish = (0,) if (name == "dq" and causal) else ()
        rows = row_errors(g, want[name], floor=floor, vanishing=vanish) if name != "den" else \
            row_errors(g[..., None], want[name][..., None])
        print(f"  {name}: rel={e:.2e} rows_max={rows.max():.2e}", flush=True)
        assert np.all(np.isfinite(g))
        assert e <= TOL[dtype], (name, e)
        assert rows.max() <= ROW_TOL[dtype], (name, rows.max())
