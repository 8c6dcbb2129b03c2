"""The allocation-free forward (race_attn_forward_noalloc) against the forward
with a caller workspace (race_attn_forward), through the C ABI.

Two calls in a row share the library's per-GPU scratch array, the second on a
smaller problem, so stale contents of the first call must not leak into the
second.  Bar: the parity bar of the dtype (relative Frobenius, per head);
the two paths run the same kernels on the same plan, so the outputs are
expected to be bitwise equal, which is reported.  A problem whose workspace
exceeds the scratch array is rejected on the host before anything runs.
"""
import numpy as np
import pytest
import torch

from sketch_attention_soft_amd import binding
from sketch_attention_soft_amd import inputs as I
from tests.gpu_util import TOL, device_inputs, head_relf, to_host64

pytestmark = pytest.mark.gpu

CALLS = [
    # dtype, B, H, N, L, tau, causal, chunk: larger first, then smaller
    [("bf16", 1, 2, 20000, 32, 1.0, True, 0), ("bf16", 1, 1, 3000, 16, 0.5, False, 0)],
    [("f32", 2, 1, 9000, 32, 1.0, True, 256), ("f32", 1, 1, 700, 8, 1.0, True, 0)],
    [("f16", 1, 1, 30000, 8, 1.0, True, 0), ("bf16", 1, 1, 129, 64, 1.0, True, 0)],
]


def _one(dtype, B, H, N, L, tau, causal, chunk):
    x = I.make_inputs(B, H, N, 64, L, 4, dtype, 31337 + N + L, with_grad=False)
    dx = device_inputs(x, dtype)
    need = binding.workspace_bytes(B, H, N, 64, L, 4, causal, chunk, dx["q"].dtype, False)
    assert need <= binding.NOALLOC_SCRATCH_BYTES
    print(f"[case] noalloc {dtype} B={B} H={H} N={N} L={L} causal={causal} "
          f"workspace={need} bytes", flush=True)
    o1, d1 = binding.forward_noalloc(dx["q"], dx["k"], dx["v"], dx["W"], tau, causal, chunk)
    o2, d2 = binding.forward(dx["q"], dx["k"], dx["v"], dx["W"], tau, causal, chunk)
    torch.cuda.synchronize()
    e_o = head_relf(to_host64(o1), to_host64(o2))
    e_d = head_relf(to_host64(d1), to_host64(d2))
    same = torch.equal(o1, o2) and torch.equal(d1, d2)
    print(f"  rel_o={e_o:.2e} rel_den={e_d:.2e} bitwise={same}", flush=True)
    assert np.all(np.isfinite(to_host64(o1)))
    assert e_o <= TOL[dtype] and e_d <= TOL[dtype]


@pytest.mark.parametrize("calls", CALLS, ids=["bf16", "f32", "f16_then_bf16_L64"])
def test_noalloc_matches_forward_twice(calls):
    for c in calls:
        _one(*c)


def test_noalloc_rejects_oversize():
    B, H, N, L = 1, 1, 1 << 20, 32
    need = binding.workspace_bytes(B, H, N, 64, L, 4, True, 0, torch.bfloat16, False)
    assert need > binding.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, H, N, 64), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((L, 4, 64), dtype=torch.float32, device="cuda")
    o = torch.full_like(q, 7.0)
    den = torch.full((B, H, N), 7.0, device="cuda")
    with pytest.raises(binding.RaceError) as ei:
        binding.forward_noalloc(q, q, q, W, 1.0, True, out=(o, den))
    assert ei.value.code == 6  # RACE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((den == 7.0).all())  # outputs untouched
