"""The library under HIP-graph capture: it enqueues only kernels on the
caller's stream (no allocation, copy, memset or synchronisation), so a
training step -- forward with the saved state, then backward -- can be
captured once and replayed.  Every replay, with eager work and
synchronisations between replays, must write the eager step's bits exactly:
o, den, dQ, dK, dV (bf16, fp16 and fp32 rows; 16-bit rows with L > 32 run in
table passes; the hard forward on bucket ids)."""
import pytest
import torch

from sketch_attention_soft_amd import binding
from sketch_attention_soft_amd import inputs as I
from tests.gpu_util import device_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, B, H, N, L, tau, causal
    ("bf16", 1, 2, 3000, 32, 1.0, True),
    ("f16", 2, 1, 1000, 16, 0.5, False),
    ("bf16", 1, 1, 2000, 64, 1.0, True),
    ("f32", 1, 2, 1500, 8, 1.0, True),
]
TDT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s_B%dH%dN%dL%d_tau%g_c%d" % c)
def test_training_step_replays_bitwise(case):
    dtype, B, H, N, L, tau, causal = case
    x = I.make_inputs(B, H, N, 64, L, 4, dtype, 2600 + N + L, with_grad=True)
    dx = device_inputs(x, dtype)
    q, k, v, do, W = dx["q"], dx["k"], dx["v"], dx["do"], dx["W"]
    print(f"[case] graph {dtype} B={B} H={H} N={N} L={L} causal={causal}", flush=True)
    tdt = TDT[dtype]
    wsf = torch.empty(binding.workspace_bytes(B, H, N, 64, L, 4, causal, 0, tdt, 0), dtype=torch.uint8,
                      device="cuda")
    wsb = torch.empty(binding.workspace_bytes(B, H, N, 64, L, 4, causal, 0, tdt, 1), dtype=torch.uint8,
                      device="cuda")
    saved = binding.new_saved(q, W, causal) if dtype != "f32" else None
    o, den = torch.empty_like(q), torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    grads = tuple(torch.empty_like(q) for _ in range(3))
    outs = (o, den) + grads

    def step():
        binding.forward(q, k, v, W, tau, causal, workspace=wsf, out=(o, den), saved=saved)
        binding.backward(q, k, v, W, o, den, do, tau, causal, workspace=wsb, out=grads, saved=saved)

    step()
    torch.cuda.synchronize()
    ref = tuple(t.clone() for t in outs)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in outs:
            t.fill_(float("nan") if t.is_floating_point() else 0)
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(outs, ref)), rep
        # eager work between replays, on the same buffers
        step()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(outs, ref)), rep


def test_hard_forward_replays_bitwise():
    B, H, N, L = 1, 2, 2000, 16
    x = I.make_inputs(B, H, N, 64, L, 4, "bf16", 2690, with_grad=False)
    dx = device_inputs(x, "bf16")
    print("[case] graph hard", flush=True)
    ws = torch.empty(binding.workspace_bytes(B, H, N, 64, L, 4, True, 0, torch.bfloat16, 4),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty_like(dx["q"])
    den = torch.empty((B, H, N), dtype=torch.float32, device="cuda")

    def step():
        binding.forward_hard(dx["q"], dx["k"], dx["v"], dx["W"], True, 0, workspace=ws, out=(o, den))

    step()
    torch.cuda.synchronize()
    ref = (o.clone(), den.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    for rep in range(3):
        o.fill_(float("nan"))
        den.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref[0]) and torch.equal(den, ref[1]), rep
        step()
        torch.cuda.synchronize()
