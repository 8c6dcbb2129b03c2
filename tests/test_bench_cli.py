"""bench.py's host-side contract, without a GPU: one GPU only (any other
--gpus exits with a message before touching a device), and the algorithmic
work per token that its rooflines divide by."""
import os
import subprocess
import sys

import bench
from sketch_attention_soft_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()


def test_algorithmic_work_of_the_headline():
    w = I.WORKLOADS["causal_n4m_bf16"]
    d, L, P = w.d, w.L, w.P
    F = L << P
    fused = ("sum_kv", "fwd_o", "sum_qd", "dq", "dk", "dv")
    # the backward recomputing the hash: 12 d L P + 8 F (d + 1) + 4 F d
    flops, nbytes, per_kernel = bench.algorithmic_per_token(w, saved=False)
    assert flops == 12 * d * L * P + 8 * F * (d + 1) + 4 * F * d == 495616
    assert sum(per_kernel[k] for k in fused) == flops
    # with the forward's saved hash features (as the step is timed): 8 d L P
    flops, nbytes, per_kernel = bench.algorithmic_per_token(w)
    assert flops == 8 * d * L * P + 8 * F * (d + 1) + 4 * F * d == 462848
    assert sum(per_kernel[k] for k in fused) == flops
    # one read of Q, K, V, O, dO, den and one write of O, dQ, dK, dV (e = 2 bytes)
    assert nbytes == 12 * d * 2 + 8 == 1544


def test_metric_names():
    assert bench.metric_name(I.WORKLOADS["causal_n4m_bf16"]) == bench.METRIC
    names = {k: bench.metric_name(w) for k, w in I.WORKLOADS.items()}
    assert len(set(names.values())) == len(names)
    assert "N=75M" in names["causal_n75m_bf16"] and "L=16" in names["causal_n75m_bf16"]
    assert "N=16K" in names["causal_b4h16_n16k_bf16"] and "B*H=64" in names["causal_b4h16_n16k_bf16"]
    assert "latency" in names["noncausal_fwd_n1k_f32"] and "fwd" in names["noncausal_fwd_n1k_f32"]
    assert "4M" not in names["causal_h8_n64k_f32"]
