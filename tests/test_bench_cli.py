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
    flops, nbytes, per_kernel = bench.algorithmic_per_token(w)
    d, L, P = w.d, w.L, w.P
    F = L << P
    # 12 d L P + 8 F (d + 1) + 4 F d and 12 d e + 8 (e = 2 bytes)
    assert flops == 12 * d * L * P + 8 * F * (d + 1) + 4 * F * d == 495616
    assert nbytes == 12 * d * 2 + 8 == 1544
    # the fused kernels' shares add up to the whole step
    fused = ("sum_kv", "fwd_o", "sum_qd", "dq", "dk", "dv")
    assert sum(per_kernel[k] for k in fused) == flops
