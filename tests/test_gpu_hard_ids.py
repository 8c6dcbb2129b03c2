"""Hard-hash bucket ids (race_attn_hash_ids) against the oracle's hard
assignment (gist.science/zh/paper/2510.04008, technical summary §2.2 and §3:
the tau -> 0 limit of the soft hash, one corner per table).

The kernel decides each sign on exact products (W and the row split into bf16
terms that add up to their values) with fp32 additions, so an id may differ
from the oracle's only where some |u_lp| = |sum_t W_t x_t| is within
n 2^-24 sum_t |W_t x_t| of zero (n = 3 t ceil32(d) + 16, t = 1, 2, 3 row terms
for bf16, fp16, fp32); every other id must be equal, and the number of
exceptions is reported.  Rows include zero rows (all signs +: the last
corner) and rows scaled over [1e-3, 1e3].
"""
import numpy as np
import pytest
import torch

import oracle
from sketch_attention_soft_amd import binding
from sketch_attention_soft_amd import inputs as I
from tests.gpu_util import device_inputs, host_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, d, L, P, rows
    ("bf16", 64, 32, 4, 5000),
    ("f16", 64, 8, 4, 3000),
    ("f32", 64, 16, 4, 3000),
    ("bf16", 32, 100, 3, 2000),
    ("bf16", 128, 16, 6, 2500),
    ("f32", 128, 5, 1, 1000),
    ("f16", 8, 128, 5, 777),
]
TERMS = {"bf16": 1, "f16": 2, "f32": 3}


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s_d%d_L%d_P%d_n%d" % c)
def test_ids_against_the_oracle(case):
    dtype, d, L, P, rows = case
    x = I.make_inputs(1, 1, rows, d, L, P, dtype, 6100 + rows + L, with_grad=False, row_scale=True)
    dx, hx = device_inputs(x, dtype), host_inputs(x, dtype)
    print(f"[case] ids {dtype} d={d} L={L} P={P} rows={rows}", flush=True)
    ids = binding.hash_ids(dx["q"][0, 0], dx["W"])
    torch.cuda.synchronize()
    got = ids.cpu().numpy().astype(np.int64)
    q, W = hx["q"][0, 0], hx["W"]
    phi, _ = oracle.soft_hash(q, W, 1.0, hard=True)          # [rows, L, R] one-hot
    want = phi.argmax(axis=-1)
    assert np.all(phi.max(axis=-1) == 1.0)
    # the rounding bound of each hyperplane's fp32 sum
    u = np.einsum("lpd,nd->nlp", W, q)
    mag = np.einsum("lpd,nd->nlp", np.abs(W), np.abs(q))
    n = 3 * TERMS[dtype] * (-(-d // 32) * 32) + 16
    near = (np.abs(u) <= n * 2.0 ** -24 * mag).any(axis=-1)  # [rows, L]
    diff = got != want
    print(f"  ids differing: {int(diff.sum())} of {diff.size}; within the bound of zero: "
          f"{int(near.sum())}")
    assert not np.any(diff & ~near)
    zero = np.abs(q).sum(-1) == 0
    assert zero.any() and np.all(got[zero] == (1 << P) - 1)


def test_ids_empty_and_errors():
    W = torch.zeros((4, 4, 64), dtype=torch.float32, device="cuda")
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    assert binding.hash_ids(x, W).shape == (0, 4)
    with pytest.raises(binding.RaceError):
        binding.hash_ids(torch.zeros((3, 60), dtype=torch.bfloat16, device="cuda"),
                         torch.zeros((4, 4, 60), dtype=torch.float32, device="cuda"))
