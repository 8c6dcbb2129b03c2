"""The seeded input generator: determinism, prefixes, rounding, normalisation."""
import numpy as np
import torch

from sketch_attention_soft_amd import inputs as I


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 3.4e38], np.float32)])
    ours = I.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(I.bf16_bits_to_f32(ours),
                          torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_deterministic_and_prefix_consistent():
    a = I.make_inputs(1, 2, 70000, 64, 8, 4, "bf16", seed=5)
    b = I.make_inputs(1, 2, 70000, 64, 8, 4, "bf16", seed=5)
    for k in a:
        assert np.array_equal(a[k], b[k])
    p = I.make_inputs(1, 2, 70000, 64, 8, 4, "bf16", seed=5, n_rows=1000)
    for k in ("q", "k", "v", "do"):
        assert np.array_equal(p[k], a[k][:, :, :1000])
    c = I.make_inputs(1, 2, 70000, 64, 8, 4, "bf16", seed=6)
    assert not np.array_equal(c["q"], a["q"])


def test_q_k_rows_normalised_v_not():
    x = I.make_inputs(2, 1, 3000, 64, 8, 4, "f32", seed=7)
    for k in ("q", "k"):
        n = np.linalg.norm(x[k].astype(np.float64), axis=-1)
        np.testing.assert_allclose(n, 1.0, atol=1e-6)
    n = np.linalg.norm(x["v"].astype(np.float64), axis=-1)
    assert n.std() > 0.1
    assert x["W"].shape == (8, 4, 64) and x["W"].dtype == np.float32


def test_workloads_table():
    w = I.WORKLOADS["causal_n4m_bf16"]
    assert (w.N, w.L, w.P, w.d, w.dtype, w.causal, w.tau) == (4194304, 32, 4, 64, "bf16", True,
                                                             1.0)
    assert I.WORKLOADS["causal_h8_n64k_f32"].chunk == 256
    assert I.WORKLOADS["noncausal_fwd_n1k_f32"].backward is False
    assert len({w.seed for w in I.WORKLOADS.values()}) == len(I.WORKLOADS)


def test_f16_storage_matches_torch():
    # fp16 workloads store IEEE half bits rounded to nearest even, as torch does
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 100,
                        np.array([0.0, -0.0, 1.0, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 6e-8], np.float32)])
    ours = I._store(x, "f16")
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert ours.dtype == np.uint16 and np.array_equal(ours, ref)
    assert np.array_equal(I.to_f64(ours, "f16"), torch.from_numpy(x).to(torch.float16).double().numpy())
    f = I.make_inputs(1, 1, 500, 64, 8, 4, "f16", seed=9)
    g = I.make_inputs(1, 1, 500, 64, 8, 4, "f32", seed=9)
    for k in ("q", "k", "v", "do"):
        assert f[k].dtype == np.uint16
        assert np.array_equal(I.to_f64(f[k], "f16"), g[k].astype(np.float16).astype(np.float64))


def test_row_scale_recipe():
    """Un-normalised rows: the normalised recipe's directions, norms log-uniform
    in [1e-3, 1e3] or exactly zero (about 1 row in 64); V and dO unchanged."""
    a = I.make_inputs(1, 2, 70000, 64, 4, 4, "f32", 5, row_scale=True)
    b = I.make_inputs(1, 2, 70000, 64, 4, 4, "f32", 5)
    for n in ("q", "k"):
        x, y = a[n].astype(np.float64), b[n].astype(np.float64)
        nx = np.linalg.norm(x, axis=-1)
        zero = nx == 0
        assert 0.8 / 64 < zero.mean() < 1.25 / 64
        assert nx[~zero].min() >= 0.999e-3 and nx.max() <= 1.001e3
        # roughly log-uniform: about half the rows on each side of 1
        assert 0.45 < (nx[~zero] > 1).mean() < 0.55
        cos = (x * y).sum(-1)[~zero] / (nx[~zero] * np.linalg.norm(y, axis=-1)[~zero])
        assert cos.min() > 1 - 1e-6
    for n in ("v", "do"):
        assert np.array_equal(a[n], b[n])
    # the same rows (head 0: stream rows 0..99) in every storage type
    c = I.make_inputs(1, 2, 100, 64, 4, 4, "bf16", 5, row_scale=True)
    assert np.array_equal(c["q"][:, 0], I.f32_to_bf16_bits(a["q"][:, 0, :100]))
