"""Pins of the fp64 oracle against facts the pages and mathematics fix.

Pages (title "RACE Attention: A Strictly Linear-Time Attention for
Long-Sequence Training", gist.science/<lang>/paper/2510.04008, technical
summaries): [zh] §2.1 kernel, §2.2 soft hashing / sketch / ratio readout,
§2.3 causal streaming, §3 error bound; [es] §2 items 1-3 (normalised angular
kernel, soft assignment, tanh and temperature); [pt] §2 (tanh then softmax
over hypercube corners).

Each pin is something other than the oracle itself: a closed form, an
invariant, a textbook special case, brute force or finite differences.
"""
import math

import numpy as np
import pytest

import oracle
from tests import quadratic_ref as qr


def _unit_rows(rng, n, d):
    return qr.normalise(rng.standard_normal((n, d)))


def _relf(a, b):
    return np.linalg.norm(a - b) / np.linalg.norm(b)


# -- P-1: each table's soft assignment is a distribution over the R corners
@pytest.mark.parametrize("P,tau", [(1, 1.0), (3, 0.3), (4, 1.0), (4, 0.5), (6, 2.0)])
def test_p1_assignment_sums_to_one(P, tau):
    rng = np.random.default_rng(11)
    x = rng.standard_normal((50, 16)) * 3.0
    W = rng.standard_normal((5, P, 16))
    phi, _ = oracle.soft_hash(x, W, tau)
    assert phi.shape == (50, 5, 1 << P)
    assert np.all(phi > 0)
    np.testing.assert_allclose(phi.sum(-1), 1.0, rtol=0, atol=1e-14)


# -- P-2: corner softmax factorises into per-hyperplane logistic factors
@pytest.mark.parametrize("P,tau", [(2, 1.0), (4, 1.0), (4, 0.5), (5, 0.2)])
def test_p2_factorisation(P, tau):
    rng = np.random.default_rng(12)
    d, L = 16, 7
    x = rng.standard_normal((40, d))
    W = rng.standard_normal((L, P, d))
    phi, z = oracle.soft_hash(x, W, tau)
    # z recomputed here from the definition, not taken from the oracle
    z_ref = np.tanh(np.einsum("lpd,nd->nlp", W, qr.normalise(x)))
    np.testing.assert_allclose(z, z_ref, rtol=0, atol=1e-14)
    R = 1 << P
    c = np.array([[1.0 if (r >> p) & 1 else -1.0 for p in range(P)] for r in range(R)])
    sig = 1.0 / (1.0 + np.exp(-2.0 * c[None, None, :, :] * z_ref[:, :, None, :] / tau))
    np.testing.assert_allclose(phi, sig.prod(-1), rtol=1e-13, atol=1e-15)


# -- P-12: P = 1 is the two-way logistic split
def test_p12_single_hyperplane_is_logistic():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((30, 8))
    W = rng.standard_normal((3, 1, 8))
    for tau in (0.25, 1.0, 3.0):
        phi, _ = oracle.soft_hash(x, W, tau)
        z = np.tanh(np.einsum("ld,nd->nl", W[:, 0, :], qr.normalise(x)))
        s = 1.0 / (1.0 + np.exp(-2.0 * z / tau))
        np.testing.assert_allclose(phi[:, :, 1], s, rtol=1e-14, atol=1e-16)
        np.testing.assert_allclose(phi[:, :, 0], 1.0 - s, rtol=1e-13, atol=1e-16)


# -- P-3: exact quadratic closed form, causal and non-causal
@pytest.mark.parametrize("N,d,L,P,tau", [(200, 16, 6, 3, 0.7), (128, 64, 8, 4, 1.0),
                                         (97, 32, 5, 4, 0.5), (64, 8, 3, 1, 1.3),
                                         (90, 128, 4, 4, 1.0), (77, 24, 3, 5, 0.8),
                                         (66, 16, 2, 6, 1.0)])
@pytest.mark.parametrize("causal", [False, True])
def test_p3_quadratic_closed_form(N, d, L, P, tau, causal):
    rng = np.random.default_rng(N + d + L)
    q = rng.standard_normal((N, d)) * 2.0
    k = rng.standard_normal((N, d)) * 0.5
    v = rng.standard_normal((N, d))
    W = rng.standard_normal((L, P, d))
    o, den = oracle.forward(q, k, v, W, tau, causal)
    o_ref, den_ref = qr.soft_race_attention(q, k, v, W, tau, causal)
    np.testing.assert_allclose(den, den_ref, rtol=1e-12)
    assert _relf(o, o_ref) < 1e-12
    np.testing.assert_allclose(o, o_ref, rtol=1e-10, atol=1e-12)


def test_p3_batched_heads_are_independent():
    rng = np.random.default_rng(5)
    B, H, N, d = 2, 3, 40, 8
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    W = rng.standard_normal((4, 3, d))
    o, den = oracle.forward(q, k, v, W, 0.8, True)
    for b in range(B):
        for h in range(H):
            o_ref, den_ref = qr.soft_race_attention(q[b, h], k[b, h], v[b, h], W, 0.8, True)
            np.testing.assert_allclose(o[b, h], o_ref, rtol=1e-11, atol=1e-13)
            np.testing.assert_allclose(den[b, h], den_ref, rtol=1e-12)


def test_p3_hand_example():
    # d = 2, one table, one hyperplane along e1, tau = 1.  Key k0 = e1 has
    # z = tanh(1); key k1 = e2 has z = 0 and so phi = (1/2, 1/2).  The query
    # q = e1 hashes like k0.  kappa(q, k0) = s^2 + (1-s)^2 with
    # s = sigmoid(2 tanh 1); kappa(q, k1) = 1/2.
    W = np.array([[[1.0, 0.0]]])
    k = np.array([[1.0, 0.0], [0.0, 1.0]])
    v = np.array([[2.0, -1.0], [-4.0, 3.0]])
    q = np.array([[3.0, 0.0], [1.0, 0.0]])  # row 0 sees k0 only (causal)
    s = 1.0 / (1.0 + math.exp(-2.0 * math.tanh(1.0)))
    k0 = s * s + (1 - s) * (1 - s)
    k1 = 0.5
    o, den = oracle.forward(q, k, v, W, 1.0, True)
    np.testing.assert_allclose(o[0], v[0], rtol=1e-15)
    np.testing.assert_allclose(den[0], k0, rtol=1e-15)
    np.testing.assert_allclose(o[1], (k0 * v[0] + k1 * v[1]) / (k0 + k1), rtol=1e-14)
    np.testing.assert_allclose(den[1], k0 + k1, rtol=1e-15)


# -- P-4: hard hashing collides with probability (1 - theta/pi)^P (SimHash)
@pytest.mark.parametrize("theta", [math.pi / 6, math.pi / 3, math.pi / 2, 2 * math.pi / 3])
def test_p4_hard_hash_collision_rate(theta):
    P, L, d = 4, 200_000, 8
    rng = np.random.default_rng(int(theta * 1000))
    W = rng.standard_normal((L, P, d))
    e1 = np.zeros(d)
    e1[0] = 1.0
    e2 = np.zeros(d)
    e2[1] = 1.0
    x = np.stack([e1, math.cos(theta) * e1 + math.sin(theta) * e2]) * np.array([[2.0], [0.7]])
    phi, _ = oracle.soft_hash(x, W, 1.0, hard=True)
    assert np.all(phi.sum(-1) == 1.0)
    rate = float((phi[0] * phi[1]).sum(-1).mean())
    p = (1.0 - theta / math.pi) ** P
    sigma = math.sqrt(p * (1 - p) / L)
    assert abs(rate - p) < 5 * sigma, (rate, p, sigma)


# -- P-5: a constant value row maps to itself
@pytest.mark.parametrize("causal", [False, True])
def test_p5_constant_values(causal):
    rng = np.random.default_rng(21)
    N, d = 150, 16
    q, k = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    c = rng.standard_normal(d)
    v = np.tile(c, (N, 1))
    W = rng.standard_normal((6, 4, d))
    o, _ = oracle.forward(q, k, v, W, 0.6, causal)
    np.testing.assert_allclose(o, v, rtol=1e-13, atol=1e-15)


# -- P-6: convexity, linearity in V, permutation and scale invariance
def test_p6_invariants():
    rng = np.random.default_rng(22)
    N, d, L, P, tau = 120, 12, 5, 4, 0.9
    q, k = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    v1, v2 = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    W = rng.standard_normal((L, P, d))
    for causal in (False, True):
        o1, _ = oracle.forward(q, k, v1, W, tau, causal)
        o2, _ = oracle.forward(q, k, v2, W, tau, causal)
        o12, _ = oracle.forward(q, k, 2.0 * v1 - 0.5 * v2, W, tau, causal)
        np.testing.assert_allclose(o12, 2.0 * o1 - 0.5 * o2, rtol=1e-12, atol=1e-13)
        for i in range(N):
            vis = v1[: i + 1] if causal else v1
            assert np.all(o1[i] <= vis.max(0) + 1e-13) and np.all(o1[i] >= vis.min(0) - 1e-13)
        # positive scaling of query or key rows changes nothing (normalisation)
        sq = rng.uniform(0.1, 10.0, (N, 1))
        sk = rng.uniform(0.1, 10.0, (N, 1))
        o_s, _ = oracle.forward(q * sq, k * sk, v1, W, tau, causal)
        np.testing.assert_allclose(o_s, o1, rtol=1e-12, atol=1e-13)
    # non-causal: joint permutation of keys and values, and permutation of queries
    o1, _ = oracle.forward(q, k, v1, W, tau, False)
    pk, pq = rng.permutation(N), rng.permutation(N)
    o_p, _ = oracle.forward(q[pq], k[pk], v1[pk], W, tau, False)
    np.testing.assert_allclose(o_p, o1[pq], rtol=1e-12, atol=1e-13)


# -- P-7: hard-hash RACE converges to angular attention with gamma = P as 1/sqrt(L)
@pytest.mark.slow
def test_p7_convergence_to_angular_attention():
    N, d, P = 256, 64, 4
    Ls = [16, 64, 256, 1024, 4096]
    errs = np.zeros(len(Ls))
    seeds = range(4)
    for s in seeds:
        rng = np.random.default_rng(700 + s)
        q = rng.standard_normal((N, d))
        k = q + 0.8 * rng.standard_normal((N, d))  # related keys: a peaked kernel
        v = rng.standard_normal((N, d))
        o_ang, _ = qr.angular_attention(q, k, v, P)
        for a, L in enumerate(Ls):
            W = rng.standard_normal((L, P, d))
            o, den = oracle.forward(q, k, v, W, 1.0, False, hard=True)
            assert np.all(den > 0)
            errs[a] += _relf(o, o_ang) / len(seeds)
    assert np.all(np.diff(errs) < 0), errs
    slope = np.polyfit(np.log(Ls), np.log(errs), 1)[0]
    assert -0.6 <= slope <= -0.4, (slope, errs)


# -- soft -> hard: as tau -> 0 the soft oracle becomes the hard-hash oracle,
#    and its error to angular attention shrinks with the bias term P/beta
def test_soft_to_hard_limit_and_bias():
    rng = np.random.default_rng(31)
    N, d, L, P = 96, 16, 256, 4
    q = rng.standard_normal((N, d))
    k = q + 0.7 * rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    W = rng.standard_normal((L, P, d))
    o_h, _ = oracle.forward(q, k, v, W, 1.0, True, hard=True)
    # only hyperplanes with |z| of order tau can differ from the hard choice,
    # so the gap closes as tau shrinks
    gaps = [_relf(oracle.forward(q, k, v, W, t, True)[0], o_h) for t in (1e-2, 1e-5, 1e-10)]
    assert gaps[0] > gaps[1] and gaps[2] < 1e-6, gaps
    o_ang, _ = qr.angular_attention(q, k, v, P, causal=True)
    e = [_relf(oracle.forward(q, k, v, W, t, True)[0], o_ang) for t in (2.0, 0.5, 0.125)]
    assert e[0] > e[1] > e[2], e


# -- P-8: causality
def test_p8_causal_perturbation_and_prefix():
    rng = np.random.default_rng(41)
    N, d, L, P, tau = 90, 10, 4, 3, 0.8
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    W = rng.standard_normal((L, P, d))
    o, den = oracle.forward(q, k, v, W, tau, True)
    j = 37
    k2, v2 = k.copy(), v.copy()
    k2[j] += rng.standard_normal(d)
    v2[j] += rng.standard_normal(d)
    o2, den2 = oracle.forward(q, k2, v2, W, tau, True)
    assert np.array_equal(o2[:j], o[:j]) and np.array_equal(den2[:j], den[:j])
    assert np.all(np.abs(o2[j:] - o[j:]).max(1) > 0)
    for i in (0, 1, 17, N - 1):
        o_nc, den_nc = oracle.forward(q[: i + 1], k[: i + 1], v[: i + 1], W, tau, False)
        np.testing.assert_allclose(o[i], o_nc[i], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(den[i], den_nc[i], rtol=1e-12)
    # the first row sees only its own key
    np.testing.assert_allclose(o[0], v[0], rtol=1e-14)


def _loss_grads_fd(fwd, q, k, v, g, h=1e-6):
    """Central finite differences of sum(g * fwd(q, k, v)) w.r.t. q, k, v."""
    out = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        x = args[which]
        gr = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = float((g * fwd(*args)).sum())
            x[idx] = old - h
            lm = float((g * fwd(*args)).sum())
            x[idx] = old
            gr[idx] = (lp - lm) / (2 * h)
        out.append(gr)
    return out


# -- P-9: backward against finite differences of the oracle's forward
@pytest.mark.parametrize("P,tau,causal", [(2, 1.0, True), (3, 0.5, False), (4, 1.0, True),
                                          (4, 0.5, False), (3, 0.7, True), (5, 0.8, True),
                                          (6, 1.0, False), (6, 0.5, True)])
def test_p9_finite_differences(P, tau, causal):
    rng = np.random.default_rng(50 + P)
    N, d, L = 12, 6, 3
    q = rng.standard_normal((N, d)) * 1.7  # un-normalised rows
    k = rng.standard_normal((N, d)) * 0.6
    v = rng.standard_normal((N, d))
    g = rng.standard_normal((N, d))
    W = rng.standard_normal((L, P, d))
    o, den, dq, dk, dv = oracle.forward_backward(q, k, v, g, W, tau, causal)
    fd = _loss_grads_fd(lambda a, b, c: oracle.forward(a, b, c, W, tau, causal)[0], q, k, v, g)
    for an, num in zip((dq, dk, dv), fd):
        assert _relf(an, num) < 1e-6, _relf(an, num)


# -- P-9 at head dimension 128 (un-normalised rows, causal and not)
@pytest.mark.parametrize("causal", [True, False])
def test_p9_finite_differences_d128(causal):
    rng = np.random.default_rng(57)
    N, d, L, P, tau = 6, 128, 2, 4, 0.8
    q = rng.standard_normal((N, d)) * 1.3
    k = rng.standard_normal((N, d)) * 0.4
    v = rng.standard_normal((N, d))
    g = rng.standard_normal((N, d))
    W = rng.standard_normal((L, P, d))
    o, den, dq, dk, dv = oracle.forward_backward(q, k, v, g, W, tau, causal)
    fd = _loss_grads_fd(lambda a, b, c: oracle.forward(a, b, c, W, tau, causal)[0], q, k, v, g)
    for an, num in zip((dq, dk, dv), fd):
        assert _relf(an, num) < 1e-6, _relf(an, num)


# -- P-11: backward against finite differences of the brute-force closed form
@pytest.mark.parametrize("causal", [False, True])
def test_p11_backward_vs_closed_form_fd(causal):
    rng = np.random.default_rng(60)
    N, d, L, P, tau = 10, 5, 2, 3, 0.6
    q, k, v, g = (rng.standard_normal((N, d)) for _ in range(4))
    W = rng.standard_normal((L, P, d))
    _, _, dq, dk, dv = oracle.forward_backward(q, k, v, g, W, tau, causal)
    fd = _loss_grads_fd(lambda a, b, c: qr.soft_race_attention(a, b, c, W, tau, causal)[0],
                        q, k, v, g)
    for an, num in zip((dq, dk, dv), fd):
        assert _relf(an, num) < 1e-6, _relf(an, num)


# -- P-10: exact identities of the backward
@pytest.mark.parametrize("causal", [False, True])
def test_p10_gradient_identities(causal):
    rng = np.random.default_rng(70)
    B, H, N, d, L, P, tau = 1, 2, 300, 16, 4, 4, 0.5
    q, k, v, g = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    W = rng.standard_normal((L, P, d))
    o, den, dq, dk, dv = oracle.forward_backward(q, k, v, g, W, tau, causal)
    # degree-0 homogeneity in every q and k row
    sc = np.abs((dq * q).sum(-1)) / (np.linalg.norm(dq, axis=-1) * np.linalg.norm(q, axis=-1))
    assert sc.max() < 1e-12
    sc = np.abs((dk * k).sum(-1)) / (np.linalg.norm(dk, axis=-1) * np.linalg.norm(k, axis=-1))
    assert sc.max() < 1e-12
    for h in range(H):
        # linearity in V and shift equivariance
        lhs = (dv[0, h] * v[0, h]).sum()
        rhs = (g[0, h] * o[0, h]).sum()
        assert abs(lhs - rhs) < 1e-12 * max(1.0, abs(rhs))
        np.testing.assert_allclose(dv[0, h].sum(0), g[0, h].sum(0), rtol=1e-12, atol=1e-11)


def test_edge_zero_rows_and_single_token():
    rng = np.random.default_rng(80)
    d = 8
    W = rng.standard_normal((3, 4, d))
    # a zero query row hashes to the uniform assignment 1/R
    phi, _ = oracle.soft_hash(np.zeros((1, d)), W, 1.0)
    np.testing.assert_allclose(phi, 1.0 / 16, rtol=1e-15)
    # N = 1: the output is the single value row, forward and backward finite
    q, k, v, g = (rng.standard_normal((1, d)) for _ in range(4))
    o, den, dq, dk, dv = oracle.forward_backward(q, k, v, g, W, 1.0, True)
    np.testing.assert_allclose(o, v, rtol=1e-15)
    np.testing.assert_allclose(dv, g, rtol=1e-14)
    assert np.all(np.isfinite(dq)) and np.all(np.isfinite(dk))


def test_invalid_arguments_raise():
    W = np.ones((2, 4, 8))
    x = np.ones((3, 8))
    with pytest.raises(ValueError):
        oracle.forward(x, x, x, W, 0.0, True)
    with pytest.raises(ValueError):
        oracle.forward(x, x, x, W, float("nan"), True)


# -- P-13: the streaming state in the Walsh basis (zh §2.2 bucket sums, §2.3
# running sums) -- pins of oracle.bucket_sums and oracle.walsh_state
@pytest.mark.parametrize("P", [2, 3, 4])
def test_p13_walsh_state_closed_forms(P):
    rng = np.random.default_rng(61 + P)
    N, d, L, tau = 57, 12, 3, 0.7
    R, sc = 1 << P, 2.0 ** (-P / 2)
    k, v = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    W = rng.standard_normal((L, P, d))
    S = oracle.walsh_state(k, v, W, tau)
    assert S.shape == (L * R, d + 1)
    # the empty subset has psi = 2^(-P/2) for every key: count column N 2^(-P/2)
    for l in range(L):
        np.testing.assert_allclose(S[R * l, d], N * sc, rtol=1e-13)
        np.testing.assert_allclose(S[R * l, :d], v.sum(0) * sc, rtol=1e-12, atol=1e-13)
    # brute force: psi_s = 2^(-P/2) prod_{p in s} tanh(z_p / tau), from the oracle's z
    _, z = oracle.soft_hash(k, W, tau)
    t = np.tanh(z / tau)
    psi = np.empty((N, L, R))
    for s_ in range(R):
        psi[:, :, s_] = sc * np.prod([t[:, :, p] if (s_ >> p) & 1 else np.ones((N, L))
                                      for p in range(P)], axis=0)
    brute = np.einsum("jf,jc->fc", psi.reshape(N, L * R),
                      np.concatenate([v, np.ones((N, 1))], axis=1))
    np.testing.assert_allclose(S, brute, rtol=1e-10, atol=1e-12)
    # additive over a split of the keys
    S2 = oracle.walsh_state(k[:20], v[:20], W, tau) + oracle.walsh_state(k[20:], v[20:], W, tau)
    np.testing.assert_allclose(S2, S, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("P", [1, 2, 3, 4])
def test_p13_walsh_readout_is_the_non_causal_forward(P):
    rng = np.random.default_rng(62 + P)
    N, M, d, L, tau = 40, 9, 16, 5, 1.3
    R, sc = 1 << P, 2.0 ** (-P / 2)
    k, v, q = (rng.standard_normal((n, d)) for n in (N, N, M))
    W = rng.standard_normal((L, P, d))
    S = oracle.walsh_state(k, v, W, tau)
    _, zq = oracle.soft_hash(q, W, tau)
    tq = np.tanh(zq / tau)
    psi = np.empty((M, L, R))
    for s_ in range(R):
        psi[:, :, s_] = sc * np.prod([tq[:, :, p] if (s_ >> p) & 1 else np.ones((M, L))
                                      for p in range(P)], axis=0)
    nm = psi.reshape(M, L * R) @ S
    # the same queries against all N keys, from the oracle's own readout
    qq = np.concatenate([q, np.zeros((N - M, d))]) if M < N else q
    o, den = oracle.forward(qq, k, v, W, tau, False)
    np.testing.assert_allclose(nm[:, d], den[:M], rtol=1e-11)
    np.testing.assert_allclose(nm[:, :d] / nm[:, d:], o[:M], rtol=1e-10, atol=1e-12)


# -- P-14: the projection gradient dW against finite differences of the
# oracle's forward and of the independent closed form (tests/quadratic_ref.py)
@pytest.mark.parametrize("P,tau,causal", [(4, 1.0, True), (3, 0.6, False), (2, 1.3, True)])
def test_p14_dw_finite_differences(P, tau, causal):
    rng = np.random.default_rng(80 + P)
    B, H, N, d, L = 1, 2, 9, 5, 2
    q = rng.standard_normal((B, H, N, d)) * 1.4
    k = rng.standard_normal((B, H, N, d)) * 0.7
    v, g = rng.standard_normal((B, H, N, d)), rng.standard_normal((B, H, N, d))
    W = rng.standard_normal((L, P, d))
    out = oracle.forward_backward(q, k, v, g, W, tau, causal, with_dw=True)
    dW = out[5]
    assert dW.shape == (L, P, d)
    # the other gradients are unchanged by asking for dW
    for a, b in zip(out[:5], oracle.forward_backward(q, k, v, g, W, tau, causal)):
        assert np.array_equal(a, b)
    h = 1e-6

    def loss(WW, closed=False):
        if closed:
            o = np.stack([np.stack([qr.soft_race_attention(q[0, i], k[0, i], v[0, i], WW, tau,
                                                           causal)[0] for i in range(H)])])
        else:
            o = oracle.forward(q, k, v, WW, tau, causal)[0]
        return float((g * o).sum())

    for closed in (False, True):
        num = np.zeros_like(W)
        for idx in np.ndindex(W.shape):
            Wp, Wm = W.copy(), W.copy()
            Wp[idx] += h
            Wm[idx] -= h
            num[idx] = (loss(Wp, closed) - loss(Wm, closed)) / (2 * h)
        assert _relf(dW, num) < 1e-6, (closed, _relf(dW, num))
