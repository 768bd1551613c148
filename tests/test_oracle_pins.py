"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each test checks the oracle against something its own code does not contain: an
independent least-squares solve, a textbook limit, a closed form, an algebraic identity
from the pages written in a different form, or an invariance of the definition.  A
plausible slip in the oracle (a dropped ridge rescale, a wrong sign, a transposed moment,
an off-by-one prefix, normalised instead of raw weights) fails at least one of them:

* dropped e^{-m} on the ridge, raw-vs-normalised weights -> brute force (unshifted weights)
* sign of the correction, transposed C_vk                  -> brute force, affine exactness
* prefix j < i instead of j <= i                           -> first row, brute force, causality
* wrong centring                                           -> affine exactness, value shift
"""
import math

import numpy as np
import pytest

import lla_inputs
from oracle import lla_forward, lla_row, lla_row_parts, lla_rows


# ---------------------------------------------------------------- independent solvers
def ridge_lstsq_row(q_i, K, V, h, lam, weights=None):
    """Weighted ridge fit with intercept, solved as an augmented least-squares problem.

    Minimises sum_j w_j ||v_j - b - W (k_j - q_i)||^2 + lam ||W||_F^2 with raw (unshifted)
    weights w_j = exp(q_i.k_j/h) by SVD least squares on the stacked system
    [sqrt(w) * (1, z_j^T)] theta = sqrt(w) v_j  and  [0, sqrt(lam) e_a^T] theta = 0.
    """
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    q_i = np.asarray(q_i, np.float64)
    n, d = K.shape
    if weights is None:
        weights = np.exp(K @ q_i / h)
    sw = np.sqrt(weights)
    Z = K - q_i
    X = np.hstack([np.ones((n, 1)), Z]) * sw[:, None]
    Y = V * sw[:, None]
    if lam > 0:
        X = np.vstack([X, np.hstack([np.zeros((d, 1)), math.sqrt(lam) * np.eye(d)])])
        Y = np.vstack([Y, np.zeros((d, V.shape[1]))])
    theta, *_ = np.linalg.lstsq(X, Y, rcond=None)
    return theta[0]


def normal_equations_row(q_i, K, V, h, lam):
    """The explicit (d+1)-unknown weighted normal equations with raw weights.

    [X^T W X + diag(0, lam I)] theta = X^T W v with rows x_j = (1, z_j), per output channel.
    """
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    n, d = K.shape
    w = np.exp(K @ q_i / h)
    X = np.hstack([np.ones((n, 1)), K - q_i])
    G = X.T @ (w[:, None] * X)
    G[1:, 1:] += lam * np.eye(d)
    rhs = X.T @ (w[:, None] * V)
    return np.linalg.solve(G, rhs)[0]


def softmax_attention(q, K, V, h):
    s = K @ q / h
    p = np.exp(s - s.max())
    return (p / p.sum()) @ V


def relerr(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def rand_case(seed, n, d, dv=None, qscale=1.0):
    rng = np.random.default_rng(seed)
    dv = dv or d
    q = rng.standard_normal((n, d)) * qscale
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, dv))
    return q, k, v


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("seed,n,d,dv,h,lam", [
    (0, 8, 2, 2, 1.0, 1e-2),
    (1, 16, 4, 4, 2.0, 1e-1),
    (2, 32, 8, 8, 2.8, 1e-2),
    (3, 32, 8, 3, 1.5, 1.0),
    (4, 24, 5, 7, 0.7, 1e-3),
])
def test_matches_bruteforce_weighted_ridge(seed, n, d, dv, h, lam):
    # qscale makes the per-row maxima large, so a missing e^{-m} on the ridge would show.
    q, k, v = rand_case(seed, n, d, dv, qscale=2.0)
    for i in range(n):
        ref = ridge_lstsq_row(q[i], k[: i + 1], v[: i + 1], h, lam)
        ne = normal_equations_row(q[i], k[: i + 1], v[: i + 1], h, lam)
        got = lla_row(q[i], k[: i + 1], v[: i + 1], h, lam)
        assert relerr(got, ref) < 1e-9, (i, relerr(got, ref))
        # the uncentred normal equations square the condition number: looser bound
        assert relerr(got, ne) < 1e-5, (i, relerr(got, ne))


def test_matches_bruteforce_on_tiny_workload():
    w = lla_inputs.WORKLOADS["tiny"]
    q, k, v, _ = lla_inputs.generate(w)
    out = lla_forward(q, k, v, w.h, w.lam)[0, 0]
    for i in range(w.n):
        ref = ridge_lstsq_row(q[0, 0, i], k[0, 0, : i + 1], v[0, 0, : i + 1], w.h, w.lam)
        assert relerr(out[i], ref) < 1e-9, i


# ---------------------------------------------------------------- special cases, closed forms
def test_first_row_is_its_own_value():
    q, k, v = rand_case(7, 4, 6)
    for lam in (1e-6, 1e-2, 10.0):
        assert np.allclose(lla_row(q[0], k[:1], v[:1], 2.0, lam), v[0], rtol=0, atol=1e-12)


def test_two_points_in_one_dimension_closed_form():
    # d = 1, prefix {(k0, v0), (k1, v1)}: with lam = 0 the local linear fit is the line
    # through both points, evaluated at the query (extrapolating outside [k0, k1]).
    k = np.array([[0.3], [1.1]])
    v = np.array([[2.0], [-1.0]])
    for qv in (-0.5, 0.3, 0.7, 2.5):
        q = np.array([qv])
        expect = v[0, 0] + (v[1, 0] - v[0, 0]) * (qv - k[0, 0]) / (k[1, 0] - k[0, 0])
        got = lla_row(q, k, v, 1.3, 0.0)
        assert abs(got[0] - expect) < 1e-12
        # lam > 0: W = C_vk / (C_kk + lam) with C = w0 w1/(w0+w1) * products of differences
        lam = 0.37
        w0, w1 = np.exp(q[0] * k[:, 0] / 1.3)
        c = w0 * w1 / (w0 + w1)
        slope = c * (v[1, 0] - v[0, 0]) * (k[1, 0] - k[0, 0]) / (c * (k[1, 0] - k[0, 0]) ** 2 + lam)
        vbar = (w0 * v[0, 0] + w1 * v[1, 0]) / (w0 + w1)
        kbar = (w0 * k[0, 0] + w1 * k[1, 0]) / (w0 + w1)
        expect = vbar - slope * (kbar - qv)
        assert abs(lla_row(q, k, v, 1.3, lam)[0] - expect) < 1e-12


# ---------------------------------------------------------------- limits named on the pages
def test_strong_regularisation_limit_is_softmax_attention():
    # lambda -> infinity suppresses the probe; LLA reduces to softmax attention
    # (Nadaraya-Watson).  The gap must shrink like 1/lambda.
    q, k, v = rand_case(11, 40, 6)
    gaps = []
    for lam in (1e6, 1e8, 1e10):
        g = max(relerr(lla_row(q[i], k[: i + 1], v[: i + 1], 2.0, lam),
                       softmax_attention(q[i], k[: i + 1], v[: i + 1], 2.0))
                for i in range(5, 40))
        gaps.append(g)
    assert gaps[2] < 1e-7
    assert 50 < gaps[0] / gaps[1] < 200 and 50 < gaps[1] / gaps[2] < 200


def test_wide_bandwidth_limit_is_global_ridge_with_intercept():
    # h -> infinity makes every weight 1: the fit becomes ordinary ridge regression with an
    # intercept over the whole prefix, evaluated at the query.
    q, k, v = rand_case(12, 30, 5)
    for i in range(30):
        ref = ridge_lstsq_row(q[i], k[: i + 1], v[: i + 1], 1.0, 0.05,
                              weights=np.ones(i + 1))
        got = lla_row(q[i], k[: i + 1], v[: i + 1], 1e13, 0.05)
        assert relerr(got, ref) < 1e-8, i


def test_lambda_zero_affine_values_are_recovered_exactly():
    # With lambda = 0 and v = A k + c exactly, the local linear fit is exact: b_i = A q_i + c
    # (no boundary bias) on every row whose prefix spans the key space (i >= d).  Checked on
    # the pre-cast fp64 inputs of the tiny affine workload.
    w = lla_inputs.WORKLOADS["tiny_affine"]
    q, k, v, ex = lla_inputs.make_inputs(w.B, w.H, w.n, w.d, w.seed, w.recipe, extras=True)
    A, c = ex["A"][0, 0], ex["c"][0, 0]
    rows = [(0, 0, i) for i in range(w.d, w.n)]
    out = lla_rows(q, k, v, w.h, 0.0, rows)
    for r, (_, _, i) in enumerate(rows):
        expect = A @ q[0, 0, i] + c
        assert relerr(out[r], expect) < 1e-8, i
    # softmax attention on the same data is visibly biased on these rows
    sa = softmax_attention(q[0, 0, -1], k[0, 0], v[0, 0], w.h)
    assert relerr(sa, A @ q[0, 0, -1] + c) > 1e-2


def test_lambda_zero_is_the_small_lambda_limit():
    q, k, v = rand_case(13, 24, 4)
    for i in (2, 3, 10, 23):  # rank-deficient (i < d) and full-rank rows
        # The gap closes like lambda; below ~1e-9 the rank-deficient rows' own rounding
        # (amplified by 1/lambda) dominates, so the limit is checked at 1e-6 and 1e-8.
        a = lla_row(q[i], k[: i + 1], v[: i + 1], 1.5, 0.0)
        g6 = relerr(a, lla_row(q[i], k[: i + 1], v[: i + 1], 1.5, 1e-6))
        g8 = relerr(a, lla_row(q[i], k[: i + 1], v[: i + 1], 1.5, 1e-8))
        assert g6 < 1e-5 and g8 < 1e-7, (i, g6, g8)


# ---------------------------------------------------------------- identities of the pages
def test_scoring_form_and_additive_form_agree():
    # Scoring form: solve Sigma_i rho = mu_i, t_ij = rho.z_ij,
    #   b = sum_j w (1 - t_ij) v_j / sum_j w (1 - t_ij).
    # Additive form: b = o_SA - (1 + eta) Sigma_KV rho, eta = tbar / (1 - tbar) >= 0.
    # Appendix E: eta = omega * zbar^T (C_kk + lambda I)^{-1} zbar (a Mahalanobis distance).
    q, k, v = rand_case(21, 20, 4, qscale=1.5)
    h, lam = 1.7, 0.05
    for i in range(20):
        K, V = k[: i + 1], v[: i + 1]
        w = np.exp(K @ q[i] / h)
        Z = K - q[i]
        mu = w @ Z
        Sigma = (Z * w[:, None]).T @ Z + lam * np.eye(4)
        rho = np.linalg.solve(Sigma, mu)
        t = Z @ rho
        b_scoring = (w * (1 - t)) @ V / np.sum(w * (1 - t))
        p = w / w.sum()
        vbar, kbar = p @ V, p @ K
        sigma_kv = ((V - vbar) * p[:, None]).T @ (K - kbar)
        tbar = p @ t
        eta = tbar / (1 - tbar)
        b_additive = vbar - (1 + eta) * sigma_kv @ rho
        got = lla_row_parts(q[i], K, V, h, lam)
        assert relerr(got["b"], b_scoring) < 1e-9
        assert relerr(got["b"], b_additive) < 1e-9
        zbar = kbar - q[i]
        Ckk = ((K - kbar) * w[:, None]).T @ (K - kbar)
        eta_mahal = w.sum() * zbar @ np.linalg.solve(Ckk + lam * np.eye(4), zbar)
        assert eta >= 0 and abs(eta - eta_mahal) <= 1e-8 * max(1.0, eta)


# ---------------------------------------------------------------- invariances of the definition
def test_linear_in_values_and_equivariant_to_value_shift():
    q, k, v = rand_case(31, 16, 4)
    v2 = np.random.default_rng(32).standard_normal(v.shape)
    c = np.array([3.0, -2.0, 0.5, 7.0])
    for i in (0, 3, 9, 15):
        K = k[: i + 1]
        f = lambda V: lla_row(q[i], K, V, 1.3, 0.02)  # noqa: E731
        assert relerr(f(2.0 * v[: i + 1] - 0.5 * v2[: i + 1]),
                      2.0 * f(v[: i + 1]) - 0.5 * f(v2[: i + 1])) < 1e-10
        assert relerr(f(v[: i + 1] + c), f(v[: i + 1]) + c) < 1e-10


def test_invariant_to_joint_rotation_of_queries_and_keys():
    q, k, v = rand_case(41, 16, 5)
    Rm, _ = np.linalg.qr(np.random.default_rng(42).standard_normal((5, 5)))
    for i in (1, 4, 8, 15):
        a = lla_row(q[i], k[: i + 1], v[: i + 1], 1.1, 0.03)
        b = lla_row(Rm @ q[i], k[: i + 1] @ Rm.T, v[: i + 1], 1.1, 0.03)
        assert relerr(a, b) < 1e-10


def test_causal_prefix_only():
    w = lla_inputs.WORKLOADS["tiny"].with_shape(n=24, d=4)
    q, k, v, _ = lla_inputs.generate(w)
    base = lla_forward(q, k, v, w.h, w.lam)
    k2, v2 = k.copy(), v.copy()
    k2[..., 12:, :] += 1.0
    v2[..., 12:, :] -= 2.0
    pert = lla_forward(q, k2, v2, w.h, w.lam)
    assert np.array_equal(base[..., :12, :], pert[..., :12, :])
    assert not np.allclose(base[..., 12:, :], pert[..., 12:, :])


def test_row_subset_and_pool_match_full_forward():
    w = lla_inputs.WORKLOADS["tiny"].with_shape(B=2, H=2, n=40, d=4)
    q, k, v, _ = lla_inputs.generate(w)
    full = lla_forward(q, k, v, w.h, w.lam)
    rows = [(b, hh, i) for b in range(2) for hh in range(2) for i in range(0, 40, 3)]
    sub = lla_rows(q, k, v, w.h, w.lam, rows, workers=2)
    for r, (b, hh, i) in enumerate(rows):
        assert np.array_equal(sub[r], full[b, hh, i])


def test_tiny_golden_fixture_unchanged():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle.txt")
    stored = np.loadtxt(path)
    w = lla_inputs.WORKLOADS["tiny"]
    q, k, v, _ = lla_inputs.generate(w)
    assert relerr(lla_forward(q, k, v, w.h, w.lam)[0, 0], stored) < 1e-13


def test_decode_is_the_last_row_and_ignores_cache_order():
    from oracle import lla_decode
    rng = np.random.default_rng(101)
    B, H, L, d = 2, 2, 30, 4
    qs, k, v = (rng.standard_normal((B, H, L, d)) for _ in range(3))
    full = lla_forward(qs, k, v, 1.4, 0.05)
    dec = lla_decode(qs[:, :, -1], k, v, 1.4, 0.05)
    assert np.array_equal(dec, full[:, :, -1])
    perm = rng.permutation(L)
    assert relerr(lla_decode(qs[:, :, -1], k[:, :, perm], v[:, :, perm], 1.4, 0.05), dec) < 1e-10
