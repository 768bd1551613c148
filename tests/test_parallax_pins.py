"""Pins of the fp64 Parallax oracle to facts outside itself (CPU only).

Each test checks ``oracle.parallax_*`` against something its code does not contain: the
pages' streaming two-branch algorithm with its final merge, the zero-probe limit, the LLA
output recovered from the solved probe (through the pinned LLA oracle), the centred scoring
form, a library weighted covariance, a two-key closed form, and invariances.  A plausible
slip fails at least one of them:

* sign of the correction, 1/h on the probe scores     -> streaming merge, closed form
* uncentred cross moment E[v k^T] rho                   -> streaming merge, key shift
* transposed Sigma_KV                                   -> streaming merge, library cov
* normalised vs raw weights, wrong max shift            -> zero probe, streaming merge
* prefix j < i instead of j <= i                        -> first row, causality
"""
import numpy as np
import pytest

import lla_inputs
from oracle import lla_row, parallax_forward, parallax_row, parallax_row_parts, parallax_rows


def relerr(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def rand_case(seed, n, d, dv=None, qscale=1.0, rscale=1.0):
    rng = np.random.default_rng(seed)
    dv = dv or d
    q = rng.standard_normal((n, d)) * qscale
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, dv))
    rho = rng.standard_normal((n, d)) * rscale
    return q, k, v, rho


def streaming_two_branch(q_i, K, V, rho_i, h, block):
    """Section 3 of the blog ("One extra branch, no extra I/O"): one pass over KV blocks
    with a shared running max m, rescale alpha, the softmax branch (d1, O1) with
    P1 = exp(S1 - m), and the covariance branch (d2, O2) with S2 = R K_c^T unscaled and
    P2 = P1 * S2; Appendix C, item 3, merges them as (1 + d2/d1) O1/d1 - O2/d1."""
    m = -np.inf
    d1 = d2 = 0.0
    O1 = np.zeros(V.shape[1])
    O2 = np.zeros(V.shape[1])
    for j0 in range(0, K.shape[0], block):
        Kc, Vc = K[j0: j0 + block], V[j0: j0 + block]
        S1 = Kc @ q_i / h
        m_new = max(m, float(S1.max()))
        alpha = np.exp(m - m_new)
        P1 = np.exp(S1 - m_new)
        S2 = Kc @ rho_i
        P2 = P1 * S2
        d1 = alpha * d1 + P1.sum()
        d2 = alpha * d2 + P2.sum()
        O1 = alpha * O1 + P1 @ Vc
        O2 = alpha * O2 + P2 @ Vc
        m = m_new
    return (1.0 + d2 / d1) * O1 / d1 - O2 / d1


@pytest.mark.parametrize("seed,n,d,dv,h,block", [
    (0, 9, 3, 3, 1.0, 1),
    (1, 40, 8, 8, 2.0, 7),       # ragged last block
    (2, 64, 16, 16, 4.0, 16),
    (3, 50, 6, 9, 0.8, 64),      # one block
    (4, 33, 5, 5, 1.3, 4),
])
def test_streaming_two_branch_merge_matches(seed, n, d, dv, h, block):
    # large query scale: the per-row maxima move a lot, so the rescale is exercised
    q, k, v, rho = rand_case(seed, n, d, dv, qscale=2.5)
    for i in range(n):
        ref = streaming_two_branch(q[i], k[: i + 1], v[: i + 1], rho[i], h, block)
        got = parallax_row(q[i], k[: i + 1], v[: i + 1], rho[i], h)
        assert relerr(got, ref) < 1e-10, (i, relerr(got, ref))


def test_zero_probe_is_softmax_attention():
    # blog, "Perspectives on Parallax": a zero probe leaves the intercept, softmax attention
    q, k, v, _ = rand_case(11, 30, 6)
    for i in range(30):
        s = k[: i + 1] @ q[i] / 1.7
        p = np.exp(s - s.max())
        ref = (p / p.sum()) @ v[: i + 1]
        got = parallax_row(q[i], k[: i + 1], v[: i + 1], np.zeros(6), 1.7)
        assert relerr(got, ref) < 1e-13


def test_solved_probe_with_boundary_factor_reproduces_lla():
    # Appendix B: LLA = o_SA - (1 + eta) Sigma_KV rho*, with rho* = Sigma_i^{-1} mu_i from the
    # uncentred moments of section 2 (raw weights) and eta = tbar / (1 - tbar).  Parallax with
    # the probe (1 + eta) rho* is therefore LLA; the LLA oracle is pinned by brute force.
    q, k, v, _ = rand_case(21, 24, 5, 4, qscale=1.5)
    h, lam = 1.7, 0.05
    for i in range(24):
        K, V = k[: i + 1], v[: i + 1]
        w = np.exp(K @ q[i] / h)
        Z = K - q[i]
        mu = w @ Z
        Sigma = (Z * w[:, None]).T @ Z + lam * np.eye(5)
        rho_star = np.linalg.solve(Sigma, mu)
        tbar = (w / w.sum()) @ (Z @ rho_star)
        eta = tbar / (1.0 - tbar)
        got = parallax_row(q[i], K, V, (1.0 + eta) * rho_star, h)
        assert relerr(got, lla_row(q[i], K, V, h, lam)) < 1e-9, i


def test_centred_scoring_form():
    # arXiv page, Parallax paragraph: eta = 0 is the scoring form with centred scores
    # t_ij - tbar_i and denominator omega_i; its combined weights sum to one.
    q, k, v, rho = rand_case(31, 20, 4, 6, qscale=1.2)
    h = 0.9
    for i in range(20):
        K, V = k[: i + 1], v[: i + 1]
        w = np.exp(K @ q[i] / h)
        t = (K - q[i]) @ rho[i]
        tbar = w @ t / w.sum()
        s = w * (1.0 - (t - tbar)) / w.sum()
        assert abs(s.sum() - 1.0) < 1e-12
        assert relerr(parallax_row(q[i], K, V, rho[i], h), s @ V) < 1e-11


def test_library_weighted_covariance():
    # Sigma_KV from numpy's weighted covariance (aweights = softmax weights, no bias
    # correction), values stacked over keys
    q, k, v, rho = rand_case(41, 25, 5, 3)
    h = 1.1
    for i in range(1, 25):
        K, V = k[: i + 1], v[: i + 1]
        s = K @ q[i] / h
        p = np.exp(s - s.max())
        p /= p.sum()
        C = np.cov(np.vstack([V.T, K.T]), aweights=p, bias=True)[:3, 3:]
        ref = p @ V - C @ rho[i]
        assert relerr(parallax_row(q[i], K, V, rho[i], h), ref) < 1e-11


def test_wide_bandwidth_limit_is_uniform_covariance():
    # h -> infinity: uniform weights, o = mean(v) - cov(v, k) rho over the prefix
    q, k, v, rho = rand_case(42, 16, 4)
    for i in range(1, 16):
        K, V = k[: i + 1], v[: i + 1]
        C = np.cov(V.T, K.T, bias=True)[:4, 4:]
        ref = V.mean(0) - C @ rho[i]
        assert relerr(parallax_row(q[i], K, V, rho[i], 1e15), ref) < 1e-9


def test_two_keys_in_one_dimension_closed_form():
    # d = 1, keys k0, k1: Sigma_KV = p0 p1 (v1 - v0)(k1 - k0), o = vbar - Sigma_KV rho
    K = np.array([[0.4], [-1.3]])
    V = np.array([[2.0], [-0.5]])
    for qv, r in ((0.7, 0.3), (-2.0, -1.5), (3.0, 4.0)):
        s = K[:, 0] * qv / 0.6
        p0 = 1.0 / (1.0 + np.exp(s[1] - s[0]))
        p1 = 1.0 - p0
        expect = p0 * V[0, 0] + p1 * V[1, 0] - p0 * p1 * (V[1, 0] - V[0, 0]) * (K[1, 0] - K[0, 0]) * r
        got = parallax_row(np.array([qv]), K, V, np.array([r]), 0.6)
        assert abs(got[0] - expect) < 1e-13


# ---------------------------------------------------------------- invariances of the definition
def test_first_row_is_its_own_value():
    q, k, v, rho = rand_case(51, 3, 6, rscale=10.0)
    assert np.allclose(parallax_row(q[0], k[:1], v[:1], rho[0], 2.0), v[0], rtol=0, atol=1e-13)


def test_affine_in_probe_linear_in_values_and_shift_rules():
    q, k, v, rho = rand_case(61, 18, 5)
    rng = np.random.default_rng(62)
    rho2 = rng.standard_normal(rho.shape)
    v2 = rng.standard_normal(v.shape)
    c = rng.standard_normal(5)
    h = 1.4
    for i in range(18):
        K, V = k[: i + 1], v[: i + 1]
        o0 = parallax_row(q[i], K, V, np.zeros(5), h)
        o1 = parallax_row(q[i], K, V, rho[i], h)
        o2 = parallax_row(q[i], K, V, rho2[i], h)
        o12 = parallax_row(q[i], K, V, 2.0 * rho[i] - 3.0 * rho2[i], h)
        assert relerr(o12 - o0, 2.0 * (o1 - o0) - 3.0 * (o2 - o0)) < 1e-9
        # linear in V, equivariant to a value shift
        ov = parallax_row(q[i], K, 2.0 * V - v2[: i + 1], rho[i], h)
        ref = 2.0 * o1 - parallax_row(q[i], K, v2[: i + 1], rho[i], h)
        assert relerr(ov, ref) < 1e-10
        assert relerr(parallax_row(q[i], K, V + c, rho[i], h), o1 + c) < 1e-12
        # a common key shift rescales every weight by the same factor and leaves the
        # covariance unchanged: the output does not move
        assert relerr(parallax_row(q[i], K + c, V, rho[i], h), o1) < 1e-10


def test_invariant_to_joint_rotation_of_queries_keys_and_probe():
    q, k, v, rho = rand_case(71, 14, 4)
    Qm, _ = np.linalg.qr(np.random.default_rng(72).standard_normal((4, 4)))
    for i in range(14):
        a = parallax_row(q[i], k[: i + 1], v[: i + 1], rho[i], 1.2)
        b = parallax_row(Qm @ q[i], k[: i + 1] @ Qm.T, v[: i + 1], Qm @ rho[i], 1.2)
        assert relerr(b, a) < 1e-11


def test_causal_prefix_only():
    w = lla_inputs.WORKLOADS["parallax_d12"].with_shape(B=1, H=1, n=24, d=4)
    q, k, v, _ = lla_inputs.generate(w)
    rho, _ = lla_inputs.generate_probe(w)
    out = parallax_forward(q, k, v, rho, w.h)[0, 0]
    k2, v2, rho2 = k.copy(), v.copy(), rho.copy()
    k2[..., 12:, :] += 3.0
    v2[..., 12:, :] -= 5.0
    rho2[..., 12:, :] *= -2.0
    out2 = parallax_forward(q, k2, v2, rho2, w.h)[0, 0]
    assert np.array_equal(out[:12], out2[:12])
    assert not np.allclose(out[12:], out2[12:])


def test_row_subset_and_pool_match_full_forward():
    w = lla_inputs.WORKLOADS["parallax_d12"].with_shape(B=2, H=2, n=40, d=4)
    q, k, v, _ = lla_inputs.generate(w)
    rho, _ = lla_inputs.generate_probe(w)
    full = parallax_forward(q, k, v, rho, w.h)
    rows = [(1, 0, 39), (0, 1, 0), (1, 1, 17), (0, 0, 5)]
    got = parallax_rows(q, k, v, rho, w.h, rows, workers=2)
    for t, (b, hh, i) in enumerate(rows):
        assert np.array_equal(got[t], full[b, hh, i])
    parts = parallax_row_parts(q[0, 0, 9], k[0, 0, :10], v[0, 0, :10], rho[0, 0, 9], w.h)
    assert abs(parts["p"].sum() - 1.0) < 1e-14
    assert np.array_equal(parts["o"], full[0, 0, 9])


# ---------------------------------------------------------------- decode (one query against a cache)
def test_decode_is_the_last_row_of_the_causal_forward():
    from oracle import parallax_decode
    rng = np.random.default_rng(81)
    B, H, L, d = 2, 3, 37, 5
    qs, k, v, rhos = (rng.standard_normal((B, H, L, d)) for _ in range(4))
    full = parallax_forward(qs, k, v, rhos, 1.3)
    dec = parallax_decode(qs[:, :, -1], k, v, rhos[:, :, -1], 1.3)
    assert np.array_equal(dec, full[:, :, -1])


def test_decode_ignores_cache_order_and_negligible_keys():
    # every cached key is visible to the decode query: the output does not depend on the
    # order of the cache, and a key whose weight underflows changes nothing
    from oracle import parallax_decode
    rng = np.random.default_rng(82)
    B, H, L, d = 1, 2, 50, 6
    q, rho = rng.standard_normal((B, H, d)), rng.standard_normal((B, H, d))
    k, v = rng.standard_normal((B, H, L, d)), rng.standard_normal((B, H, L, d))
    base = parallax_decode(q, k, v, rho, 0.9)
    perm = rng.permutation(L)
    assert relerr(parallax_decode(q, k[:, :, perm], v[:, :, perm], rho, 0.9), base) < 1e-12
    far = -50.0 * q[:, :, None, :] / np.linalg.norm(q, axis=-1)[..., None, None]
    k2 = np.concatenate([k, far], axis=2)
    v2 = np.concatenate([v, rng.standard_normal((B, H, 1, d))], axis=2)
    assert relerr(parallax_decode(q, k2, v2, rho, 0.9), base) < 1e-12


# ---------------------------------------------------------------- backward
def _bwd_case(seed, B=1, H=2, n=7, d=3, qscale=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, n, d)) * qscale
    k, v, rho, dout = (rng.standard_normal((B, H, n, d)) for _ in range(4))
    return q, k, v, rho, dout


def test_backward_forward_matches_the_definition():
    # the oracle differentiates a torch transcription of the definition; it must be the
    # same function as the pinned numpy forward
    import torch
    from oracle.parallax_oracle import _parallax_head_torch
    q, k, v, rho, _ = _bwd_case(91, n=12, d=4)
    ref = parallax_forward(q, k, v, rho, 1.3)
    for hh in range(2):
        got = _parallax_head_torch(*(torch.tensor(x[0, hh]) for x in (q, k, v, rho)), 1.3).numpy()
        assert relerr(got, ref[0, hh]) < 1e-12


def test_backward_matches_central_differences():
    # every gradient entry against a central difference of sum(o * dout), with o from the
    # numpy forward (no autograd involved)
    from oracle import parallax_backward
    q, k, v, rho, dout = _bwd_case(92, qscale=1.5)
    h = 0.9
    grads = parallax_backward(q, k, v, rho, h, dout)
    base = [q, k, v, rho]
    eps = 1e-6
    for which, g in enumerate(grads):
        num = np.zeros_like(g)
        for idx in np.ndindex(g.shape):
            xs = [x.copy() for x in base]
            xs[which][idx] += eps
            lp = np.sum(parallax_forward(*xs, h) * dout)
            xs[which][idx] -= 2 * eps
            lm = np.sum(parallax_forward(*xs, h) * dout)
            num[idx] = (lp - lm) / (2 * eps)
        assert np.max(np.abs(num - g)) <= 1e-7 * max(1.0, np.max(np.abs(g))), which


def closed_form_backward(q, k, v, rho, h, dout):
    """The gradients in closed form, one head (the row-tile / column-tile quantities of the
    blog's Appendix F, derived from the scoring form o_i = sum_j a_ij v_j,
    a_ij = p_ij (1 - (u_ij - ubar_i))): g = dO V^T, G_i = sum_j p_ij g_ij,
    dp = g (1 - u + ubar) + u G, du = p (G - g), ds = p (dp - sum_j p dp),
    dq = ds K / h, dk = ds^T Q / h + du^T R, dv = a^T dO, drho = du K."""
    n = q.shape[0]
    s = q @ k.T / h
    s[np.triu_indices(n, 1)] = -np.inf
    p = np.exp(s - s.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    u = rho @ k.T
    ubar = np.sum(p * u, -1, keepdims=True)
    a = p * (1 - u + ubar)
    g = dout @ v.T
    G = np.sum(p * g, -1, keepdims=True)
    dp = g * (1 - u + ubar) + u * G
    du = p * (G - g)
    ds = p * (dp - np.sum(p * dp, -1, keepdims=True))
    return ds @ k / h, ds.T @ q / h + du.T @ rho, a.T @ dout, du @ k


def test_backward_closed_form():
    from oracle import parallax_backward
    q, k, v, rho, dout = _bwd_case(93, B=2, H=2, n=20, d=5, qscale=1.2)
    grads = parallax_backward(q, k, v, rho, 1.1, dout)
    for b in range(2):
        for hh in range(2):
            cf = closed_form_backward(q[b, hh], k[b, hh], v[b, hh], rho[b, hh], 1.1, dout[b, hh])
            for got, ref in zip((g[b, hh] for g in grads), cf):
                assert relerr(got, ref) < 1e-10


def test_backward_zero_probe_is_softmax_attention_backward():
    # with rho = 0 the gradients are those of softmax attention (FlashAttention's closed
    # form: dv = P^T dO, ds = P (dO V^T - rowsum(P dO V^T)), dq = ds K / h, dk = ds^T Q / h)
    from oracle import parallax_backward
    q, k, v, _, dout = _bwd_case(94, n=15, d=4)
    rho = np.zeros_like(q)
    dq, dk, dv, drho = parallax_backward(q, k, v, rho, 1.7, dout)
    for hh in range(2):
        Q, K, V, dO = q[0, hh], k[0, hh], v[0, hh], dout[0, hh]
        s = Q @ K.T / 1.7
        s[np.triu_indices(15, 1)] = -np.inf
        P = np.exp(s - s.max(-1, keepdims=True))
        P /= P.sum(-1, keepdims=True)
        dP = dO @ V.T
        dS = P * (dP - np.sum(P * dP, -1, keepdims=True))
        assert relerr(dv[0, hh], P.T @ dO) < 1e-12
        assert relerr(dq[0, hh], dS @ K / 1.7) < 1e-12
        assert relerr(dk[0, hh], dS.T @ Q / 1.7) < 1e-12
        # the probe gradient is then drho_i = sum_j p_ij (G_i - g_ij) k_j, not zero
        G = np.sum(P * dP, -1, keepdims=True)
        assert relerr(drho[0, hh], (P * (G - dP)) @ K) < 1e-12
