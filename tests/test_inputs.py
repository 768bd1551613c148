"""Seeded input generator: determinism, casts, recipe structure (CPU only)."""
import numpy as np
import pytest

import lla_inputs


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    x = (np.random.default_rng(5).standard_normal(200000) * 7).astype(np.float32)
    x[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]  # ties to even
    ours = lla_inputs.round_to_bf16(x)
    ref = torch.tensor(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_generate_is_deterministic_and_exactly_cast():
    w = lla_inputs.WORKLOADS["d12"].with_shape(B=1, H=2, n=32)
    a = lla_inputs.generate(w)
    b = lla_inputs.generate(w)
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x, y)
        assert x.dtype == np.float32 and x.shape == (1, 2, 32, 64)
        assert np.array_equal(lla_inputs.round_to_bf16(x), x)  # exactly bf16


def test_recipes_have_their_structure():
    q, k, v = lla_inputs.make_inputs(1, 2, 256, 64, 1, "halfnormal")
    assert (k[..., 0] >= 0).all() and abs(np.std(q) - 64 ** -0.25) < 0.02
    q, k, v = lla_inputs.make_inputs(1, 2, 64, 64, 2, "rms")
    assert np.allclose(np.mean(q * q, -1), 1.0, atol=1e-5)
    q, k, v, ex = lla_inputs.make_inputs(1, 1, 64, 16, 0, "affine_exact", extras=True)
    q0, k0, _ = lla_inputs.make_inputs(1, 1, 64, 16, 0, "normal")
    assert np.array_equal(q, q0) and np.array_equal(k, k0)  # same q, k as the plain draw
    assert np.allclose(v[0, 0], k[0, 0] @ ex["A"][0, 0].T + ex["c"][0, 0])


def test_probe_stream_is_separate_and_rms_normalised():
    w = lla_inputs.WORKLOADS["parallax_d24"].with_shape(B=1, H=2, n=48)
    base = lla_inputs.WORKLOADS["d24"].with_shape(B=1, H=2, n=48)
    a, b = lla_inputs.generate(w), lla_inputs.generate(base)
    for x, y in zip(a[:3], b[:3]):   # the probe draw leaves q, k, v untouched
        assert np.array_equal(x, y)
    rho, rho64 = lla_inputs.generate_probe(w)
    rho2, _ = lla_inputs.generate_probe(w)
    assert np.array_equal(rho, rho2) and rho.shape == (1, 2, 48, 64) and rho.dtype == np.float32
    assert np.array_equal(lla_inputs.round_to_bf16(rho), rho)
    assert np.allclose(np.mean(rho64 * rho64, -1), 1.0, atol=1e-5)
    assert not np.allclose(rho64, lla_inputs.make_inputs(1, 2, 48, 64, w.seed, "rms")[0])


def test_decode_generator_is_deterministic_and_cast():
    w = lla_inputs.DECODE_WORKLOADS["decode_b8_l8192"].with_shape(B=2, H=3, L=40)
    a, b = lla_inputs.generate_decode(w), lla_inputs.generate_decode(w)
    shapes = [(2, 3, 64), (2, 3, 40, 64), (2, 3, 40, 64), (2, 3, 64)]
    for x, y, shp in zip(a, b, shapes):
        assert np.array_equal(x, y) and x.shape == shp and x.dtype == np.float32
        assert np.array_equal(lla_inputs.round_to_bf16(x), x)
    assert np.allclose(np.mean(a[1].astype(np.float64) ** 2, -1), 1.0, atol=2e-2)


def test_cotangent_stream_is_separate_and_deterministic():
    w = lla_inputs.WORKLOADS["parallax_d12"].with_shape(B=1, H=2, n=50)
    d1, d64 = lla_inputs.generate_cotangent(w)
    d2, _ = lla_inputs.generate_cotangent(w)
    assert np.array_equal(d1, d2)
    assert np.array_equal(d1, lla_inputs.round_to_bf16(d64.astype(np.float32)))
    q, k, v, _ = lla_inputs.generate(w)
    rho, _ = lla_inputs.generate_probe(w)
    for x in (q, k, v, rho):   # its own stream: no draw shared with the forward inputs
        assert not np.allclose(d1, x)
    assert abs(float(np.std(d64)) - 1.0) < 0.05
