"""GPU parity of the Parallax forward (given probe) against the fp64 Parallax oracle.

Small shapes compare every row (several key tiles plus a ragged tail, several row blocks,
head counts that do not fill the 8-head XCD groups); the Parallax workloads at full size
compare a seeded sample of rows.  Pass bar (per-row normwise relative error): 1e-4 for fp32
inputs, 3e-3 for bf16 inputs; the fp64 path is also held to a tight bound.
"""
import numpy as np
import pytest

import lla_inputs
from oracle import parallax_forward as oracle_forward
from oracle import parallax_rows as oracle_rows
from parity_util import TOL, require_gpu, row_errors, sample_rows, to_device

pytestmark = pytest.mark.gpu

EXACT_BOUND = 2e-6
WORKERS = 8


def arrays(name, **shape):
    w = lla_inputs.WORKLOADS[name]
    if shape:
        w = w.with_shape(**shape)
    q, k, v, _ = lla_inputs.generate(w)
    rho, _ = lla_inputs.generate_probe(w)
    return w, q, k, v, rho


def run(q, k, v, rho, dtype, h, path="auto"):
    import torch
    from local_linear_attention_amd import lla_parallax_forward
    tq, tk, tv, tr = (to_device(x, dtype) for x in (q, k, v, rho))
    out = lla_parallax_forward(tq, tk, tv, tr, h, path=path)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def check(got, ref, dtype, path, label):
    err = row_errors(got, ref)
    worst = float(err.max())
    print(f"[parallax parity] {label} path={path} rows={err.size} max_row_err={worst:.3e} "
          f"median={float(np.median(err)):.2e}", flush=True)
    assert np.isfinite(got).all(), label
    assert worst <= TOL[dtype], (label, worst)
    if path == "exact":
        assert worst <= EXACT_BOUND, (label, worst)
    return worst


FAST_SMALL = [
    ("parallax_d24", {"B": 1, "H": 1, "n": 1}),
    ("parallax_d24", {"B": 1, "H": 1, "n": 63}),
    ("parallax_d24", {"B": 1, "H": 1, "n": 129}),
    ("parallax_d24", {"B": 1, "H": 2, "n": 333}),
    ("parallax_d12", {"B": 2, "H": 3, "n": 261}),
    ("parallax_d24", {"B": 1, "H": 9, "n": 300}),
    ("parallax_d24", {"B": 1, "H": 1, "n": 1000}),
]


@pytest.mark.parametrize("name,shape", FAST_SMALL, ids=[f"{n}-{s}" for n, s in FAST_SMALL])
@pytest.mark.parametrize("path", ["fast", "exact"])
def test_every_row(name, shape, path):
    require_gpu()
    w, q, k, v, rho = arrays(name, **shape)
    ref = oracle_forward(q, k, v, rho, w.h, workers=WORKERS)
    got = run(q, k, v, rho, w.dtype, w.h, path=path)
    check(got, ref, w.dtype, path, f"{name}{shape}")


EXACT_SMALL = [
    ("parallax_d12", {"B": 1, "H": 2, "n": 150, "d": 16, "dtype": "f32"}),
    ("parallax_d12", {"B": 2, "H": 1, "n": 130, "d": 32, "dtype": "f32"}),
    ("parallax_d12", {"B": 1, "H": 2, "n": 300, "d": 64, "dtype": "f32"}),
    ("parallax_d12", {"B": 1, "H": 1, "n": 260, "d": 128, "dtype": "f32"}),
    ("parallax_d12", {"B": 1, "H": 2, "n": 200, "d": 128}),
    ("parallax_d12", {"B": 1, "H": 1, "n": 90, "d": 16}),
]


@pytest.mark.parametrize("name,shape", EXACT_SMALL, ids=[f"{n}-{s}" for n, s in EXACT_SMALL])
def test_exact_path_other_shapes_and_auto_choice(name, shape):
    # fp32 inputs and heads other than 64 run on the fp64 path, which AUTO picks for them.
    require_gpu()
    w, q, k, v, rho = arrays(name, **shape)
    ref = oracle_forward(q, k, v, rho, w.h, workers=WORKERS)
    for path in ("exact", "auto"):
        got = run(q, k, v, rho, w.dtype, w.h, path=path)
        check(got, ref, w.dtype, "exact", f"{name}{shape} ({path})")


def test_zero_probe_is_softmax_attention():
    require_gpu()
    w, q, k, v, rho = arrays("parallax_d24", B=1, H=2, n=300)
    zero = np.zeros_like(rho)
    ref = oracle_forward(q, k, v, zero, w.h)
    got = run(q, k, v, zero, w.dtype, w.h, path="fast")
    check(got, ref, w.dtype, "fast", "zero probe")


@pytest.mark.parametrize("scale", [2.0 ** 20, 2.0 ** -20])
def test_probe_scale_extremes(scale):
    # The per-query power-of-two scaling of the probe scores keeps P2 in fp16 range for
    # large probes and away from fp16 underflow for small ones; scaling rho by a power of
    # two is exact in bf16.
    require_gpu()
    w, q, k, v, rho = arrays("parallax_d24", B=1, H=2, n=300)
    rs = lla_inputs.round_to_bf16((rho * scale).astype(np.float32))
    ref = oracle_forward(q, k, v, rs, w.h)
    got = run(q, k, v, rs, w.dtype, w.h, path="fast")
    check(got, ref, w.dtype, "fast", f"rho x {scale:g}")


def test_key_offset():
    # A common key offset leaves the result unchanged (softmax weights rescale by one factor,
    # the covariance does not move); the kernel's centring at the head's mean key keeps the
    # probe scores small.  The offset is chosen exactly representable.
    require_gpu()
    w, q, k, v, rho = arrays("parallax_d24", B=1, H=2, n=300)
    k2 = lla_inputs.round_to_bf16((k + 4.0).astype(np.float32))
    ref = oracle_forward(q, k2, v, rho, w.h)
    got = run(q, k2, v, rho, w.dtype, w.h, path="fast")
    check(got, ref, w.dtype, "fast", "keys + 4")


@pytest.mark.parametrize("scale", [2.0 ** -16, 2.0 ** 17])
def test_value_range_guard(scale):
    # The matrix-core path holds the values as fp16: a head whose largest |v| falls below
    # 2^-10 or reaches 2^16 goes to the fp64 row code instead.  Only head 1 of three is
    # scaled (a power of two, exact in bf16); every row of every head is compared, and the
    # listed head must carry the fp64 path's accuracy.
    require_gpu()
    w, q, k, v, rho = arrays("parallax_d24", B=1, H=3, n=333)
    v2 = v.copy()
    v2[:, 1] = lla_inputs.round_to_bf16((v[:, 1] * scale).astype(np.float32))
    ref = oracle_forward(q, k, v2, rho, w.h)
    got = run(q, k, v2, rho, w.dtype, w.h, path="auto")
    check(got, ref, w.dtype, "fast", f"head 1 values x {scale:g}")
    listed = float(row_errors(got[:, 1:2], ref[:, 1:2]).max())
    assert listed <= EXACT_BOUND, listed


def test_value_range_guard_list_is_per_call():
    # Two calls on one workspace: the first lists a head, the second (values in range) must
    # not run the fp64 code over a stale list -- its result equals a fresh call's, bitwise.
    torch = require_gpu()
    from local_linear_attention_amd import lla_parallax_forward, lla_parallax_forward_ws, lla_parallax_workspace_size
    w, q, k, v, rho = arrays("parallax_d24", B=1, H=2, n=300)
    v2 = v.copy()
    v2[:, 0] = lla_inputs.round_to_bf16((v[:, 0] * 2.0 ** 18).astype(np.float32))
    tq, tk, tv, tv2, tr = (to_device(x, "bf16") for x in (q, k, v, v2, rho))
    ws = torch.empty(lla_parallax_workspace_size(w.B, w.H, w.n, w.d, "bf16", "fast"), dtype=torch.uint8,
                     device="cuda")
    first = lla_parallax_forward_ws(tq, tk, tv2, tr, w.h, ws, path="fast")
    second = lla_parallax_forward_ws(tq, tk, tv, tr, w.h, ws, path="fast")
    fresh = lla_parallax_forward(tq, tk, tv, tr, w.h, path="fast")
    torch.cuda.synchronize()
    assert torch.equal(second, fresh)
    ref = oracle_forward(q, k, v2, rho, w.h)
    check(first.cpu().numpy().astype(np.float64), ref, w.dtype, "fast", "head 0 values x 2^18")


def test_workspace_entry_point_matches():
    torch = require_gpu()
    from local_linear_attention_amd import (LLAError, lla_parallax_forward, lla_parallax_forward_ws,
                                            lla_parallax_workspace_size)
    w, q, k, v, rho = arrays("parallax_d24", B=2, H=2, n=400)
    tq, tk, tv, tr = (to_device(x, "bf16") for x in (q, k, v, rho))
    nbytes = lla_parallax_workspace_size(w.B, w.H, w.n, w.d, "bf16", "fast")
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a = lla_parallax_forward_ws(tq, tk, tv, tr, w.h, ws, path="fast")
    b = lla_parallax_forward(tq, tk, tv, tr, w.h, path="fast")
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    with pytest.raises(LLAError, match="WORKSPACE"):
        lla_parallax_forward_ws(tq, tk, tv, tr, w.h, ws[: nbytes // 2], path="fast")


def test_profiling_records_each_kernel():
    torch = require_gpu()
    from local_linear_attention_amd import lla_parallax_forward, lla_profile_collect, lla_profile_enable
    w, q, k, v, rho = arrays("parallax_d24", B=1, H=2, n=300)
    tq, tk, tv, tr = (to_device(x, "bf16") for x in (q, k, v, rho))
    lla_profile_enable(True)
    try:
        lla_parallax_forward(tq, tk, tv, tr, w.h, path="fast")
        rec = lla_profile_collect()
    finally:
        lla_profile_enable(False)
    torch.cuda.synchronize()
    assert [name for name, _ in rec] == ["lla_parallax_pack_kernel", "lla_parallax_kernel",
                                         "lla_parallax_fallback_kernel"]
    assert all(ms > 0 for _, ms in rec)


def test_affine_in_probe_and_deterministic():
    require_gpu()
    w, q, k, v, rho = arrays("parallax_d24", B=1, H=2, n=333)
    zero = np.zeros_like(rho)
    o0 = run(q, k, v, zero, w.dtype, w.h, path="fast")
    o1 = run(q, k, v, rho, w.dtype, w.h, path="fast")
    o2 = run(q, k, v, 2.0 * rho, w.dtype, w.h, path="fast")   # exact doubling in bf16
    again = run(q, k, v, rho, w.dtype, w.h, path="fast")
    assert np.array_equal(o1, again)
    err = float(row_errors(o2 - o0, 2.0 * (o1 - o0)).max())
    print(f"[parallax affine] max per-row error of o(2 rho) - o(0) vs 2 (o(rho) - o(0)): {err:.2e}", flush=True)
    assert err <= 1e-5


def test_causal_future_does_not_leak():
    require_gpu()
    w, q, k, v, rho = arrays("parallax_d12", B=1, H=2, n=256)
    a = run(q, k, v, rho, w.dtype, w.h, path="fast")
    # future values and probes: nothing of them may reach rows before 200
    v2, r2 = v.copy(), rho.copy()
    v2[..., 200:, :] = -v2[..., 200:, :]
    r2[..., 200:, :] = -r2[..., 200:, :]
    b = run(q, k, v2, r2, w.dtype, w.h, path="fast")
    assert np.array_equal(a[..., :200, :], b[..., :200, :])
    assert not np.allclose(a[..., 200:, :], b[..., 200:, :])
    # future keys: they also move the head's mean key and key-norm bound (a centring constant
    # and a power-of-two scale that cancel exactly), so earlier rows agree to rounding
    k2 = k.copy()
    k2[..., 200:, :] = lla_inputs.round_to_bf16(k2[..., 200:, :] * 1.5)
    c = run(q, k2, v, rho, w.dtype, w.h, path="fast")
    err = float(row_errors(c[..., :200, :], a[..., :200, :]).max())
    print(f"[parallax causal] rows < 200 after changing future keys: {err:.2e}", flush=True)
    assert err <= 1e-3


@pytest.mark.parametrize("name", ["parallax_d12", "parallax_d24"])
def test_full_size_workload_sampled_rows(name):
    require_gpu()
    w, q, k, v, rho = arrays(name)
    rows = sample_rows(w.B, w.H, w.n, w.d, w.seed, per_head=40)
    got_full = run(q, k, v, rho, w.dtype, w.h, path="auto")
    assert np.isfinite(got_full).all()
    ref = oracle_rows(q, k, v, rho, w.h, rows, workers=WORKERS)
    got = np.stack([got_full[b, hh, i] for (b, hh, i) in rows])
    check(got, ref, w.dtype, "auto", f"{name} full-size sampled")


def test_long_sequence_sampled_rows():
    require_gpu()
    w, q, k, v, rho = arrays("parallax_d24", B=1, H=2, n=16384)
    rows = sample_rows(w.B, w.H, w.n, w.d, w.seed, per_head=8)
    got_full = run(q, k, v, rho, w.dtype, w.h, path="fast")
    assert np.isfinite(got_full).all()
    ref = oracle_rows(q, k, v, rho, w.h, rows, workers=WORKERS)
    got = np.stack([got_full[b, hh, i] for (b, hh, i) in rows])
    check(got, ref, w.dtype, "fast", "parallax n=16384 sampled")
