"""GPU parity: the HIP path against the fp64 oracle on identical seeded inputs.

Small shapes compare every row (several key chunks plus a ragged tail); the five workload
shapes at full size compare a seeded sample of rows (all hard early rows included).
Pass bar (per-row normwise relative error): 1e-4 for fp32 inputs, 3e-3 for bf16 inputs.
The fp64 path is also held to a tighter bound that catches regressions well inside the
contract tolerance.
"""
import numpy as np
import pytest

import lla_inputs
from oracle import lla_forward as oracle_forward
from oracle import lla_rows as oracle_rows
from parity_util import (TOL, oracle_all_rows, oracle_some_rows, require_gpu, row_errors, run_gpu,
                         sample_rows, workload_arrays)

pytestmark = pytest.mark.gpu

EXACT_BOUND = 2e-6   # fp64 path: fp32 output rounding plus fp64 arithmetic
WORKERS = 8


def check(got, ref, dtype, path, label, positions=None, d=None):
    """Per-row normwise errors against the oracle, within the tolerance.  With the rows'
    positions in their sequence and the head size, the worst error of each row range of
    the matrix-core path is reported too: fp64 short rows (i < 2d), explicit cross moment
    (2d <= i < 4d), probe pass (i >= 4d)."""
    err = row_errors(got, ref)
    worst = float(err.max())
    ranges = ""
    if positions is not None and d is not None:
        pos = np.broadcast_to(np.asarray(positions), err.shape)
        for name, lo, hi in (("i<2d", 0, 2 * d), ("2d<=i<4d", 2 * d, 4 * d), ("i>=4d", 4 * d, None)):
            sel = (pos >= lo) & ((pos < hi) if hi is not None else True)
            if sel.any():
                ranges += f" {name}:{float(err[sel].max()):.2e}"
    print(f"[parity] {label} path={path} rows={err.size} max_row_err={worst:.3e}{ranges}", flush=True)
    assert np.isfinite(got).all(), label
    assert worst <= TOL[dtype], (label, worst)
    if path == "exact":
        assert worst <= EXACT_BOUND, (label, worst)
    return worst


# ---------------------------------------------------------------- full-row comparisons
SMALL = [
    # (workload recipe, shape overrides)
    ("tiny", {}),
    ("tiny", {"B": 2, "H": 3, "n": 77}),
    ("halfnormal", {"H": 1, "n": 300}),
    ("d12", {"B": 1, "H": 2, "n": 300}),
    ("d24", {"B": 1, "H": 2, "n": 333}),
    ("long", {"B": 1, "H": 1, "n": 200}),
    ("d12", {"B": 1, "H": 1, "n": 150, "d": 32}),
    ("d12", {"B": 1, "H": 1, "n": 150, "d": 16}),
    ("tiny", {"B": 1, "H": 2, "n": 130, "d": 128, "dtype": "f32"}),
]


@pytest.mark.parametrize("name,shape", SMALL, ids=[f"{n}-{s}" for n, s in SMALL])
@pytest.mark.parametrize("path", ["exact", "default"])
def test_small_shapes_every_row(name, shape, path):
    require_gpu()
    w, q, k, v = workload_arrays(name, **shape)
    ref = oracle_forward(q, k, v, w.h, w.lam, workers=WORKERS)
    got = run_gpu(q, k, v, w.dtype, w.h, w.lam, path=path)
    check(got, ref, w.dtype, path if path != "default" else "auto", f"{name}{shape}")


# Matrix-core path (bf16, d = 64): rows below 2d run on the fp64 kernel, the rest on MFMA.
# Shapes cover no MFMA rows (n <= 2d), one ragged row block, several key tiles with a
# ragged tail, and several heads and batches.
FAST_SMALL = [
    ("d24", {"B": 1, "H": 1, "n": 100}),
    ("d24", {"B": 1, "H": 1, "n": 129}),
    ("d24", {"B": 1, "H": 2, "n": 333}),
    ("d12", {"B": 2, "H": 3, "n": 261}),
    ("d24", {"B": 1, "H": 1, "n": 700}),
]


@pytest.mark.parametrize("name,shape", FAST_SMALL, ids=[f"{n}-{s}" for n, s in FAST_SMALL])
def test_fast_path_every_row(name, shape):
    require_gpu()
    w, q, k, v = workload_arrays(name, **shape)
    ref = oracle_forward(q, k, v, w.h, w.lam, workers=WORKERS)
    got = run_gpu(q, k, v, w.dtype, w.h, w.lam, path="fast")
    check(got, ref, w.dtype, "fast", f"{name}{shape}", positions=np.arange(w.n), d=w.d)


# Matrix-core path at d = 128 (bf16): rows below 4d run on the fp64 kernel, the rest on MFMA
# (key moments and solve, then the probe pass).  Shapes cover no MFMA rows (n <= 4d), one
# ragged row block past 4d, several key tiles with a ragged tail, two heads and two batches.
FAST128_SMALL = [
    ("long", {"B": 1, "H": 1, "n": 500}),
    ("long", {"B": 1, "H": 2, "n": 600}),
    ("long", {"B": 2, "H": 1, "n": 777}),
    ("long", {"B": 1, "H": 1, "n": 1100}),
]


@pytest.mark.parametrize("name,shape", FAST128_SMALL, ids=[f"{n}-{s}" for n, s in FAST128_SMALL])
def test_fast_path_d128_every_row(name, shape):
    require_gpu()
    w, q, k, v = workload_arrays(name, **shape)
    ref = oracle_all_rows(q, k, v, w.h, w.lam)
    got = run_gpu(q, k, v, w.dtype, w.h, w.lam, path="fast")
    check(got, ref, w.dtype, "fast", f"{name}{shape}", positions=np.arange(w.n), d=w.d)


@pytest.mark.parametrize("lam", [0.0, 1e8])
def test_fast_path_d128_extreme_ridge(lam):
    # lambda = 0: rows i >= d have a unique minimiser (rows below d only need to be finite);
    # lambda = 1e8: the ridge dominates and b_i tends to the softmax-weighted mean of the values.
    require_gpu()
    w, q, k, v = workload_arrays("long", B=1, H=1, n=800)
    ref = oracle_all_rows(q, k, v, w.h, lam)
    got = run_gpu(q, k, v, w.dtype, w.h, lam, path="fast")
    assert np.isfinite(got).all()
    lo = w.d if lam == 0.0 else 0
    check(got[..., lo:, :], ref[..., lo:, :], w.dtype, "fast", f"long n=800 lambda={lam:g}",
          positions=np.arange(lo, w.n), d=w.d)


@pytest.mark.parametrize("name", ["d24", "long"])
@pytest.mark.parametrize("case", ["sharp_h", "q_x3", "rank16_keys", "v_2^-16", "v_2^17", "k_offset",
                                  "k_x64_h_x64", "k_x1024_h_x1024"])
def test_default_path_envelope_every_row(name, case):
    # Inputs outside the RMS-normalised regime: AUTO (the matrix-core path for bf16) must still
    # hold the tolerance on every row, handing the rows its checks reject to the fp64 kernel.
    torch = require_gpu()
    from local_linear_attention_amd.lla import lla_forward_fallback_rows, lla_forward_workspace_bytes, lla_forward_ws
    from parity_util import envelope_case, to_device
    w, q, k, v, h, lam = envelope_case(name, case)
    ref = oracle_all_rows(q, k, v, h, lam)
    tq, tk, tv = (to_device(x, "bf16") for x in (q, k, v))
    nbytes = lla_forward_workspace_bytes(w.B, w.H, w.n, w.d, "bf16")
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    got = lla_forward_ws(tq, tk, tv, h, lam, ws).cpu().numpy().astype(np.float64)
    back = lla_forward_fallback_rows(ws, (w.B, w.H, w.n, w.d), "bf16")
    err = row_errors(got, ref)
    print(f"[envelope] {name} {case}: rows handed back {back} of {w.B * w.H * w.n}, "
          f"max row err {np.max(err):.3e}", flush=True)
    assert np.isfinite(got).all()
    assert np.max(err) <= TOL["bf16"]


def test_fast_path_workspace_entry_point_matches():
    torch = require_gpu()
    from local_linear_attention_amd import lla_forward_ex, lla_forward_ws, lla_workspace_size
    from parity_util import to_device
    w, q, k, v = workload_arrays("d24", B=2, H=2, n=400)
    tq, tk, tv = (to_device(x, "bf16") for x in (q, k, v))
    nbytes = lla_workspace_size(w.B, w.H, w.n, w.d, "bf16", "fast")
    from parity_util import fast_workspace_bytes
    assert nbytes == fast_workspace_bytes(w.B * w.H, w.n, w.d)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a = lla_forward_ws(tq, tk, tv, w.h, w.lam, ws, path="fast")
    b = lla_forward_ex(tq, tk, tv, w.h, w.lam, path="fast")
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    from local_linear_attention_amd import LLAError
    with pytest.raises(LLAError, match="WORKSPACE"):
        lla_forward_ws(tq, tk, tv, w.h, w.lam, ws[: nbytes // 2], path="fast")


def test_profiling_records_each_kernel():
    torch = require_gpu()
    from local_linear_attention_amd import lla_forward_ex, lla_profile_collect, lla_profile_enable
    from parity_util import to_device
    w, q, k, v = workload_arrays("d24", B=1, H=2, n=300)
    tq, tk, tv = (to_device(x, "bf16") for x in (q, k, v))
    lla_profile_enable(True)
    try:
        lla_forward_ex(tq, tk, tv, w.h, w.lam, path="fast")
        rec = lla_profile_collect()
    finally:
        lla_profile_enable(False)
    assert [name for name, _ in rec] == ["lla_anchor_kernel", "lla_pack_kernel", "lla_rowmax_kernel",
                                         "lla_rows_kernel", "lla_probe_kernel", "lla_refine_kernel"]
    assert all(ms > 0 for _, ms in rec)


def test_concurrent_host_threads_and_profiling():
    # Two host threads launch forwards on streams of their own at the same time, with the kernel
    # timing on: each output equals its single-threaded result bit for bit, and the timing
    # record holds every launch of both threads, each bracketed on its own.
    torch = require_gpu()
    import threading
    from local_linear_attention_amd import (lla_forward_ws, lla_profile_collect, lla_profile_enable,
                                            lla_workspace_size)
    from parity_util import to_device
    w, q, k, v = workload_arrays("d24", B=1, H=2, n=300)
    cases = [(to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16")),
             (to_device(q, "bf16"), to_device(k, "bf16"), to_device(2.0 * v, "bf16"))]
    nbytes = lla_workspace_size(w.B, w.H, w.n, w.d, "bf16", "fast")
    refs = []
    for tq, tk, tv in cases:
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        refs.append(lla_forward_ws(tq, tk, tv, w.h, w.lam, ws, path="fast"))
    torch.cuda.synchronize()
    outs, errors = [None, None], []
    reps = 3

    def worker(i):
        try:
            stream = torch.cuda.Stream()
            ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
            torch.cuda.synchronize()
            with torch.cuda.stream(stream):
                for _ in range(reps):
                    outs[i] = lla_forward_ws(*cases[i], w.h, w.lam, ws, path="fast", stream=stream)
            stream.synchronize()
        except Exception as e:  # reported below, in the test's own thread
            errors.append(e)

    lla_profile_enable(True)
    try:
        threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        torch.cuda.synchronize()
        rec = lla_profile_collect()
    finally:
        lla_profile_enable(False)
    assert not errors, errors
    for got, ref in zip(outs, refs):
        assert torch.equal(got, ref)
    kernels = ["lla_anchor_kernel", "lla_pack_kernel", "lla_rowmax_kernel", "lla_rows_kernel", "lla_probe_kernel",
               "lla_refine_kernel"]
    assert sorted(name for name, _ in rec) == sorted(kernels * (2 * reps))
    assert all(ms > 0 for _, ms in rec)


def test_tiny_affine_lambda_zero_rows_beyond_d():
    require_gpu()
    w, q, k, v = workload_arrays("tiny_affine")
    ref = oracle_forward(q, k, v, w.h, 0.0)
    got = run_gpu(q, k, v, w.dtype, w.h, 0.0, path="exact")
    assert np.isfinite(got).all()  # rank-deficient rows: unspecified but finite
    check(got[..., w.d:, :], ref[..., w.d:, :], w.dtype, "exact", "tiny_affine rows>=d")


def test_fast_path_lambda_zero_rows_beyond_d():
    # lambda = 0 on the matrix-core path: rows i >= d have a unique minimiser ([Blog] §2 with
    # the ridge removed); rows i < d are rank-deficient and only need to be finite.
    require_gpu()
    w, q, k, v = workload_arrays("d24", B=1, H=2, n=400)
    ref = oracle_forward(q, k, v, w.h, 0.0, workers=WORKERS)
    got = run_gpu(q, k, v, w.dtype, w.h, 0.0, path="fast")
    assert np.isfinite(got).all()
    check(got[..., w.d:, :], ref[..., w.d:, :], w.dtype, "fast", "d24 lambda=0 rows>=d",
          positions=np.arange(w.d, w.n), d=w.d)


def test_fast_path_large_lambda():
    # lambda -> infinity drives b_i to the softmax-weighted mean of the values ([Blog] §2):
    # the ridge term dominates every regime of the path (fp64 short rows, explicit rows,
    # probe rows with tiny solutions and their 2^e scaling).
    require_gpu()
    w, q, k, v = workload_arrays("d24", B=1, H=2, n=400)
    ref = oracle_forward(q, k, v, w.h, 1e8, workers=WORKERS)
    got = run_gpu(q, k, v, w.dtype, w.h, 1e8, path="fast")
    check(got, ref, w.dtype, "fast", "d24 lambda=1e8", positions=np.arange(w.n), d=w.d)


def test_fast_path_linear_in_values():
    # b is linear in V.  Doubling V is exact in bf16 and in every product and sum that
    # touches V except fp16 subnormals (|x| < 2^-14), whose grid does not scale: the output
    # doubles to within rounding far below the tolerance.
    require_gpu()
    w, q, k, v = workload_arrays("d24", B=1, H=2, n=333)
    a = run_gpu(q, k, v, w.dtype, w.h, w.lam, path="fast")
    b = run_gpu(q, k, 2.0 * v, w.dtype, w.h, w.lam, path="fast")
    err = float(row_errors(b, 2.0 * a).max())
    print(f"[linearity] max per-row |b(2v) - 2 b(v)| / |2 b(v)| = {err:.2e}", flush=True)
    assert err <= 1e-5


def test_fast_path_long_sequence_sampled_rows():
    # n = 16384 on the matrix-core path: many tiles per head, the probe pass over long
    # prefixes, the full XCD-ordered grid.
    require_gpu()
    w, q, k, v = workload_arrays("d24", B=1, H=2, n=16384)
    rows = sample_rows(w.B, w.H, w.n, w.d, w.seed, per_head=8)
    got_full = run_gpu(q, k, v, w.dtype, w.h, w.lam, path="fast")
    assert np.isfinite(got_full).all()
    ref = oracle_rows(q, k, v, w.h, w.lam, rows, workers=WORKERS)
    got = np.stack([got_full[b, hh, i] for (b, hh, i) in rows])
    check(got, ref, w.dtype, "fast", "d24 n=16384 sampled", positions=np.array([i for (_, _, i) in rows]), d=w.d)


def test_single_position_returns_value():
    require_gpu()
    w, q, k, v = workload_arrays("d24", B=2, H=3, n=1)
    got = run_gpu(q, k, v, w.dtype, w.h, w.lam)
    assert np.array_equal(got, v.astype(np.float64))


# ---------------------------------------------------------------- full-size workloads
# The contract metric is the worst per-row error over every (b, h, i).  The d = 64 workloads
# at full size compare every row against the oracle (about a minute of CPU in the oracle's
# process pool for the largest); the worst error of each row range is printed.
@pytest.mark.parametrize("name", ["halfnormal", "d12", "d24"])
def test_full_size_workload_every_row(name):
    require_gpu()
    w, q, k, v = workload_arrays(name)
    got = run_gpu(q, k, v, w.dtype, w.h, w.lam, path="default")
    assert np.isfinite(got).all()
    ref = oracle_all_rows(q, k, v, w.h, w.lam)
    check(got, ref, w.dtype, "auto", f"{name} full size, every row", positions=np.arange(w.n), d=w.d)


# The d = 128 long-context workload (2^17 rows of up to 16384 keys, about 16 times the
# oracle work of the d = 64 headline) compares a stratified sample: every row i < 4d of head 0,
# the first 64 rows past 2d and past 4d of every head, random rows of every head and the last
# row of every head.
def test_full_size_long_workload_stratified_rows():
    require_gpu()
    w, q, k, v = workload_arrays("long")
    got_full = run_gpu(q, k, v, w.dtype, w.h, w.lam, path="default")
    assert np.isfinite(got_full).all()
    rng = np.random.default_rng(4321)
    d = w.d
    rows = {(0, 0, i) for i in range(4 * d)}
    for hh in range(w.H):
        rows |= {(0, hh, i) for i in range(2 * d, 2 * d + 64)}
        rows |= {(0, hh, i) for i in range(4 * d, 4 * d + 64)}
        rows |= {(0, hh, int(i)) for i in rng.integers(0, w.n, 24)}
        rows.add((0, hh, w.n - 1))
    rows = sorted(rows)
    ref = oracle_some_rows(q, k, v, w.h, w.lam, rows)
    got = np.stack([got_full[b, hh, i] for (b, hh, i) in rows])
    check(got, ref, w.dtype, "auto", f"long full size, {len(rows)} stratified rows",
          positions=np.array([i for (_, _, i) in rows]), d=d)


# ---------------------------------------------------------------- properties
def test_deterministic_reruns():
    require_gpu()
    w, q, k, v = workload_arrays("d24", B=1, H=4, n=512)
    a = run_gpu(q, k, v, w.dtype, w.h, w.lam)
    b = run_gpu(q, k, v, w.dtype, w.h, w.lam)
    assert np.array_equal(a, b)


def test_causal_future_does_not_leak():
    require_gpu()
    w, q, k, v = workload_arrays("d12", B=1, H=2, n=256)
    a = run_gpu(q, k, v, w.dtype, w.h, w.lam)
    k2, v2 = k.copy(), v.copy()
    k2[..., 200:, :] = lla_inputs.round_to_bf16(k2[..., 200:, :] * 1.5)
    v2[..., 200:, :] = -v2[..., 200:, :]
    b = run_gpu(q, k2, v2, w.dtype, w.h, w.lam)
    assert np.array_equal(a[..., :200, :], b[..., :200, :])
    assert not np.allclose(a[..., 200:, :], b[..., 200:, :])
