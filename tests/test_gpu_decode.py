"""GPU parity of the two decode steps (one query per head against its key-value cache)
against the fp64 oracles.

Parallax decode: every (batch, head) output is compared: small caches (one chunk per head,
written directly) and long ones (several chunks merged by the second launch), every
supported head size and both dtypes, and the four decode workloads at full size.  The
kernels compute in fp32, so besides the contract bars (1e-4 fp32, 3e-3 bf16 inputs) they
are held to 2e-5.

LLA decode: every (batch, head) output against the LLA oracle applied to the head's whole
cache: caches shorter than twice the head size (fp64 moments), longer ones (fp32 matrix-core
moments, several chunks), every head size, both dtypes, lambda at 0 and at a size where the
result is softmax attention, the decode workload at full size, and the workspace entry point.
"""
import numpy as np
import pytest

import lla_inputs
from oracle import parallax_decode as oracle_decode
from parity_util import TOL, require_gpu, row_errors, to_device

pytestmark = pytest.mark.gpu

FP32_BOUND = 2e-5


def arrays(name, **shape):
    w = lla_inputs.DECODE_WORKLOADS[name]
    if shape:
        w = w.with_shape(**shape)
    return (w,) + lla_inputs.generate_decode(w)


def run(q, k, v, rho, dtype, h):
    import torch
    from local_linear_attention_amd import lla_parallax_decode
    tq, tk, tv, tr = (to_device(x, dtype) for x in (q, k, v, rho))
    out = lla_parallax_decode(tq, tk, tv, tr, h)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def check(got, ref, dtype, label):
    err = row_errors(got, ref)
    worst = float(err.max())
    print(f"[decode parity] {label} rows={err.size} max_row_err={worst:.3e}", flush=True)
    assert np.isfinite(got).all(), label
    assert worst <= TOL[dtype], (label, worst)
    assert worst <= FP32_BOUND, (label, worst)


SMALL = [
    ({"B": 1, "H": 1, "L": 1}, {}),
    ({"B": 2, "H": 3, "L": 2}, {}),
    ({"B": 2, "H": 3, "L": 63}, {}),
    ({"B": 1, "H": 2, "L": 300}, {}),
    ({"B": 1, "H": 1, "L": 5000}, {}),          # many chunks, ragged last one
    ({"B": 1, "H": 1, "L": 2049}, {}),
    ({"B": 3, "H": 2, "L": 700, "d": 16}, {}),
    ({"B": 3, "H": 2, "L": 700, "d": 32}, {}),
    ({"B": 2, "H": 2, "L": 1000, "d": 128, "h": 11.3}, {}),
    ({"B": 2, "H": 3, "L": 900, "dtype": "f32"}, {}),
    ({"B": 1, "H": 2, "L": 600, "d": 128, "dtype": "f32", "h": 11.3}, {}),
    ({"B": 600, "H": 4, "L": 40}, {}),            # one chunk per head, many heads
]


@pytest.mark.parametrize("shape,_", SMALL, ids=[str(s) for s, _ in SMALL])
def test_small_caches_every_head(shape, _):
    require_gpu()
    w, q, k, v, rho = arrays("decode_b8_l8192", **shape)
    ref = oracle_decode(q, k, v, rho, w.h)
    got = run(q, k, v, rho, w.dtype, w.h)
    check(got, ref, w.dtype, str(shape))


@pytest.mark.parametrize("name", ["decode_b8_l8192", "decode_b1_l32768", "decode_b64_l1024", "decode_d128"])
def test_workload_every_head(name):
    require_gpu()
    w, q, k, v, rho = arrays(name)
    ref = oracle_decode(q, k, v, rho, w.h)
    got = run(q, k, v, rho, w.dtype, w.h)
    check(got, ref, w.dtype, name)


def test_workspace_entry_point_and_profile():
    torch = require_gpu()
    from local_linear_attention_amd import (LLAError, lla_parallax_decode, lla_parallax_decode_workspace_size,
                                            lla_parallax_decode_ws, lla_profile_collect, lla_profile_enable)
    w, q, k, v, rho = arrays("decode_b8_l8192", B=2, H=2, L=3000)
    tq, tk, tv, tr = (to_device(x, "bf16") for x in (q, k, v, rho))
    nbytes = lla_parallax_decode_workspace_size(w.B, w.H, w.L, w.d, "bf16")
    assert nbytes > 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    lla_profile_enable(True)
    try:
        a = lla_parallax_decode_ws(tq, tk, tv, tr, w.h, ws)
        rec = lla_profile_collect()
    finally:
        lla_profile_enable(False)
    b = lla_parallax_decode(tq, tk, tv, tr, w.h)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert [name for name, _ in rec] == ["lla_parallax_decode_kernel", "lla_parallax_merge_kernel"]
    with pytest.raises(LLAError, match="WORKSPACE"):
        lla_parallax_decode_ws(tq, tk, tv, tr, w.h, ws[: nbytes // 2])
    # one chunk per head: no scratch, one launch
    w1, q1, k1, v1, r1 = arrays("decode_b8_l8192", B=64, H=16, L=64)
    assert lla_parallax_decode_workspace_size(w1.B, w1.H, w1.L, w1.d, "bf16") == 0
    t1 = [to_device(x, "bf16") for x in (q1, k1, v1, r1)]
    c = lla_parallax_decode_ws(*t1, w1.h, None)
    torch.cuda.synchronize()
    check(c.cpu().numpy().astype(np.float64), oracle_decode(q1, k1, v1, r1, w1.h), "bf16", "no scratch")


def test_decode_matches_the_forward_last_row():
    # the decode query is the newest position: the Parallax forward over the same positions
    # gives the same last row (both paths, up to their rounding)
    torch = require_gpu()
    from local_linear_attention_amd import lla_parallax_forward
    w, q, k, v, rho = arrays("decode_b8_l8192", B=1, H=2, L=700)
    qs = np.array(lla_inputs.round_to_bf16(np.random.default_rng(9).standard_normal(k.shape).astype(np.float32)))
    rs = np.array(lla_inputs.round_to_bf16(np.random.default_rng(10).standard_normal(k.shape).astype(np.float32)))
    qs[:, :, -1] = q
    rs[:, :, -1] = rho
    fwd = lla_parallax_forward(*(to_device(x, "bf16") for x in (qs, k, v, rs)), w.h, path="exact")
    torch.cuda.synchronize()
    got = run(q, k, v, rho, "bf16", w.h)
    err = float(row_errors(got, fwd.cpu().numpy()[:, :, -1].astype(np.float64)).max())
    assert err <= FP32_BOUND, err


# ---------------------------------------------------------------- LLA decode
def run_lla(q, k, v, dtype, h, lam):
    import torch
    from local_linear_attention_amd import lla_decode
    tq, tk, tv = (to_device(x, dtype) for x in (q, k, v))
    out = lla_decode(tq, tk, tv, h, lam)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def check_lla(got, ref, dtype, label):
    err = row_errors(got, ref)
    worst = float(err.max())
    print(f"[lla decode parity] {label} rows={err.size} max_row_err={worst:.3e}", flush=True)
    assert np.isfinite(got).all(), label
    assert worst <= TOL[dtype], (label, worst)


LLA_SMALL = [
    {"B": 1, "H": 1, "L": 1},
    {"B": 2, "H": 3, "L": 2},
    {"B": 2, "H": 3, "L": 63},
    {"B": 1, "H": 2, "L": 100},               # L < 2d: fp64 moments
    {"B": 1, "H": 2, "L": 129},               # fp32 moments, three sub-tiles with a ragged one
    {"B": 2, "H": 2, "L": 700},
    {"B": 1, "H": 1, "L": 5000},              # several chunks
    {"B": 3, "H": 2, "L": 700, "d": 16},
    {"B": 3, "H": 2, "L": 700, "d": 32},
    {"B": 2, "H": 2, "L": 1000, "d": 128, "h": 11.3},
    {"B": 1, "H": 2, "L": 300, "d": 128, "h": 11.3},   # L > 2d at d = 128
    {"B": 2, "H": 3, "L": 900, "dtype": "f32"},
    {"B": 1, "H": 2, "L": 40, "dtype": "f32"},
    {"B": 1, "H": 2, "L": 600, "d": 128, "dtype": "f32", "h": 11.3},
    {"B": 300, "H": 4, "L": 200},             # one chunk per head: the solve reads the chunk's moments
    {"B": 64, "H": 16, "L": 1024},            # one chunk per head, fp32 moments
    {"B": 1, "H": 1, "L": 40000},             # 79 chunks summed by the reduce launch
]


@pytest.mark.parametrize("shape", LLA_SMALL, ids=[str(s) for s in LLA_SMALL])
def test_lla_decode_small_caches_every_head(shape):
    require_gpu()
    from oracle import lla_decode as oracle_lla_decode
    w, q, k, v, _ = arrays("lla_decode_b8_l8192", **shape)
    ref = oracle_lla_decode(q, k, v, w.h, w.lam)
    got = run_lla(q, k, v, w.dtype, w.h, w.lam)
    check_lla(got, ref, w.dtype, str(shape))


@pytest.mark.parametrize("lam", [0.0, 1e8])
def test_lla_decode_lambda_extremes(lam):
    # lambda = 0 on caches longer than d (full-rank key covariance); lambda -> infinity gives
    # softmax attention
    require_gpu()
    from oracle import lla_decode as oracle_lla_decode
    w, q, k, v, _ = arrays("lla_decode_b8_l8192", B=2, H=2, L=800)
    ref = oracle_lla_decode(q, k, v, w.h, lam)
    got = run_lla(q, k, v, w.dtype, w.h, lam)
    check_lla(got, ref, w.dtype, f"lambda={lam:g}")


def test_lla_decode_workload_and_forward_last_row():
    torch = require_gpu()
    from local_linear_attention_amd import (lla_decode, lla_decode_workspace_size, lla_decode_ws, lla_forward_ex,
                                            lla_profile_collect, lla_profile_enable)
    from oracle import lla_decode as oracle_lla_decode
    w, q, k, v, _ = arrays("lla_decode_b8_l8192")
    ref = oracle_lla_decode(q, k, v, w.h, w.lam)
    tq, tk, tv = (to_device(x, "bf16") for x in (q, k, v))
    nbytes = lla_decode_workspace_size(w.B, w.H, w.L, w.d, "bf16")
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    lla_profile_enable(True)
    try:
        a = lla_decode_ws(tq, tk, tv, w.h, w.lam, ws)
        rec = lla_profile_collect()
    finally:
        lla_profile_enable(False)
    b = lla_decode(tq, tk, tv, w.h, w.lam)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert [n for n, _ in rec] == ["lla_decode_stats_kernel", "lla_decode_moments_kernel", "lla_decode_reduce_kernel",
                                   "lla_decode_solve_kernel"]
    check_lla(a.cpu().numpy().astype(np.float64), ref, "bf16", "lla_decode_b8_l8192")
    # the LLA forward's last row over the same positions (matrix-core path) agrees
    w2, q2, k2, v2, _ = arrays("lla_decode_b8_l8192", B=1, H=2, L=700)
    qs = np.array(lla_inputs.round_to_bf16(np.random.default_rng(11).standard_normal(k2.shape).astype(np.float32)))
    qs[:, :, -1] = q2
    fwd = lla_forward_ex(*(to_device(x, "bf16") for x in (qs, k2, v2)), w2.h, w2.lam, path="fast")
    torch.cuda.synchronize()
    dec = run_lla(q2, k2, v2, "bf16", w2.h, w2.lam)
    err = float(row_errors(dec, fwd.cpu().numpy()[:, :, -1].astype(np.float64)).max())
    print(f"[lla decode vs forward last row] {err:.2e}", flush=True)
    assert err <= 2 * TOL["bf16"]
