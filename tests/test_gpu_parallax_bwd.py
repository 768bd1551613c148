"""GPU parity of the Parallax backward (the gradients of sum(o * dout) with respect to q, k,
v and rho) against the fp64 oracle, which differentiates the forward's definition in reverse
mode, and of the forward's per-row log-sum-exp against its definition.

Error of a gradient row: max|got - ref| / max(max|ref_row|, 1e-3 F_head) -- the row's own
norm, as for the forward outputs, floored at a thousandth of F_head, the largest row of the
four gradients of its head (they share the scale of dout times keys and values), because
some gradient rows are exactly zero: drho of row 0 (one key leaves nothing to correct), and
with a single position dq and dk of the whole head.  Bars: 3e-3 for bf16 inputs, 1e-4 for fp32; the fp64 path is also
held to 1e-5.  Shapes span several 64-position tiles, 128-row blocks and ragged tails.
"""
import numpy as np
import pytest

import lla_inputs
from oracle import parallax_backward as oracle_backward
from parity_util import TOL, require_gpu, row_errors, to_device

pytestmark = pytest.mark.gpu

EXACT_BOUND = 1e-5
NAMES = ("dq", "dk", "dv", "drho")


def arrays(name, **shape):
    w = lla_inputs.WORKLOADS[name]
    if shape:
        w = w.with_shape(**shape)
    q, k, v, _ = lla_inputs.generate(w)
    rho, _ = lla_inputs.generate_probe(w)
    dout, _ = lla_inputs.generate_cotangent(w)
    return w, q, k, v, rho, dout


def grad_row_errors(got, ref, head_scale):
    num = np.max(np.abs(got - ref), axis=-1)
    row = np.max(np.abs(ref), axis=-1)
    return num / np.maximum(np.maximum(row, 1e-3 * head_scale), 1e-30)


def run(q, k, v, rho, dout, dtype, h, path):
    import torch
    from local_linear_attention_amd import lla_parallax_backward, lla_parallax_forward_stats
    t = [to_device(x, dtype) for x in (q, k, v, rho, dout)]
    _, lse = lla_parallax_forward_stats(*t[:4], h, path=path)
    grads = lla_parallax_backward(*t[:4], t[4], lse, h, path=path)
    torch.cuda.synchronize()
    return [g.cpu().numpy().astype(np.float64) for g in grads]


def check(got, ref, dtype, path, label):
    worst = {}
    scale = np.max([np.max(np.abs(r), axis=(-2, -1)) for r in ref], axis=0)[..., None]   # [B, H, 1]
    for nm, g, r in zip(NAMES, got, ref):
        assert np.isfinite(g).all(), (label, nm)
        worst[nm] = float(grad_row_errors(g, r, scale).max())
    print(f"[parallax bwd parity] {label} path={path} " + " ".join(f"{k}={v:.2e}" for k, v in worst.items()),
          flush=True)
    for nm, e in worst.items():
        assert e <= TOL[dtype], (label, nm, e)
        if path == "exact":
            assert e <= EXACT_BOUND, (label, nm, e)


SMALL = [
    ("parallax_d24", {"B": 1, "H": 1, "n": 1}),
    ("parallax_d24", {"B": 1, "H": 1, "n": 63}),
    ("parallax_d24", {"B": 1, "H": 2, "n": 129}),
    ("parallax_d12", {"B": 2, "H": 3, "n": 261}),
    ("parallax_d24", {"B": 1, "H": 9, "n": 300}),
    ("parallax_d24", {"B": 1, "H": 1, "n": 1000}),
]


@pytest.mark.parametrize("name,shape", SMALL, ids=[f"{n}-{s}" for n, s in SMALL])
@pytest.mark.parametrize("path", ["fast", "exact"])
def test_every_gradient_row(name, shape, path):
    require_gpu()
    w, q, k, v, rho, dout = arrays(name, **shape)
    ref = oracle_backward(q, k, v, rho, w.h, dout)
    got = run(q, k, v, rho, dout, w.dtype, w.h, path)
    check(got, ref, w.dtype, path, f"{name}{shape}")


OTHER = [
    {"B": 1, "H": 2, "n": 150, "d": 16, "dtype": "f32"},
    {"B": 2, "H": 1, "n": 130, "d": 32, "dtype": "f32"},
    {"B": 1, "H": 2, "n": 200, "d": 64, "dtype": "f32"},
    {"B": 1, "H": 1, "n": 140, "d": 128, "dtype": "f32"},
    {"B": 1, "H": 2, "n": 100, "d": 128},
    {"B": 1, "H": 1, "n": 90, "d": 16},
]


@pytest.mark.parametrize("shape", OTHER, ids=[str(s) for s in OTHER])
def test_exact_path_other_dtypes_and_heads(shape):
    # fp32 inputs and heads other than 64 run on the fp64 path, which AUTO picks for them
    require_gpu()
    w, q, k, v, rho, dout = arrays("parallax_d12", **shape)
    ref = oracle_backward(q, k, v, rho, w.h, dout)
    for path in ("exact", "auto"):
        check(run(q, k, v, rho, dout, w.dtype, w.h, path), ref, w.dtype, "exact", f"{shape} ({path})")


@pytest.mark.parametrize("path", ["fast", "exact"])
def test_forward_log_sum_exp(path):
    torch = require_gpu()
    from local_linear_attention_amd import lla_parallax_forward, lla_parallax_forward_stats
    w, q, k, v, rho, _ = arrays("parallax_d24", B=1, H=2, n=300)
    t = [to_device(x, "bf16") for x in (q, k, v, rho)]
    out, lse = lla_parallax_forward_stats(*t, w.h, path=path)
    plain = lla_parallax_forward(*t, w.h, path=path)
    torch.cuda.synchronize()
    assert torch.equal(out, plain)   # the same arithmetic, plus an epilogue
    got = lse.cpu().numpy().astype(np.float64)
    q64, k64 = q.astype(np.float64), k.astype(np.float64)
    err = 0.0
    for hh in range(w.H):
        s = q64[0, hh] @ k64[0, hh].T / w.h
        s[np.triu_indices(w.n, 1)] = -np.inf
        m = s.max(-1)
        ref = (m + np.log(np.sum(np.exp(s - m[:, None]), -1))) / np.log(2.0)
        err = max(err, float(np.max(np.abs(got[0, hh] - ref))))
    print(f"[parallax lse] path={path} max abs error {err:.2e}", flush=True)
    assert err <= (1e-3 if path == "fast" else 1e-5)


def test_forward_range_guard_stats_feed_the_backward():
    # A head whose values the forward's matrix-core path cannot hold as fp16 (x 2^17) runs on
    # the fp64 row code, which also writes that head's log-sum-exp: it must agree with the
    # definition like the matrix-core rows' do, and the backward fed with it must still meet
    # the bar on every gradient row of every head.
    torch = require_gpu()
    from local_linear_attention_amd import lla_parallax_forward_stats
    w, q, k, v, rho, dout = arrays("parallax_d24", B=1, H=2, n=300)
    v = v.copy()
    v[:, 1] = lla_inputs.round_to_bf16((v[:, 1] * 2.0 ** 17).astype(np.float32))
    t = [to_device(x, "bf16") for x in (q, k, v, rho)]
    _, lse = lla_parallax_forward_stats(*t, w.h, path="fast")
    torch.cuda.synchronize()
    got_lse = lse.cpu().numpy().astype(np.float64)
    q64, k64 = q.astype(np.float64), k.astype(np.float64)
    for hh in range(w.H):
        s = q64[0, hh] @ k64[0, hh].T / w.h
        s[np.triu_indices(w.n, 1)] = -np.inf
        m = s.max(-1)
        ref_lse = (m + np.log(np.sum(np.exp(s - m[:, None]), -1))) / np.log(2.0)
        err = float(np.max(np.abs(got_lse[0, hh] - ref_lse)))
        print(f"[parallax lse, head {hh} values x {2 ** 17 if hh == 1 else 1}] max abs error {err:.2e}", flush=True)
        assert err <= (1e-5 if hh == 1 else 1e-3)
    got = run(q, k, v, rho, dout, "bf16", w.h, "fast")
    ref = oracle_backward(q, k, v, rho, w.h, dout)
    check(got, ref, "bf16", "fast", "head 1 values x 2^17")


def test_zero_probe_and_determinism():
    require_gpu()
    w, q, k, v, rho, dout = arrays("parallax_d24", B=1, H=2, n=200)
    zero = np.zeros_like(rho)
    ref = oracle_backward(q, k, v, zero, w.h, dout)
    a = run(q, k, v, zero, dout, w.dtype, w.h, "fast")
    check(a, ref, w.dtype, "fast", "zero probe")
    b = run(q, k, v, zero, dout, w.dtype, w.h, "fast")
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_workspace_entry_and_profile():
    torch = require_gpu()
    from local_linear_attention_amd import (LLAError, lla_parallax_backward, lla_parallax_backward_workspace_size,
                                            lla_parallax_forward_stats, lla_parallax_workspace_size,
                                            lla_profile_collect, lla_profile_enable)
    w, q, k, v, rho, dout = arrays("parallax_d24", B=2, H=2, n=400)
    t = [to_device(x, "bf16") for x in (q, k, v, rho, dout)]
    fws = torch.empty(lla_parallax_workspace_size(w.B, w.H, w.n, w.d, "bf16", "fast"), dtype=torch.uint8,
                      device="cuda")
    _, lse = lla_parallax_forward_stats(*t[:4], w.h, path="fast", workspace=fws)
    bws = torch.empty(lla_parallax_backward_workspace_size(w.B, w.H, w.n, w.d, "bf16", "fast"), dtype=torch.uint8,
                      device="cuda")
    lla_profile_enable(True)
    try:
        a = lla_parallax_backward(*t[:4], t[4], lse, w.h, path="fast", workspace=bws)
        rec = lla_profile_collect()
    finally:
        lla_profile_enable(False)
    b = lla_parallax_backward(*t[:4], t[4], lse, w.h, path="fast")
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert [nm for nm, _ in rec] == ["lla_parallax_bwd_pack_kernel", "lla_parallax_bwd_stats_kernel",
                                     "lla_parallax_bwd_kv_kernel", "lla_parallax_bwd_qr_kernel"]
    with pytest.raises(LLAError, match="WORKSPACE"):
        lla_parallax_backward(*t[:4], t[4], lse, w.h, path="fast", workspace=bws[: bws.numel() // 2])


def test_full_length_heads():
    # two heads of the parallax_d24 workload at its full length n = 4096
    require_gpu()
    w, q, k, v, rho, dout = arrays("parallax_d24", B=1, H=2)
    ref = oracle_backward(q, k, v, rho, w.h, dout)
    check(run(q, k, v, rho, dout, w.dtype, w.h, "fast"), ref, w.dtype, "fast", "parallax_d24 B1 H2 n4096")
