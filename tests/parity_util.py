"""Helpers for the GPU parity tests: move seeded inputs to the device, run the library
through its C ABI, pick sample rows, and measure the per-row normwise error."""
import numpy as np

import lla_inputs

TOL = {"f32": 1e-4, "bf16": 3e-3}   # per-row max|out - ref| / max|ref|


def require_gpu():
    import pytest
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    return torch


def to_device(x: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)  # exact: the values are already bf16-representable
    return t.cuda().contiguous()


def run_gpu(q, k, v, dtype, h, lam, path="auto"):
    import torch
    from local_linear_attention_amd import lla_forward, lla_forward_ex
    tq, tk, tv = (to_device(x, dtype) for x in (q, k, v))
    if path == "default":
        out = lla_forward(tq, tk, tv, h, lam)
    else:
        out = lla_forward_ex(tq, tk, tv, h, lam, path=path)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def oracle_workers() -> int:
    import os
    return max(1, min(16, os.cpu_count() or 1))


def oracle_all_rows(q, k, v, h, lam):
    """The fp64 oracle over every row, in a process pool of one BLAS thread per worker (the
    workers are forked from this process and inherit the limit): a full-size forward of the
    d = 64 workloads takes about a minute on 8 to 16 cores."""
    from threadpoolctl import threadpool_limits

    from oracle import lla_forward as oracle_forward
    with threadpool_limits(1, user_api="blas"):
        return oracle_forward(q, k, v, h, lam, workers=oracle_workers())


def oracle_some_rows(q, k, v, h, lam, rows):
    from threadpoolctl import threadpool_limits

    from oracle import lla_rows
    with threadpool_limits(1, user_api="blas"):
        return lla_rows(q, k, v, h, lam, rows, workers=oracle_workers())


def row_errors(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-row normwise relative error over the last axis."""
    num = np.max(np.abs(got - ref), axis=-1)
    den = np.maximum(np.max(np.abs(ref), axis=-1), 1e-30)
    return num / den


def sample_rows(B, H, n, d, seed, per_head=6):
    """Seeded sample: the hardest rows (i < 2d, around d) of every head, the last row of
    every head, and random rows."""
    rng = np.random.default_rng(1000 + seed)
    fixed = sorted({i for i in (0, 1, 2, 3, d // 2, d - 1, d, d + 1, 2 * d, n - 1) if 0 <= i < n})
    rows = []
    for b in range(B):
        for hh in range(H):
            pick = set(fixed[:: max(1, len(fixed) // 4)]) | {n - 1}
            pick |= set(int(x) for x in rng.integers(0, n, per_head))
            pick |= set(int(x) for x in rng.integers(0, min(n, 2 * d + 2), 2))
            rows += [(b, hh, i) for i in sorted(pick)]
    return rows


def workload_arrays(name, **shape):
    w = lla_inputs.WORKLOADS[name]
    if shape:
        w = w.with_shape(**shape)
    q, k, v, _ = lla_inputs.generate(w)
    return w, q, k, v


ENVELOPE_CASES = ("sharp_h", "q_x3", "rank16_keys", "v_2^-16", "v_2^17", "k_offset", "k_x64_h_x64",
                  "k_x1024_h_x1024")


def envelope_case(name, case):
    """Inputs outside the RMS-normalised, h = sqrt(d) regime of the pages' workloads, built
    from workload `name` at a small shape (every value bf16-representable):
    sharp_h: h / 2 (sharper weights); q_x3: queries x 3 (the same, through q); rank16_keys:
    keys confined to a random 16-dimensional subspace, re-normalised; v_2^-16, v_2^17:
    values scaled out of fp16's normal range either way; k_offset: keys + 4 (a common
    offset); k_x64_h_x64, k_x1024_h_x1024: keys x 64 (x 1024) with h scaled alike (the same
    weights, large keys: the ridge shrinks against the key moments)."""
    import lla_inputs
    shape = dict(B=1, H=2, n=700) if lla_inputs.WORKLOADS[name].d == 128 else dict(B=1, H=2, n=600)
    w, q, k, v = workload_arrays(name, **shape)
    r = lla_inputs.round_to_bf16
    h, lam = w.h, w.lam
    if case == "sharp_h":
        h = w.h / 2
    elif case == "q_x3":
        q = r(q * 3.0)
    elif case == "rank16_keys":
        rng = np.random.default_rng(16)
        basis = np.linalg.qr(rng.standard_normal((w.d, 16)))[0]
        kk = k @ basis @ basis.T
        k = r(kk / np.sqrt(np.mean(kk ** 2, axis=-1, keepdims=True)))
    elif case == "v_2^-16":
        v = r(v * 2.0 ** -16)
    elif case == "v_2^17":
        v = r(v * 2.0 ** 17)
    elif case == "k_offset":
        k = r(k + 4.0)
    elif case == "k_x64_h_x64":
        k, h = r(k * 64.0), w.h * 64.0
    elif case == "k_x1024_h_x1024":
        k, h = r(k * 1024.0), w.h * 1024.0
    else:
        raise KeyError(case)
    return w, q, k, v, h, lam


def fast_workspace_bytes(BH, n, d=64):
    """Scratch bytes of the bf16 matrix-core path, region by region (each rounded up to
    256 B where the library rounds it).

    d = 64: row maxima of rows >= 3d, anchor partial sums, anchors, then per head and 64-key
    tile the fp16 K/V image (72-half rows), the two key-major key images (bf16, centred
    fp16) and the 5 KiB check image, then per row >= 3d the fp16 hi/lo solution, eight
    scalars and 32 check targets, the guard words (count of rows handed back, two maxima per
    head) and the hand-back list (one slot per row >= 3d).

    d = 128: the same regions for rows >= 4d, with the K and V feature-major images apart
    (72-half rows) and key-major rows of 136 halves."""
    up = lambda x: (x + 255) // 256 * 256
    tiles = -(-n // 64)
    if d == 128:
        prows = n - min(n, 4 * d)
        if prows <= 0:
            return 0
        return (up(BH * prows * 4) + up(BH * 16 * 2 * d * 4) + up(BH * 2 * d * 4)
                + BH * tiles * (2 * d * 72 * 2 + 2 * 64 * 136 * 2 + 5 * 1024)
                + up(BH * prows * 2 * d * 2) + up(BH * prows * 8 * 4) + up(BH * prows * 32 * 4)
                + up((1 + 2 * BH) * 4) + up(BH * prows * 4))
    prows = n - min(n, 3 * d)
    if prows <= 0:
        return 0
    return (up(BH * prows * 4) + up(BH * 16 * 2 * d * 4) + up(BH * 2 * d * 4)
            + BH * tiles * (2 * d * 72 * 2 + 2 * 64 * 72 * 2 + 5 * 1024)
            + up(BH * prows * 2 * d * 2) + up(BH * prows * 8 * 4) + up(BH * prows * 32 * 4)
            + up((1 + 2 * BH) * 4) + up(BH * prows * 4))
