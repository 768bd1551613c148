"""Throughput of the causal LLA forward (or the Parallax forward with a given probe, or one of
the two decode steps) on one MI355X.

One step is one lla_forward call (lla_parallax_forward with --method parallax; one decode
call, one query per head against its whole cache, with --method parallax_decode or
lla_decode) over the whole workload with the inputs already resident in HBM.  Prints one
JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload d24] [--path auto]
                    [--method lla|parallax|parallax_bwd|parallax_decode|lla_decode]

The default workload is B=2, H=16, n=4096, d=64 with bf16 inputs (head shape of a
1024-wide, 16-head model), h = 8, lambda = 1e-2; with --method parallax the same q, k, v
plus an RMS-normalised probe (workload parallax_d24); --method parallax_bwd times the Parallax
backward (gradients of q, k, v, rho for a seeded output cotangent) on that workload, with the
forward's log-sum-exp computed once beforehand.  The decode methods default to eight
sequences of 16 heads with 8192 cached bf16 keys and values each.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LLA fwd queries/s + TFLOP/s (% MFMA peak) at B2 H16 n4096 d64 bf16, 1 GPU"
METRIC_PARALLAX = "Parallax fwd (given probe) queries/s + TFLOP/s (% MFMA peak) at B2 H16 n4096 d64 bf16, 1 GPU"

# MI355X published peaks.
PEAK = {
    "hbm_GBps": 8000.0,
    "mfma_f16_TFLOPs": 2516.6,   # dense fp16/bf16 matrix
    "valu_f64_TFLOPs": 78.6,     # fp64 vector
    "valu_f32_TFLOPs": 157.3,    # fp32 vector
    "mfma_f32_TFLOPs": 157.3,    # dense fp32 matrix
    "mfma_f64_TFLOPs": 78.6,     # dense fp64 matrix
}


def alg_flops(B, H, n, d, form):
    """Algorithmic flops of one forward: causal pairs only, the upper triangle of the key
    covariance, no recomputation.  form "NS": explicit value-key cross moment (the
    formulation the fp64 path executes); form "min": cross moment applied through a probe
    pass."""
    P = B * H * n * (n + 1) // 2
    N = B * H * n
    common = 2 * d + 2 * (1 + 2 * d) + d * (d + 1)
    if form == "NS":
        return P * (common + 2 * d * d) + N * (d ** 3 / 3 + 2 * d * d + 2 * d * d + 2 * d)
    return P * (common + 4 * d + 2) + N * (d ** 3 / 3 + 2 * d * d + 4 * d)


# Arithmetic of each path (the dtype field) and the bound of each kernel.
PATH_ARITH = {"exact": "f64", "fast": "f16 MFMA / f32 accumulate (rows < 3d and rows the check hands back: f64)",
              "cg": "f64 (conjugate gradient over the prefix)"}
KERNEL_BOUND = {
    "lla_exact_kernel": ("alu", PEAK["valu_f64_TFLOPs"]),
    "lla_exact_list_kernel": ("alu", PEAK["valu_f64_TFLOPs"]),
    "lla_refine_kernel": ("alu", PEAK["valu_f64_TFLOPs"]),
    "lla_cg_kernel": ("alu", PEAK["valu_f64_TFLOPs"]),
    "lla_short_kernel": ("alu", PEAK["valu_f64_TFLOPs"]),
    "lla8_short_kernel": ("mfma", PEAK["mfma_f64_TFLOPs"]),
    "lla_rowmax_kernel": ("mfma", PEAK["mfma_f16_TFLOPs"]),
    "lla_anchor_kernel": ("hbm", PEAK["hbm_GBps"]),
    "lla_pack_kernel": ("hbm", PEAK["hbm_GBps"]),
    "lla_moments_kernel": ("mfma", PEAK["mfma_f16_TFLOPs"]),
    "lla_keymom_kernel": ("mfma", PEAK["mfma_f16_TFLOPs"]),
    "lla_rows_kernel": ("mfma", PEAK["mfma_f16_TFLOPs"]),
    "lla_probe_kernel": ("mfma", PEAK["mfma_f16_TFLOPs"]),
    "lla_parallax_pack_kernel": ("hbm", PEAK["hbm_GBps"]),
    "lla_parallax_kernel": ("mfma", PEAK["mfma_f16_TFLOPs"]),
    "lla_parallax_exact_kernel": ("alu", PEAK["valu_f64_TFLOPs"]),
    "lla_parallax_fallback_kernel": ("alu", PEAK["valu_f64_TFLOPs"]),
    "lla_parallax_decode_kernel": ("hbm", PEAK["hbm_GBps"]),
    "lla_parallax_merge_kernel": ("hbm", PEAK["hbm_GBps"]),
    "lla_parallax_bwd_pack_kernel": ("hbm", PEAK["hbm_GBps"]),
    "lla_parallax_bwd_stats_kernel": ("mfma", PEAK["mfma_f16_TFLOPs"]),
    "lla_parallax_bwd_kv_kernel": ("mfma", PEAK["mfma_f16_TFLOPs"]),
    "lla_parallax_bwd_qr_kernel": ("mfma", PEAK["mfma_f16_TFLOPs"]),
    "lla_parallax_bwd_exact_rows_kernel": ("alu", PEAK["valu_f64_TFLOPs"]),
    "lla_parallax_bwd_exact_cols_kernel": ("alu", PEAK["valu_f64_TFLOPs"]),
    "lla_decode_stats_kernel": ("hbm", PEAK["hbm_GBps"]),
    "lla_decode_moments_kernel": ("mfma", PEAK["mfma_f64_TFLOPs"]),   # hbm when split (see below)
    "lla_decode_reduce_kernel": ("hbm", PEAK["hbm_GBps"]),
    "lla_decode_solve_kernel": ("alu", PEAK["valu_f64_TFLOPs"]),
    "lla8_anchor_kernel": ("hbm", PEAK["hbm_GBps"]),
    "lla8_pack_kernel": ("hbm", PEAK["hbm_GBps"]),
    "lla8_rowmax_kernel": ("mfma", PEAK["mfma_f16_TFLOPs"]),
    "lla8_keymom_kernel": ("mfma", PEAK["mfma_f16_TFLOPs"]),
    "lla8_probe_kernel": ("mfma", PEAK["mfma_f16_TFLOPs"]),
}
PATH_KERNELS = {
    "exact": ["lla_exact_kernel"],
    "cg": ["lla_cg_kernel", "lla_exact_list_kernel"],   # the list: rows CG leaves unconverged
    # the last launch recomputes in fp64 the rows the range guard and the checks hand back
    "fast": ["lla_anchor_kernel", "lla_pack_kernel", "lla_rowmax_kernel", "lla_rows_kernel",
             "lla_probe_kernel", "lla_refine_kernel"],
    # d = 128: rows i < 4d on the fp64 short-row kernel, the rest on the d = 128 matrix-core
    # kernels
    "fast128": ["lla8_short_kernel", "lla8_anchor_kernel", "lla8_pack_kernel", "lla8_rowmax_kernel",
                "lla8_keymom_kernel", "lla8_probe_kernel", "lla_exact_list_kernel"],
}


def path_kernels(path, d):
    return PATH_KERNELS["fast128" if (path == "fast" and d == 128) else path]
PARALLAX_KERNELS = {
    "exact": ["lla_parallax_exact_kernel"],
    "fast": ["lla_parallax_pack_kernel", "lla_parallax_kernel", "lla_parallax_fallback_kernel"],
}


def parallax_flops(B, H, n, d):
    """Algorithmic flops of one Parallax forward (given probe): per causal pair the score
    (2d), the probe score (2d), the covariance-branch weight P1 s2 (1), the two weight sums
    (2) and the two weighted value sums (4d); per query the merge (4d)."""
    P = B * H * n * (n + 1) // 2
    return P * (8 * d + 3) + B * H * n * 4 * d


def pair_count(BH, lo, hi):
    """Causal pairs (i, j <= i) of rows lo <= i < hi, over BH heads."""
    return BH * (hi * (hi + 1) // 2 - lo * (lo + 1) // 2)


def kernel_flops(name, B, H, n, d, path):
    """Algorithmic flops of one launch of a kernel, in the formulation that kernel executes.
    The exact and CG paths form the value-key cross moment (NS); the fast path applies it
    through a pass over the values (min), its fp64 short rows included.  Fast path, d = 64:
    rows [0, 3d) on the fp64 short-row blocks of the rows kernel; the row-max kernel owns the
    score term of rows >= 3d; rows [3d, n) the key-moment blocks (first moments, C_kk, solve)
    and the probe kernel (probe scores and the weighted value sum); d = 128 the same with 4d
    for 3d and its own short-row kernel.  Scores a kernel recomputes, and the probe's check
    sums (a verification, not part of the estimator), are not counted."""
    BH = B * H
    # fp64 short rows: i < 3d at d = 64 (short-row blocks), i < 4d at d = 128 (short-row
    # kernel); the rest key moments + probe
    row0 = rowp = (min(n, 4 * d) if d == 128 else min(n, 3 * d)) if path == "fast" else n
    per_query = d ** 3 / 3 + 4 * d * d + 2 * d
    moments = 2 * (1 + 2 * d) + d * (d + 1)
    if name in ("lla_exact_kernel", "lla_cg_kernel"):
        # the CG kernel is credited with the direct formulation's count, so that both fp64
        # paths report comparable rates (its own work depends on the iteration counts)
        return pair_count(BH, 0, row0) * (2 * d + moments + 2 * d * d) + BH * row0 * per_query
    if name in ("lla_short_kernel", "lla8_short_kernel"):
        # fp64 short rows in the probe form: per pair the score, first moments, C_kk, then
        # u_j (2d) and the weighted value sums (2d + 2); per query the solve
        return pair_count(BH, 0, row0) * (2 * d + moments + 4 * d + 2) + BH * row0 * (d ** 3 / 3 + 2 * d * d)
    if name in ("lla_anchor_kernel", "lla_pack_kernel", "lla8_anchor_kernel", "lla8_pack_kernel"):
        return 0                      # data movement only (K, V summed and repacked once)
    if name in ("lla_exact_list_kernel", "lla_refine_kernel"):
        return 0                      # rows handed back by the fast path's checks (counted in fallback_rows)
    if name in ("lla_rowmax_kernel", "lla8_rowmax_kernel"):
        return pair_count(BH, row0, n) * 2 * d
    if name == "lla8_keymom_kernel":
        return pair_count(BH, rowp, n) * moments + BH * (n - rowp) * (d ** 3 / 3 + 2 * d * d)
    if name == "lla8_probe_kernel":
        return pair_count(BH, rowp, n) * (4 * d + 2) + BH * (n - rowp) * 4 * d
    if name == "lla_moments_kernel":
        return pair_count(BH, row0, rowp) * (moments + 2 * d * d) + BH * (rowp - row0) * per_query
    if name == "lla_keymom_kernel":
        return pair_count(BH, rowp, n) * moments + BH * (n - rowp) * (d ** 3 / 3 + 2 * d * d)
    if name == "lla_rows_kernel":     # one launch: short rows, key moments of rows >= 2d
        return sum(kernel_flops(part, B, H, n, d, path)
                   for part in ("lla_short_kernel", "lla_keymom_kernel"))
    if name == "lla_probe_kernel":
        return pair_count(BH, rowp, n) * (4 * d + 2) + BH * (n - rowp) * 4 * d
    if name in ("lla_parallax_kernel", "lla_parallax_exact_kernel"):
        return parallax_flops(B, H, n, d)
    if name == "lla_parallax_pack_kernel":
        return 0                      # data movement only (K, V repacked once)
    if name == "lla_parallax_fallback_kernel":
        return 0                      # heads the range guard hands to fp64 (none on the synthetic workloads)
    raise KeyError(name)


def path_flops(B, H, n, d, path):
    """Algorithmic flops of one forward in the formulations the path executes."""
    return sum(kernel_flops(k, B, H, n, d, path) for k in path_kernels(path, d))


def kernel_source_hash(kernel):
    """Hash of the HIP source file that defines `kernel` plus the shared headers: a traffic
    record taken on other sources of that kernel is stale."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "local_linear_attention_amd", "csrc")
    names = sorted(os.listdir(csrc))
    for name in names:
        path = os.path.join(csrc, name)
        if name.endswith(".h") or (name.endswith(".hip") and (f"void {kernel}(" in open(path).read()
                                                             or f'"{kernel}"' in open(path).read())):
            h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload):
    """HBM bytes per launch (fetched + written) from the committed rocprofv3 counter summary
    profiles/<kernel>_<workload>_traffic.json, if it was taken on the current kernel
    sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


def blas_threads():
    """Threads of the BLAS library numpy calls in this process (the oracle's workers are
    forked from it and inherit the setting)."""
    try:
        from threadpoolctl import threadpool_info
        return max([int(x.get("num_threads", 1)) for x in threadpool_info() if x.get("user_api") == "blas"] or [1])
    except Exception:
        return None


def stratified_rows(w, rng, uniform):
    """The long-context sample: every row i < 2d of head 0, `uniform` rows drawn uniformly over
    all heads, and the last row of every head."""
    rows = {(0, 0, i) for i in range(min(w.n, 2 * w.d))}
    rows |= {(w.B - 1 - b, hh, w.n - 1) for b in range(w.B) for hh in range(w.H)}
    rows |= {(int(rng.integers(w.B)), int(rng.integers(w.H)), int(rng.integers(w.n))) for _ in range(uniform)}
    return sorted(rows)


def cpu_baseline(w, q, k, v, seconds, rho=None):
    """The fp64 oracle (LLA, or Parallax when a probe is given) in a process pool with one BLAS
    thread per worker.  A timing sample of uniformly drawn rows comes first; when it projects
    the whole workload within twice the budget, every row of the workload is then run once and
    the measured time reported.  Otherwise the full-workload time is projected from the
    sample with per-row cost i+1 (a row's prefix length).  Long sequences (n > 8192) take a
    stratified sample: every row i < 2d of head 0, uniform rows over all heads and the last
    row of every head."""
    import numpy as np

    from oracle import default_workers, lla_rows, parallax_rows
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:   # pragma: no cover
        threadpool_limits = None
    workers = default_workers()
    rng = np.random.default_rng(12345)
    total_cost = w.B * w.H * w.n * (w.n + 1) / 2
    done_rows, done_cost, elapsed = 0, 0.0, 0.0

    def run(rows):
        if rho is None:
            lla_rows(q, k, v, w.h, w.lam, rows, workers=workers)
        else:
            parallax_rows(q, k, v, rho, w.h, rows, workers=workers)

    limit = threadpool_limits(1, user_api="blas") if threadpool_limits else None
    full = False
    try:
        bt = blas_threads()
        stratified = w.n > 8192
        batch = 8 * workers
        while elapsed < seconds:
            if done_rows and not stratified and elapsed >= min(2.0, seconds / 4):
                # When the sample projects the whole workload to fit twice the budget, run
                # every row once instead and report the measured time.
                if elapsed * total_cost / done_cost <= 2 * seconds:
                    every = [(b, hh, i) for b in range(w.B) for hh in range(w.H) for i in range(w.n)]
                    t0 = time.perf_counter()
                    run(every)
                    elapsed, done_rows, done_cost, full = time.perf_counter() - t0, len(every), total_cost, True
                    break
            if stratified and done_rows == 0:
                rows = stratified_rows(w, rng, 2048)
            else:
                rows = [(int(rng.integers(w.B)), int(rng.integers(w.H)), int(rng.integers(w.n)))
                        for _ in range(batch)]
                batch = min(4 * batch, 512 * workers)
            t0 = time.perf_counter()
            run(rows)
            elapsed += time.perf_counter() - t0
            done_rows += len(rows)
            done_cost += sum(i + 1 for (_, _, i) in rows)
    finally:
        if limit is not None:
            limit.restore_original_limits()
    full_seconds = elapsed * total_cost / done_cost
    kind = ("a stratified sample (every row i < 2d of head 0, 2048 uniform rows, the last row of every "
            "head), then uniform rows" if stratified else "uniformly drawn rows")
    if full:
        sample = (f"the whole workload, every one of its {done_rows} rows once (after a timing sample "
                  f"projected it within budget): {elapsed:.1f} s measured in {workers} worker processes "
                  f"with {bt} BLAS thread(s) each on a host with {os.cpu_count()} CPUs; no projection")
    else:
        sample = (f"{done_rows} rows of the same workload, {kind} (seed 12345): {elapsed:.1f} s in "
                  f"{workers} worker processes with {bt} BLAS thread(s) each on a host with "
                  f"{os.cpu_count()} CPUs; the full-workload time, {full_seconds:.0f} s, is a projection "
                  f"from the sample with per-row cost i+1, not a full run")
    return {
        "value": w.queries / full_seconds,
        "unit": "queries/s",
        "cores": workers * (bt or 1),
        "kind": "oracle",
        "host_cpus": os.cpu_count(),
        "workers": workers,
        "blas_threads_per_worker": bt,
        "full_workload": full,
        "sample": sample,
    }


METRIC_DECODE = "Parallax decode (given probe) queries/s and HBM GB/s at B8 H16 L8192 d64 bf16, 1 GPU"
METRIC_LLA_DECODE = "LLA decode queries/s and HBM GB/s at B8 H16 L8192 d64 bf16, 1 GPU"


def decode_bytes(B, H, L, d, elt, nvec=2):
    """Algorithmic HBM bytes of one decode step: the cache (K and V) read once, the nvec
    per-head input vectors (q, and rho for Parallax) read, the fp32 output written."""
    return 2 * B * H * L * d * elt + nvec * B * H * d * elt + B * H * d * 4


def lla_moment_flops(B, H, L, d):
    """Algorithmic flops of the LLA decode moments: per cached key the upper triangle of the
    weighted key covariance (d(d+1)/2 products and adds), the value-key cross moment (d^2)
    and the weighted value sum (d)."""
    return B * H * L * (d * (d + 1) + 2 * d * d + 2 * d)


def lla_solve_flops(B, H, d):
    """Per head: LDL^T factorisation (d^3/3), two triangular solves and the value
    correction (2 d^2 each)."""
    return B * H * (d ** 3 / 3 + 2 * d * d + 2 * d * d)


def lla_decode_chunks(BH, L):
    """Chunks per head of the LLA decode launches (the library's split: about 1024 blocks,
    512 to 2048 keys per chunk)."""
    s = min(-(-1024 // BH), -(-L // 512))
    s = max(s, -(-L // 2048), 1)
    c = -(-L // s)
    return -(-L // c)


def lla_decode_split_operands(w):
    """Whether the LLA decode moments run from split bf16 operands (bf16 inputs, caches
    of at least 2d positions): HBM-bound then (the executed matrix-core work takes less time
    at peak than the K, V read); otherwise fp64 matrix cores."""
    return w.dtype == "bf16" and w.L >= 2 * w.d


def decode_kernel_units(name, w, elt):
    """(algorithmic amount, unit) of one launch of each decode kernel at workload w."""
    B, H, L, d = w.B, w.H, w.L, w.d
    if name == "lla_parallax_decode_kernel":
        # moves every byte of the step but the merge's partial sums
        return decode_bytes(B, H, L, d, elt), "B"
    if name == "lla_decode_stats_kernel":
        # reads the keys and the query
        return B * H * L * d * elt + B * H * d * elt, "B"
    if name == "lla_decode_moments_kernel":
        if lla_decode_split_operands(w):
            # reads K and V once and the stats pass's scores
            return 2 * B * H * L * d * elt + B * H * L * 4, "B"
        return lla_moment_flops(B, H, L, d), "flop"
    if name == "lla_decode_reduce_kernel":
        # reads every chunk's moments, writes the heads' fp64 sums
        nb = d // 16
        e = (nb * (nb + 1) // 2 + nb * nb) * 256 + d
        S = lla_decode_chunks(B * H, L)
        ta = 8 if (w.dtype == "f32" or L < 2 * d) else 4
        return B * H * S * e * ta + B * H * e * 8, "B"
    if name == "lla_decode_solve_kernel":
        return lla_solve_flops(B, H, d), "flop"
    return None, None


def decode_cpu_baseline(w, q, k, v, rho, seconds):
    """The fp64 decode oracle (Parallax when a probe is given, else LLA) on whole heads drawn
    at random, projected to the workload."""
    import numpy as np

    from oracle import lla_decode, parallax_decode
    rng = np.random.default_rng(12345)
    done, elapsed = 0, 0.0
    while elapsed < seconds and done < w.B * w.H:
        b, hh = int(rng.integers(w.B)), int(rng.integers(w.H))
        sl = (slice(b, b + 1), slice(hh, hh + 1))
        t0 = time.perf_counter()
        if rho is None:
            lla_decode(q[sl], k[sl], v[sl], w.h, w.lam)
        else:
            parallax_decode(q[sl], k[sl], v[sl], rho[sl], w.h)
        elapsed += time.perf_counter() - t0
        done += 1
    full = elapsed * w.B * w.H / done
    return {"value": w.queries / full, "unit": "queries/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} (batch, head) caches drawn at random (seed 12345), {elapsed:.1f} s in one "
                      f"process; full-step time {full:.1f} s projected per head"}


def bench_decode(args):
    import numpy as np
    import torch

    import lla_inputs
    from local_linear_attention_amd import lla_decode, lla_parallax_decode, lla_profile_collect, lla_profile_enable

    parallax = args.method == "parallax_decode"
    w = lla_inputs.DECODE_WORKLOADS[args.workload or ("decode_b8_l8192" if parallax else "lla_decode_b8_l8192")]
    q, k, v, rho = lla_inputs.generate_decode(w)
    if not parallax:
        rho = None
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    tq, tk, tv = (torch.from_numpy(x).to(tdt).to(dev).contiguous() for x in (q, k, v))
    tr = torch.from_numpy(rho).to(tdt).to(dev).contiguous() if parallax else None
    out = torch.empty(tq.shape, dtype=torch.float32, device=dev)
    if args.copy_calibration_mib > 0:
        src = torch.ones((args.copy_calibration_mib << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    stream = torch.cuda.current_stream(dev)

    def step():
        if parallax:
            lla_parallax_decode(tq, tk, tv, tr, w.h, out=out, stream=stream)
        else:
            lla_decode(tq, tk, tv, w.h, w.lam, out=out, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for s_ in range(args.steps):
        starts[s_].record(stream)
        step()
        ends[s_].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    per_ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    assert torch.isfinite(out).all().item(), "non-finite output"

    lla_profile_enable(True)
    lla_profile_collect()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    rec = lla_profile_collect()
    lla_profile_enable(False)
    per_kernel = {}
    for name, ms in rec:
        per_kernel.setdefault(name, []).append(ms)
    elt = 4 if w.dtype == "f32" else 2
    nbytes = decode_bytes(w.B, w.H, w.L, w.d, elt, nvec=2 if parallax else 1)
    kernels = {}
    for name, lst in per_kernel.items():
        avg = statistics.mean(lst)
        amount, unit = decode_kernel_units(name, w, elt)
        bound, peak = KERNEL_BOUND[name]
        if name == "lla_decode_moments_kernel" and unit == "B":
            bound, peak = "hbm", PEAK["hbm_GBps"]
        ent = {"launches": len(lst), "avg_ms": avg, "bound": bound, "peak": peak}
        if unit == "B":
            ent.update(bytes=amount, GBps=amount / (avg * 1e-3) / 1e9)
        elif unit == "flop":
            ent.update(flops=amount, tflops=amount / (avg * 1e-3) / 1e12)
        kernels[name] = ent
    dom = max(kernels, key=lambda nm: kernels[nm]["avg_ms"] * kernels[nm]["launches"])
    dk = kernels[dom]
    if "GBps" in dk:
        achieved, unit = dk["GBps"], "GB/s"
    else:
        achieved, unit = dk["tflops"], "TFLOP/s"
    traffic = load_traffic(dom, w.name)
    if parallax:
        config_text = f"{w.name}: B{w.B} H{w.H} L{w.L} d{w.d} {w.dtype} cache, one query and probe per head, h={w.h:g}"
    else:
        config_text = f"{w.name}: B{w.B} H{w.H} L{w.L} d{w.d} {w.dtype} cache, one query per head, h={w.h:g}, " \
                      f"lambda={w.lam:g}"
    if parallax:
        arith = "f32 (bf16 inputs)" if w.dtype == "bf16" else "f32"
    else:
        arith = ("f32 scores, f64 moments and solve" if w.dtype == "f32" or w.L < 2 * w.d
                 else "f32 scores and matrix-core moments, f64 solve")
    result = {
        "metric": METRIC_DECODE if parallax else METRIC_LLA_DECODE,
        "value": w.queries / (ms_per_step * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": arith,
        "data": "synthetic",
        "config": {"workload": config_text,
                   "B": w.B, "H": w.H, "L": w.L, "d": w.d, "input_dtype": w.dtype, "queries": w.queries},
        "hbm_GBps": nbytes / (ms_per_step * 1e-3) / 1e9,
        "kernels": kernels,
        "timing_ms": {"median": statistics.median(per_ms), "p10": float(np.percentile(per_ms, 10)),
                      "p90": float(np.percentile(per_ms, 90))},
        "roofline": {"kernel": dom, "bound": dk["bound"], "achieved": achieved,
                     "peak": dk["peak"], "unit": unit, "frac": achieved / dk["peak"],
                     "traffic": traffic},
        "gfx": torch.cuda.get_device_properties(dev).gcnArchName,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = decode_cpu_baseline(w, q, k, v, rho, min(args.cpu_seconds, 10.0))
    print(json.dumps(result), flush=True)


METRIC_PARALLAX_BWD = ("Parallax bwd (given probe) queries/s + TFLOP/s (% MFMA peak) at B2 H16 n4096 d64 bf16, "
                       "1 GPU")


def parallax_bwd_flops(B, H, n, d):
    """Algorithmic flops of one Parallax backward: per causal pair the three products of the
    pair (score q.k, probe score rho.k, g = dout.v: 2d each) and the five weighted sums that
    use them (dv, the two terms of dk, dq, drho: 2d each) -- 16d -- plus about 16 flops of
    pair weights; per row the statistics (4d).  Scores the kernels recompute are not counted
    again, nor the second (lo) half of the split weights."""
    P = B * H * n * (n + 1) // 2
    return P * (16 * d + 16) + B * H * n * 4 * d


def parallax_bwd_kernel_flops(name, B, H, n, d):
    """Algorithmic flops of one launch of each backward kernel (its own products; the split
    weights' second halves not counted)."""
    P = B * H * n * (n + 1) // 2
    if name == "lla_parallax_bwd_stats_kernel":
        return P * (6 * d + 8)       # the three products and the four row sums
    if name == "lla_parallax_bwd_kv_kernel":
        return P * (12 * d + 12)     # the three products, a, ds, du; dv and dk
    if name == "lla_parallax_bwd_qr_kernel":
        return P * (10 * d + 10)     # the three products, ds, du; dq and drho
    if name in ("lla_parallax_bwd_exact_rows_kernel", "lla_parallax_bwd_exact_cols_kernel"):
        return parallax_bwd_flops(B, H, n, d) // 2
    return 0                         # packing: data movement only


def bench_parallax_bwd(args):
    import numpy as np
    import torch

    import lla_inputs
    from local_linear_attention_amd import (lla_parallax_backward, lla_parallax_backward_workspace_size,
                                            lla_parallax_forward_stats, lla_profile_collect, lla_profile_enable)

    w = lla_inputs.WORKLOADS[args.workload or "parallax_d24"]
    q, k, v, _ = lla_inputs.generate(w)
    rho, _ = lla_inputs.generate_probe(w)
    dout, _ = lla_inputs.generate_cotangent(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    tq, tk, tv, tr, tdo = (torch.from_numpy(x).to(tdt).to(dev).contiguous() for x in (q, k, v, rho, dout))
    path = args.path
    if path == "auto":
        path = "fast" if w.dtype == "bf16" and w.d == 64 else "exact"
    _, lse = lla_parallax_forward_stats(tq, tk, tv, tr, w.h, path=path)
    grads = tuple(torch.empty(tq.shape, dtype=torch.float32, device=dev) for _ in range(4))
    ws = torch.empty(max(1, lla_parallax_backward_workspace_size(w.B, w.H, w.n, w.d, w.dtype, path)),
                     dtype=torch.uint8, device=dev)
    if args.copy_calibration_mib > 0:
        src = torch.ones((args.copy_calibration_mib << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    stream = torch.cuda.current_stream(dev)

    def step():
        lla_parallax_backward(tq, tk, tv, tr, tdo, lse, w.h, path=path, grads=grads, stream=stream, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for s_ in range(args.steps):
        starts[s_].record(stream)
        step()
        ends[s_].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    per_ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    assert all(torch.isfinite(g).all().item() for g in grads), "non-finite gradient"

    lla_profile_enable(True)
    lla_profile_collect()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    rec = lla_profile_collect()
    lla_profile_enable(False)
    per_kernel = {}
    for name, ms in rec:
        per_kernel.setdefault(name, []).append(ms)
    kernels = {}
    for name, lst in per_kernel.items():
        fl = parallax_bwd_kernel_flops(name, w.B, w.H, w.n, w.d)
        avg = statistics.mean(lst)
        bound, peak = KERNEL_BOUND[name]
        kernels[name] = {"launches": len(lst), "avg_ms": avg, "flops": fl, "tflops": fl / (avg * 1e-3) / 1e12,
                         "bound": bound, "peak": peak}
    dom = max(kernels, key=lambda nm: kernels[nm]["avg_ms"] * kernels[nm]["launches"])
    dk = kernels[dom]
    flops = parallax_bwd_flops(w.B, w.H, w.n, w.d)
    result = {
        "metric": METRIC_PARALLAX_BWD,
        "value": w.queries / (ms_per_step * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fast": "bf16 products, bf16 hi+lo pair weights, f32 accumulate", "exact": "f64"}[path],
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B{w.B} H{w.H} n{w.n} d{w.d} {w.dtype} inputs, probe and output "
                               f"cotangent, h={w.h:g}; gradients of q, k, v, rho",
                   "B": w.B, "H": w.H, "n": w.n, "d": w.d, "input_dtype": w.dtype, "path": path,
                   "queries": w.queries},
        "tflops": flops / (ms_per_step * 1e-3) / 1e12,
        "flop_count": {"formulation": "per pair 16d + 16 (three products, five weighted sums, pair weights), "
                                      "per row 4d", "flops": flops},
        "kernels": kernels,
        "timing_ms": {"median": statistics.median(per_ms), "p10": float(np.percentile(per_ms, 10)),
                      "p90": float(np.percentile(per_ms, 90))},
        "roofline": {"kernel": dom, "bound": dk["bound"], "achieved": dk["tflops"], "peak": dk["peak"],
                     "unit": "TFLOP/s", "frac": dk["tflops"] / dk["peak"], "traffic": load_traffic(dom, w.name)},
        "mfma_peak_frac": flops / (ms_per_step * 1e-3) / 1e12 / PEAK["mfma_f16_TFLOPs"],
        "gfx": torch.cuda.get_device_properties(dev).gcnArchName,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = parallax_bwd_cpu_baseline(w, q, k, v, rho, dout, min(args.cpu_seconds, 20.0))
    print(json.dumps(result), flush=True)


def parallax_bwd_cpu_baseline(w, q, k, v, rho, dout, seconds):
    """The fp64 backward oracle on whole heads drawn at random, projected to the workload."""
    import numpy as np
    import torch

    from oracle import parallax_backward
    rng = np.random.default_rng(12345)
    done, elapsed = 0, 0.0
    while elapsed < seconds and done < w.B * w.H:
        b, hh = int(rng.integers(w.B)), int(rng.integers(w.H))
        sl = (slice(b, b + 1), slice(hh, hh + 1))
        t0 = time.perf_counter()
        parallax_backward(q[sl], k[sl], v[sl], rho[sl], w.h, dout[sl])
        elapsed += time.perf_counter() - t0
        done += 1
    full = elapsed * w.B * w.H / done
    return {"value": w.queries / full, "unit": "queries/s", "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": f"{done} (batch, head) pairs drawn at random (seed 12345), {elapsed:.1f} s in one process "
                      f"with {torch.get_num_threads()} BLAS threads; full-step time {full:.1f} s projected per head"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--method", default="lla", choices=["lla", "parallax", "parallax_bwd", "parallax_decode", "lla_decode"])
    ap.add_argument("--workload", default=None,
                    help="default: d24 (LLA), parallax_d24 (Parallax), decode_b8_l8192 (Parallax decode), "
                         "lla_decode_b8_l8192 (LLA decode)")
    ap.add_argument("--path", default="auto", choices=["auto", "exact", "fast", "cg"])
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run one device-to-device copy of this many MiB (a reference "
                         "dispatch of known traffic for hardware-counter runs)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the LLA forward here is built and measured on a "
              "single MI355X (heads shard across GPUs with no exchange; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.method in ("parallax_decode", "lla_decode"):
        bench_decode(args)
        return
    if args.method == "parallax_bwd":
        bench_parallax_bwd(args)
        return

    import numpy as np
    import torch

    import lla_inputs
    from local_linear_attention_amd import (lla_forward_ws, lla_parallax_forward_ws, lla_parallax_path_available,
                                            lla_parallax_workspace_size, lla_path_available, lla_profile_collect,
                                            lla_profile_enable, lla_workspace_size, load_library)

    parallax = args.method == "parallax"
    w = lla_inputs.WORKLOADS[args.workload or ("parallax_d24" if parallax else "d24")]
    q, k, v, _ = lla_inputs.generate(w)
    rho = lla_inputs.generate_probe(w)[0] if parallax else None
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    tq, tk, tv = (torch.from_numpy(x).to(tdt).to(dev).contiguous() for x in (q, k, v))
    tr = torch.from_numpy(rho).to(tdt).to(dev).contiguous() if parallax else None
    out = torch.empty(tq.shape, dtype=torch.float32, device=dev)
    load_library()

    if args.copy_calibration_mib > 0:
        nbytes = args.copy_calibration_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    path = args.path
    available = lla_parallax_path_available if parallax else lla_path_available
    if path == "auto":
        # the path the library picks by default for this dtype and head size
        path = "fast" if (w.dtype == "bf16" and available("fast", w.dtype, w.d)) else "exact"
    stream = torch.cuda.current_stream(dev)
    # The caller owns the scratch: one workspace allocated before the timed region and passed
    # to the _ws entry point, which allocates nothing.
    ws_size = (lla_parallax_workspace_size if parallax else lla_workspace_size)(w.B, w.H, w.n, w.d, w.dtype, path)
    ws = torch.empty(ws_size, dtype=torch.uint8, device=dev) if ws_size > 0 else None

    def step():
        if parallax:
            lla_parallax_forward_ws(tq, tk, tv, tr, w.h, ws, path=path, out=out, stream=stream)
        else:
            lla_forward_ws(tq, tk, tv, w.h, w.lam, ws, path=path, out=out, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_all0.record(stream)
    for s in range(args.steps):
        starts[s].record(stream)
        step()
        ends[s].record(stream)
    t_all1.record(stream)
    torch.cuda.synchronize()
    total_ms = t_all0.elapsed_time(t_all1)
    per_ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    ms_per_step = total_ms / args.steps
    assert torch.isfinite(out).all().item(), "non-finite output"
    # Rows of the last timed step that the matrix-core path's checks sent to the fp64 kernel.
    fallback_rows = None
    if not parallax and ws is not None:
        from local_linear_attention_amd.lla import lla_forward_fallback_rows
        fallback_rows = lla_forward_fallback_rows(ws, (w.B, w.H, w.n, w.d), w.dtype, path, stream=stream)

    # Kernel-level timing: the same steps again with the library's per-launch HIP events.
    lla_profile_enable(True)
    lla_profile_collect()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    rec = lla_profile_collect()
    lla_profile_enable(False)
    per_kernel = {}
    for name, ms in rec:
        per_kernel.setdefault(name, []).append(ms)
    kernels = {}
    for name, lst in per_kernel.items():
        fl = kernel_flops(name, w.B, w.H, w.n, w.d, path)
        avg = statistics.mean(lst)
        bound, peak = KERNEL_BOUND[name]
        kernels[name] = {"launches": len(lst), "avg_ms": avg, "flops": fl,
                         "tflops": fl / (avg * 1e-3) / 1e12, "bound": bound, "peak": peak}
    dom = max(kernels, key=lambda nm: kernels[nm]["avg_ms"] * kernels[nm]["launches"])
    dk = kernels[dom]
    flops = parallax_flops(w.B, w.H, w.n, w.d) if parallax else path_flops(w.B, w.H, w.n, w.d, path)
    achieved_tflops = flops / (ms_per_step * 1e-3) / 1e12
    traffic = load_traffic(dom, w.name)

    if parallax:
        config_text = f"{w.name}: B{w.B} H{w.H} n{w.n} d{w.d} {w.dtype} inputs and probe, h={w.h:g}"
        flop_count = {"formulation": "Parallax: per pair 8d + 3 (two scores, one weight product, "
                                     "two weight sums, two value sums), per query 4d",
                      "flops": flops}
        arith = {"exact": "f64", "fast": "bf16 scores / f16 weights and values, f32 accumulate"}[path]
    else:
        config_text = (f"{w.name}: B{w.B} H{w.H} n{w.n} d{w.d} {w.dtype} inputs, h={w.h:g}, "
                       f"lambda={w.lam:g}")
        split = "4d" if w.d == 128 else "3d"
        flop_count = {"formulation": (f"min (probe form) for every row; rows i < {split} in fp64"
                                      if path == "fast" else "NS"),
                      "flops": flops,
                      "F_NS": alg_flops(w.B, w.H, w.n, w.d, "NS"),
                      "F_min": alg_flops(w.B, w.H, w.n, w.d, "min")}
        arith = PATH_ARITH[path]
        if path == "fast" and w.d == 128:
            arith = "f16 MFMA / f32 accumulate (rows < 4d and rows the check hands back: f64)"
    result = {
        "metric": (METRIC_PARALLAX if parallax else METRIC) if w.name in ("d24", "parallax_d24") else
                  (f"{'Parallax fwd (given probe)' if parallax else 'LLA fwd'} queries/s + TFLOP/s (% MFMA peak) "
                   f"at B{w.B} H{w.H} n{w.n} d{w.d} {w.dtype}, 1 GPU"),
        "value": w.queries / (ms_per_step * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": arith,
        "data": "synthetic",
        "config": {
            "workload": config_text,
            "B": w.B, "H": w.H, "n": w.n, "d": w.d, "input_dtype": w.dtype,
            "h": w.h, "lambda": None if parallax else w.lam, "path": path, "queries": w.queries,
            "entry_point": (("lla_parallax_forward_ws" if parallax else "lla_forward_ws")
                            + f" with a caller workspace of {ws_size} bytes"),
        },
        "fallback_rows": fallback_rows,
        "tflops": achieved_tflops,
        "flop_count": flop_count,
        "kernels": kernels,
        "timing_ms": {"median": statistics.median(per_ms), "p10": float(np.percentile(per_ms, 10)),
                      "p90": float(np.percentile(per_ms, 90))},
        "roofline": {
            "kernel": dom,
            "bound": dk["bound"],
            "achieved": dk["tflops"],
            "peak": dk["peak"],
            "unit": "TFLOP/s",
            "frac": dk["tflops"] / dk["peak"],
            "traffic": traffic,
        },
        "mfma_peak_frac": achieved_tflops / PEAK["mfma_f16_TFLOPs"],
        "gfx": torch.cuda.get_device_properties(dev).gcnArchName,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_seconds, rho=rho)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
