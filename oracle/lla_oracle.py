"""Plain fp64 CPU oracle for the causal Local Linear Attention (LLA) forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP path.

What it computes (the plain definition, row by row, in fp64):

For query i of one (batch, head), LLA fits a local linear model b + W (x - q_i) to the
causal prefix {(k_j, v_j) : j <= i}, with kernel weights w_ij = exp(q_i . k_j / h) and a
ridge penalty lambda ||W||_F^2, and returns the intercept b_i.  Sources:
  * "Parallax" blog post (Tilde Research), section 2 "Canonical Formulation": the
    hypothesis class, the softmax-kernel weight, the ridge term and the moments
    z_ij = k_j - q_i, omega_i, mu_i, Sigma_i;
  * "Parallax: Parameterized Local Linear Attention for Language Modeling" (arXiv
    2605.29157, HTML), the LLA definition paragraph: LLA is the local linear
    estimator's prediction at q_i.
The display equation itself is missing from the extracted text; the reading used here is
the weighted ridge problem

    (b_i, W_i) = argmin  sum_{j<=i} w_ij || v_j - b - W z_ij ||^2 + lambda ||W||_F^2 .

Setting the gradient in b to zero gives b = vbar - W zbar; substituting into the
gradient in W gives W (C_kk + lambda I) = C_vk with the centred weighted moments below.
This is the centred (Sherman-Morrison) form of the blog's Appendix E "Boundary
amplification is non-negative", whose rank-one split of Sigma_i is
Sigma_i = (C_kk + lambda I) + omega_i zbar zbar^T.

Per row, with a per-row shift m_i (the safe-softmax maximum of the arXiv page's
scoring-form paragraph) and wt_ij = exp(s_ij - m_i):

    omega = sum wt,  kbar = sum wt k / omega,  vbar = sum wt v / omega,
    C_kk  = sum wt (k - kbar)(k - kbar)^T,  C_vk = sum wt (v - vbar)(k - kbar)^T,
    y     = (C_kk + lambda e^{-m_i} I)^{-1} (kbar - q_i),
    b_i   = vbar - C_vk y.

Multiplying every weight by e^{-m_i} multiplies every moment by e^{-m_i}; rescaling the
ridge by the same factor leaves the minimiser unchanged, so the shift is exact.

lambda = 0: on rows whose prefix leaves C_kk singular the minimiser is not unique; the
oracle returns the lambda -> 0+ limit, y = C_kk^+ zbar (symmetric pseudo-inverse,
eigenvalues <= 1e-12 * the largest dropped).  The rows of C_vk lie in range(C_kk), so this
is the limit of the lambda > 0 solutions.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os

import numpy as np

__all__ = ["lla_row", "lla_row_parts", "lla_forward", "lla_rows", "map_rows", "lla_decode"]


def lla_row_parts(q_i, K, V, h, lam):
    """All intermediate quantities of one LLA row.

    q_i: (d,), K: (i+1, d) the causal key prefix, V: (i+1, d_v) the value prefix.
    Returns a dict with m, omega (shifted), kbar, vbar, C_kk, C_vk, lam_shifted, zbar, y, b.
    """
    q_i = np.asarray(q_i, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    s = (K @ q_i) / h                     # scores s_ij = q_i . k_j / h
    m = float(np.max(s))                  # safe-softmax shift
    w = np.exp(s - m)                     # shifted kernel weights
    omega = float(np.sum(w))
    kbar = (w @ K) / omega
    vbar = (w @ V) / omega
    Kc = K - kbar                          # centred keys  k_j - kbar_i
    Vc = V - vbar                          # centred values v_j - vbar_i
    C_kk = (Kc * w[:, None]).T @ Kc        # sum_j w (k - kbar)(k - kbar)^T
    C_vk = (Vc * w[:, None]).T @ Kc        # sum_j w (v - vbar)(k - kbar)^T
    lam_s = lam * np.exp(-m)               # ridge rescaled by the same shift
    zbar = kbar - q_i
    d = K.shape[1]
    if lam_s > 0.0:
        L = np.linalg.cholesky(C_kk + lam_s * np.eye(d))
        y = np.linalg.solve(L.T, np.linalg.solve(L, zbar))
    else:
        evals, evecs = np.linalg.eigh(C_kk)
        top = max(float(evals[-1]), 0.0)
        keep = evals > 1e-12 * top if top > 0 else np.zeros_like(evals, dtype=bool)
        inv = np.zeros_like(evals)
        inv[keep] = 1.0 / evals[keep]
        y = evecs @ (inv * (evecs.T @ zbar))
    b = vbar - C_vk @ y
    return dict(m=m, w=w, omega=omega, kbar=kbar, vbar=vbar, C_kk=C_kk, C_vk=C_vk,
                lam_shifted=lam_s, zbar=zbar, y=y, b=b)


def lla_row(q_i, K, V, h, lam):
    """LLA output b_i of one query against its causal prefix (K, V rows 0..i)."""
    return lla_row_parts(q_i, K, V, h, lam)["b"]


def _rows_worker(args):
    """Rows of one head: qh [r, d] (the queries of the rows), kh/vh the prefix up to the
    longest row, xh [r, .] an optional per-row extra input (or None), idx the row positions."""
    fn, qh, kh, vh, xh, idx, extra = args
    out = np.empty((len(idx), vh.shape[-1]), dtype=np.float64)
    for t, i in enumerate(idx):
        if xh is None:
            out[t] = fn(qh[t], kh[: i + 1], vh[: i + 1], *extra)
        else:
            out[t] = fn(qh[t], kh[: i + 1], vh[: i + 1], xh[t], *extra)
    return out


def map_rows(fn, q, k, v, rows, extra, per_row=None, workers=1):
    """Apply a row function to a list of (b, head, i) rows of [B, H, n, .] inputs.

    ``fn(q_i, K, V, [x_i,] *extra)`` receives the query, the causal key and value prefixes
    (rows 0..i) and, when ``per_row`` is given, that array's row i.  Returns an fp64 array
    [len(rows), d_v].  With workers > 1 the rows run in a process pool, in tasks of one
    head each of about the same cost.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    x = None if per_row is None else np.asarray(per_row)
    rows = list(rows)
    dv = v.shape[-1]
    by_head = {}
    for t, (b, hh, i) in enumerate(rows):
        by_head.setdefault((b, hh), []).append((i, t))
    total = sum(i + 1 for (_, _, i) in rows)
    target = max(1, total // max(1, 4 * workers))
    tasks = []
    for (b, hh), lst in by_head.items():
        lst.sort(reverse=True)
        cur, cost = [], 0
        for i, t in lst:
            cur.append((i, t))
            cost += i + 1
            if cost >= target:
                tasks.append(((b, hh), cur))
                cur, cost = [], 0
        if cur:
            tasks.append(((b, hh), cur))

    def task_args(task):
        (b, hh), lst = task
        top = max(i for i, _ in lst) + 1
        idx = [i for i, _ in lst]
        xh = None if x is None else np.asarray(x[b, hh, idx], np.float64)
        return (fn, np.asarray(q[b, hh, idx], np.float64), np.asarray(k[b, hh, :top], np.float64),
                np.asarray(v[b, hh, :top], np.float64), xh, idx, tuple(extra))

    out = np.empty((len(rows), dv), dtype=np.float64)
    if workers <= 1 or len(tasks) < 2:
        for task in tasks:
            res = _rows_worker(task_args(task))
            for r, (_, t) in zip(res, task[1]):
                out[t] = r
        return out
    with _cf.ProcessPoolExecutor(max_workers=workers) as ex:
        futs = {ex.submit(_rows_worker, task_args(task)): task for task in tasks}
        for f in _cf.as_completed(futs):
            for r, (_, t) in zip(f.result(), futs[f][1]):
                out[t] = r
    return out


def lla_rows(q, k, v, h, lam, rows, workers=1):
    """LLA outputs for a list of (b, head, i) rows.

    q, k, v: [B, H, n, d] arrays (any float dtype; upcast exactly to fp64).
    rows: iterable of (b, head, i).  Returns an fp64 array [len(rows), d_v].
    With workers > 1 the rows run in a process pool, in tasks of one head each.
    """
    return map_rows(lla_row, q, k, v, rows, (h, lam), workers=workers)


def lla_forward(q, k, v, h, lam, workers=1):
    """Causal LLA forward over every row: [B, H, n, d] -> [B, H, n, d_v] fp64."""
    q = np.asarray(q, dtype=np.float64)
    B, H, n, _ = q.shape
    rows = [(b, hh, i) for b in range(B) for hh in range(H) for i in range(n)]
    out = lla_rows(q, k, v, h, lam, rows, workers=workers)
    return out.reshape(B, H, n, -1)


def default_workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def lla_decode(q, k, v, h, lam):
    """LLA decode step: one query per (batch, head) against its whole key-value cache.

    q: [B, H, d]; k: [B, H, L, d]; v: [B, H, L, d_v].  The query is the newest position and
    every cached key is in its prefix, so each output is lla_row over the full cache.
    Returns [B, H, d_v] fp64."""
    q = np.asarray(q)
    B, H, _ = q.shape
    out = np.empty((B, H, np.asarray(v).shape[-1]), dtype=np.float64)
    for b in range(B):
        for hh in range(H):
            out[b, hh] = lla_row(q[b, hh], k[b, hh], v[b, hh], h, lam)
    return out
