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

__all__ = ["lla_row", "lla_row_parts", "lla_forward", "lla_rows"]


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
    q, k, v, h, lam, items = args
    out = np.empty((len(items), v.shape[-1]), dtype=np.float64)
    for t, (bh, i) in enumerate(items):
        out[t] = lla_row(q[bh, i], k[bh, : i + 1], v[bh, : i + 1], h, lam)
    return out


def lla_rows(q, k, v, h, lam, rows, workers=1):
    """LLA outputs for a list of (b, head, i) rows.

    q, k, v: [B, H, n, d] arrays (any float dtype; upcast exactly to fp64).
    rows: iterable of (b, head, i).  Returns an fp64 array [len(rows), d_v].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, n, d = q.shape
    qf = q.reshape(B * H, n, d)
    kf = k.reshape(B * H, n, d)
    vf = v.reshape(B * H, n, v.shape[-1])
    items = [(b * H + hh, i) for (b, hh, i) in rows]
    if workers <= 1 or len(items) < 64:
        return _rows_worker((qf, kf, vf, h, lam, items))
    # Split the rows into chunks of about equal cost (row i costs ~ i+1).
    order = sorted(range(len(items)), key=lambda t: -items[t][1])
    chunks = [[] for _ in range(4 * workers)]
    loads = [0] * len(chunks)
    for t in order:
        c = min(range(len(chunks)), key=loads.__getitem__)
        chunks[c].append(t)
        loads[c] += items[t][1] + 1
    chunks = [c for c in chunks if c]
    out = np.empty((len(items), vf.shape[-1]), dtype=np.float64)
    with _cf.ProcessPoolExecutor(max_workers=workers) as ex:
        futs = {ex.submit(_rows_worker, (qf, kf, vf, h, lam, [items[t] for t in c])): c
                for c in chunks}
        for f in _cf.as_completed(futs):
            res = f.result()
            for r, t in zip(res, futs[f]):
                out[t] = r
    return out


def lla_forward(q, k, v, h, lam, workers=1):
    """Causal LLA forward over every row: [B, H, n, d] -> [B, H, n, d_v] fp64."""
    q = np.asarray(q, dtype=np.float64)
    B, H, n, _ = q.shape
    rows = [(b, hh, i) for b in range(B) for hh in range(H) for i in range(n)]
    out = lla_rows(q, k, v, h, lam, rows, workers=workers)
    return out.reshape(B, H, n, -1)


def default_workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))
