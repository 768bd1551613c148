"""Plain fp64 CPU oracle for the causal Parallax forward with a given probe.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP path.

What it computes (the plain definition, row by row, in fp64):

For query i of one (batch, head), with the causal prefix {(k_j, v_j) : j <= i}, the
softmax weights p_ij = softmax_j(q_i . k_j / h), the softmax output vbar_i = E_p[v]
(softmax attention), the weighted key mean kbar_i = E_p[k] and the softmax-weighted
key-value covariance Sigma_KV = E_p[(v - vbar)(k - kbar)^T], the Parallax output for the
probe rho_i is

    o_i = vbar_i - Sigma_KV rho_i .

Sources:
  * "Parallax" blog post (Tilde Research), section 2, "Additive Correction to Softmax"
    (p_i, Sigma_KV, the additive form with the boundary factor eta) and "Parallax" (eta set
    to 0, the probe taken as given instead of solved);
  * the same post, Appendix B "LLA as an additive correction -- the derivation" (the
    additive form from the LLA forward; eta = 0 with a given probe is Parallax);
  * "Parallax: Parameterized Local Linear Attention for Language Modeling" (arXiv
    2605.29157, HTML), the Parallax paragraph (eta = 0 is the scoring form with centred
    scores t_ij - tbar_i and denominator omega_i).
Here rho_i is an input (the pages produce it by a learned projection of the layer input;
that projection and any normalisation of rho belong to the caller).  The display equations
are missing from the extracted text; the reading used is the one above, which is what the
additive form gives with eta = 0 and which the streaming two-branch form of section 3 ("One
extra branch, no extra I/O") and the merge of Appendix C reproduce.
"""
from __future__ import annotations

import numpy as np

from .lla_oracle import map_rows

__all__ = ["parallax_row", "parallax_row_parts", "parallax_rows", "parallax_forward",
           "parallax_decode", "parallax_backward"]


def parallax_row_parts(q_i, K, V, rho_i, h):
    """All intermediate quantities of one Parallax row.

    q_i: (d,), K: (i+1, d) the causal key prefix, V: (i+1, d_v) the value prefix, rho_i: (d,)
    the probe.  Returns a dict with p (softmax weights), vbar (= softmax attention output),
    kbar, sigma_kv (d_v x d) and o.
    """
    q_i = np.asarray(q_i, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    rho_i = np.asarray(rho_i, dtype=np.float64)
    s = (K @ q_i) / h                      # scores q_i . k_j / h
    w = np.exp(s - np.max(s))              # safe softmax: the shift cancels in p
    p = w / np.sum(w)
    vbar = p @ V                           # softmax attention output
    kbar = p @ K
    sigma_kv = ((V - vbar) * p[:, None]).T @ (K - kbar)   # E_p[(v - vbar)(k - kbar)^T]
    o = vbar - sigma_kv @ rho_i
    return dict(p=p, vbar=vbar, kbar=kbar, sigma_kv=sigma_kv, o=o)


def parallax_row(q_i, K, V, rho_i, h):
    """Parallax output o_i of one query against its causal prefix (K, V rows 0..i)."""
    return parallax_row_parts(q_i, K, V, rho_i, h)["o"]


def parallax_rows(q, k, v, rho, h, rows, workers=1):
    """Parallax outputs for a list of (b, head, i) rows.

    q, k, rho: [B, H, n, d]; v: [B, H, n, d_v] (any float dtype; upcast exactly to fp64).
    Returns an fp64 array [len(rows), d_v]."""
    return map_rows(parallax_row, q, k, v, rows, (h,), per_row=rho, workers=workers)


def parallax_forward(q, k, v, rho, h, workers=1):
    """Causal Parallax forward over every row: [B, H, n, d] -> [B, H, n, d_v] fp64."""
    q = np.asarray(q)
    B, H, n, _ = q.shape
    rows = [(b, hh, i) for b in range(B) for hh in range(H) for i in range(n)]
    return parallax_rows(q, k, v, rho, h, rows, workers=workers).reshape(B, H, n, -1)



def parallax_decode(q, k, v, rho, h):
    """Parallax decode step: one query per (batch, head) against its whole key-value cache.

    q, rho: [B, H, d]; k: [B, H, L, d]; v: [B, H, L, d_v].  Every cached key is in the
    query's prefix (the query is the newest position; its own key is the cache's last
    entry), so each output is parallax_row over the full cache.  Returns [B, H, d_v] fp64.
    (The decode setting of the "Parallax" blog post, section 3 "Optimized Decode Kernel".)
    """
    q = np.asarray(q)
    B, H, _ = q.shape
    out = np.empty((B, H, np.asarray(v).shape[-1]), dtype=np.float64)
    for b in range(B):
        for hh in range(H):
            out[b, hh] = parallax_row(q[b, hh], k[b, hh], v[b, hh], rho[b, hh], h)
    return out


def _parallax_head_torch(Q, K, V, R, h):
    """Causal Parallax forward of one head in torch fp64 ops: the definition
    o_i = vbar_i - Sigma_KV rho_i with Sigma_KV rho_i expanded as
    sum_j p_ij (v_j - vbar_i)(u_ij - ubar_i), u_ij = rho_i . k_j, ubar_i = kbar_i . rho_i."""
    import torch
    n = Q.shape[0]
    S = (Q @ K.T) / h
    mask = torch.triu(torch.ones(n, n, dtype=torch.bool), diagonal=1)
    P = torch.softmax(S.masked_fill(mask, float("-inf")), dim=-1)
    Vbar = P @ V
    Kbar = P @ K
    U = R @ K.T
    Ubar = (Kbar * R).sum(-1, keepdim=True)
    W = P * (U - Ubar)                                   # p_ij (u_ij - ubar_i)
    sigma_rho = W @ V - Vbar * W.sum(-1, keepdim=True)   # sum_j p_ij (v_j - vbar_i)(u_ij - ubar_i)
    return Vbar - sigma_rho


def parallax_backward(q, k, v, rho, h, dout):
    """Gradients (dq, dk, dv, drho) of sum(o * dout) for the causal Parallax forward with a
    given probe, in fp64, by reverse-mode differentiation (torch autograd on the CPU) of the
    definition above, head by head.  All arrays [B, H, n, d]; returns fp64 numpy arrays.
    (The backward the "Parallax" blog post outlines in Appendix F, "Parallax backward".)"""
    import torch
    q, k, v, rho, dout = (np.asarray(x, dtype=np.float64) for x in (q, k, v, rho, dout))
    grads = [np.empty_like(x) for x in (q, k, v, rho)]
    B, H = q.shape[:2]
    for b in range(B):
        for hh in range(H):
            ts = [torch.tensor(x[b, hh], dtype=torch.float64, requires_grad=True) for x in (q, k, v, rho)]
            o = _parallax_head_torch(*ts, h)
            (o * torch.tensor(dout[b, hh], dtype=torch.float64)).sum().backward()
            for g, t in zip(grads, ts):
                g[b, hh] = t.grad.numpy()
    return tuple(grads)
