"""Chunkwise (WY / UT-transform) evaluation of the KDA recurrence in fp64.

Test helper: it checks, against the token-serial oracle, the chunk algebra
that the HIP kernels implement.  It is derived from the state-update equation
[core.today "Kimi Linear 특집", ch.4 혁신 2] by unrolling one chunk of C tokens
with a start state S0 (local positions r = 0..C-1, G = within-chunk inclusive
cumulative sum of g, Gamma = exp(G)):

  A[r, i]  = beta_r * sum_c k_rc k_ic exp(G_rc - G_ic)          (i <  r)
  Tm       = (I + A)^-1 diag(beta)
  U'       = Tm (V - (K * Gamma) S0)      (= beta_r times the delta-rule error)
  M[r, i]  = sum_c q_rc k_ic exp(G_rc - G_ic)                    (i <= r)
  O        = scale * ((Q * Gamma) S0 + M U')
  S_C      = Diag(Gamma_last) S0 + (K * exp(G_last - G))^T U'

The pages only state that this diagonal-plus-low-rank transition admits an
efficient chunkwise parallel algorithm [same page, ch.4 혁신 2]; the formulas
above are the plain reading of that remark.
"""
from __future__ import annotations

import numpy as np


def chunkwise_fwd(q, k, v, g, beta, scale, S0, C):
    """One sequence, one head.  q, k, g: [T, DK]; v: [T, DV]; beta: [T]."""
    T, DK = q.shape
    DV = v.shape[1]
    S = np.zeros((DK, DV)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, DV))
    for s in range(0, T, C):
        e = min(s + C, T)
        n = e - s
        Q, K, V, b = q[s:e], k[s:e], v[s:e], beta[s:e]
        G = np.cumsum(g[s:e], axis=0)
        A = np.zeros((n, n))
        M = np.zeros((n, n))
        for r in range(n):
            for i in range(r + 1):
                w = np.exp(G[r] - G[i])
                if i < r:
                    A[r, i] = b[r] * np.sum(K[r] * K[i] * w)
                M[r, i] = np.sum(Q[r] * K[i] * w)
        Tm = np.linalg.solve(np.eye(n) + A, np.diag(b))
        Gam = np.exp(G)
        Up = Tm @ (V - (K * Gam) @ S)
        o[s:e] = scale * ((Q * Gam) @ S + M @ Up)
        S = np.exp(G[-1])[:, None] * S + (K * np.exp(G[-1] - G)).T @ Up
    return o, S
