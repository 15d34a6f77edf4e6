"""A float64 numpy model of the chunked (WY) form of the gated delta rule.

This is the algorithm the prefill kernel implements, written plainly so that it
can be checked against the sequential oracle. It is test-side only and shares
nothing with the HIP sources.

For one (b, h) and a chunk of C tokens with start state S (dv x dk):

* G_t = sum_{s<=t} g_s (within the chunk), gamma_t = exp(G_t),
  Gamma_ts = exp(G_t - G_s) for s <= t.
* A = strict_lower(diag(beta) (K K^T o Gamma)),  T = (I + A)^{-1}.
* R = diag(beta) (V - diag(gamma) K S^T),  U = T R.
* O = diag(gamma) (scale Q) S^T + lower_incl(scale Q K^T o Gamma) U.
* S <- gamma_C S + (diag(exp(G_C - G)) U)^T K.

Derivation: with u_t = beta_t (v_t - alpha_t S_{t-1} k_t) the recurrence is
S_t = alpha_t S_{t-1} + u_t k_t^T, so S_t = gamma_t S + sum_{s<=t} Gamma_ts u_s k_s^T;
substituting S_{t-1} gives the unit-lower system (I + A) U = R above. A padded
step (beta = 0, g = 0, zero q/k/v) has a zero row in A and R, so it contributes
nothing: the no-op rule in chunked form.

The triangular inverse follows the forward substitution of the tinygrad helper
``inverse_unit_lower`` ("27b 935/47" compare page, llm/kernels/generic.py),
which inverts I - x for a strictly lower-triangular x; here x = -A.
"""
from __future__ import annotations

import numpy as np


def inverse_unit_lower(x: np.ndarray) -> np.ndarray:
    """(I - x)^{-1} for strictly lower-triangular x, row by row:
    N = (I - x)^{-1} - I satisfies N[r] = x[r] + sum_{i<r} x[r, i] N[i]."""
    n = x.shape[-1]
    N = np.zeros_like(x)
    for r in range(1, n):
        N[r] = x[r] + x[r, :r] @ N[:r]
        N[r, r:] = 0.0
    return N + np.eye(n)


def chunked_prefill(q, k, v, g, beta, s0, scale, chunk, head_map=0):
    """Chunked WY prefill in float64. Shapes as the oracle's prefill; returns (o, s_final)."""
    B, Hk, T, dk = q.shape
    Hv, dv = v.shape[1], v.shape[3]
    o = np.zeros((B, Hv, T, dv))
    S_out = np.zeros((B, Hv, dv, dk))
    C = chunk
    for b in range(B):
        for h in range(Hv):
            kh = h % Hk if head_map == 0 else h // (Hv // Hk)
            S = np.zeros((dv, dk)) if s0 is None else np.array(s0[b, h], dtype=np.float64)
            for t0 in range(0, T, C):
                n = min(C, T - t0)
                Q = np.zeros((C, dk)); K = np.zeros((C, dk)); V = np.zeros((C, dv))
                gc = np.zeros(C); bc = np.zeros(C)
                Q[:n] = q[b, kh, t0:t0 + n]; K[:n] = k[b, kh, t0:t0 + n]; V[:n] = v[b, h, t0:t0 + n]
                gc[:n] = g[b, h, t0:t0 + n]; bc[:n] = beta[b, h, t0:t0 + n]
                G = np.cumsum(gc)
                gamma = np.exp(G)
                diff = G[:, None] - G[None, :]
                Gam = np.where(np.tril(np.ones((C, C), bool)), np.exp(np.minimum(diff, 0.0)), 0.0)
                A = np.tril(bc[:, None] * (K @ K.T) * Gam, -1)
                Tm = inverse_unit_lower(-A)
                R = bc[:, None] * (V - gamma[:, None] * (K @ S.T))
                U = Tm @ R
                Aqk = np.tril(scale * (Q @ K.T) * Gam)
                O = gamma[:, None] * (scale * Q @ S.T) + Aqk @ U
                o[b, h, t0:t0 + n] = O[:n]
                S = gamma[-1] * S + (np.exp(G[-1] - G)[:, None] * U).T @ K
            S_out[b, h] = S
    return o, S_out
