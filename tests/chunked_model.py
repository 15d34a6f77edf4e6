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

Segmented form (``segmented_prefill``): the chunk update is affine in the start
state, S_new = S M_c + N_c with M_c = gamma_C I - W^T diag(exp(G_C - G)) K,
W = T diag(beta gamma) K. So a run of chunks (a segment) maps its start state
S_p to S_p M_p + N_p, where N_p is the end state from a zero start and M_p is
what the same chunk steps make of the identity with v = 0 (each row of the
identity is a state row; rows never mix). With the maps of segments 1 .. P-2
and the true end state of segment 0, every segment start follows by
S_{p+1} = S_p M_p + N_p, and each segment then runs as an ordinary chunked pass
from its true start. This is the decomposition the GPU prefill uses to run the
segments of one sequence in parallel.
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


def _chunk(x, b, h, kh, t0, C):
    """Chunk of C tokens from t0 (rows past the end zero, with g = beta = 0)."""
    q, k, v, g, beta = x
    T, dk, dv = q.shape[2], q.shape[3], v.shape[3]
    n = max(0, min(C, T - t0))
    Q = np.zeros((C, dk)); K = np.zeros((C, dk)); V = np.zeros((C, dv))
    gc = np.zeros(C); bc = np.zeros(C)
    Q[:n] = q[b, kh, t0:t0 + n]; K[:n] = k[b, kh, t0:t0 + n]; V[:n] = v[b, h, t0:t0 + n]
    gc[:n] = g[b, h, t0:t0 + n]; bc[:n] = beta[b, h, t0:t0 + n]
    return Q, K, V, gc, bc, n


def chunk_step(S, Q, K, V, gc, bc, scale):
    """One chunk of the WY form from start state S: returns (O, S at the chunk end)."""
    C = K.shape[0]
    G = np.cumsum(gc)
    gamma = np.exp(G)
    diff = G[:, None] - G[None, :]
    lower = np.tril(np.ones((C, C), bool))
    Gam = np.where(lower, np.exp(np.where(lower, diff, 0.0)), 0.0)
    A = np.tril(bc[:, None] * (K @ K.T) * Gam, -1)
    Tm = inverse_unit_lower(-A)
    R = bc[:, None] * (V - gamma[:, None] * (K @ S.T))
    U = Tm @ R
    Aqk = np.tril(scale * (Q @ K.T) * Gam)
    O = gamma[:, None] * (scale * Q @ S.T) + Aqk @ U
    S = gamma[-1] * S + (np.exp(G[-1] - G)[:, None] * U).T @ K
    return O, S


def chunked_prefill(q, k, v, g, beta, s0, scale, chunk, head_map=0):
    """Chunked WY prefill in float64. Shapes as the oracle's prefill; returns (o, s_final)."""
    B, Hk, T, dk = q.shape
    Hv, dv = v.shape[1], v.shape[3]
    o = np.zeros((B, Hv, T, dv))
    S_out = np.zeros((B, Hv, dv, dk))
    C = chunk
    x = (q, k, v, g, beta)
    for b in range(B):
        for h in range(Hv):
            kh = h % Hk if head_map == 0 else h // (Hv // Hk)
            S = np.zeros((dv, dk)) if s0 is None else np.array(s0[b, h], dtype=np.float64)
            for t0 in range(0, T, C):
                Q, K, V, gc, bc, n = _chunk(x, b, h, kh, t0, C)
                O, S = chunk_step(S, Q, K, V, gc, bc, scale)
                o[b, h, t0:t0 + n] = O[:n]
            S_out[b, h] = S
    return o, S_out


def segment_bounds(T, chunk, P):
    """Chunk ranges [c0, c1) of P segments of equal chunk counts (the last may be shorter)."""
    nc = -(-T // chunk)
    per = -(-nc // P)
    return [(min(p * per, nc), min((p + 1) * per, nc)) for p in range(P)]


def segmented_prefill(q, k, v, g, beta, s0, scale, chunk, P, head_map=0):
    """The chunked prefill run as P segments: maps of segments 1 .. P-2 (from a zero state with v,
    and from the identity with v = 0), the true end state of segment 0, the chain of segment
    starts, then every segment from its start. Returns (o, s_final, starts)."""
    B, Hk, T, dk = q.shape
    Hv, dv = v.shape[1], v.shape[3]
    C = chunk
    x = (q, k, v, g, beta)
    bounds = segment_bounds(T, C, P)
    o = np.zeros((B, Hv, T, dv))
    S_out = np.zeros((B, Hv, dv, dk))
    starts = np.zeros((B, Hv, P, dv, dk))
    for b in range(B):
        for h in range(Hv):
            kh = h % Hk if head_map == 0 else h // (Hv // Hk)
            S0 = np.zeros((dv, dk)) if s0 is None else np.array(s0[b, h], dtype=np.float64)

            def run(S, c0, c1, with_v=True, out=False):
                for c in range(c0, c1):
                    Q, K, V, gc, bc, n = _chunk(x, b, h, kh, c * C, C)
                    O, S = chunk_step(S, Q, K, V if with_v else np.zeros_like(V), gc, bc, scale)
                    if out:
                        o[b, h, c * C:c * C + n] = O[:n]
                return S

            starts[b, h, 0] = S0
            if P > 1:
                starts[b, h, 1] = run(S0, *bounds[0])
            for p in range(1, P - 1):
                N = run(np.zeros((dv, dk)), *bounds[p])
                M = run(np.eye(dk), *bounds[p], with_v=False)
                starts[b, h, p + 1] = starts[b, h, p] @ M + N
            for p in range(P):
                S = run(starts[b, h, p], *bounds[p], out=True)
            S_out[b, h] = S
    return o, S_out, starts
