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


# ---- per-channel decay (KDA): S_t = S_{t-1} diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
#
# With G [C][dk] the per-channel prefix of g inside a chunk and u_t = beta_t (v_t - S_{t-1}
# diag(alpha_t) k_t), S_t = S diag(e^{G_t}) + sum_{s<=t} u_s (k_s o e^{G_t - G_s})^T, so
# (I + A) U = R with
#   A[t, s]   = beta_t sum_c k_tc k_sc e^{G_tc - G_sc}          (s < t)
#   R         = diag(beta) (V - (K o e^G) S^T)
#   O         = scale (Q o e^G) S^T + A_qk U,  A_qk[t, s] = scale sum_c q_tc k_sc e^{G_tc - G_sc} (s <= t)
#   S        <- S diag(e^{G_C}) + U^T (K o e^{G_C - G}).
# The decays inside A and A_qk differ per channel, so they cannot be a mask on K K^T; the kernel
# forms them from scaled operands (kda_blocks_factored), which needs every factor in range.

KDA_G_MIN = -10.0  # the chunked form takes log-decays below this as this (see kda_blocks_factored)
KDA_TILE = 16


def kda_blocks_exact(Q, K, G, bc, scale):
    """A (strict lower, with beta) and A_qk (lower incl., with scale) from the pairwise decays."""
    C = K.shape[0]
    A = np.zeros((C, C))
    Aqk = np.zeros((C, C))
    for t in range(C):
        for s in range(t + 1):
            f = np.exp(G[t] - G[s])
            if s < t:
                A[t, s] = bc[t] * np.dot(K[t] * f, K[s])
            Aqk[t, s] = scale * np.dot(Q[t] * f, K[s])
    return A, Aqk


def kda_blocks_factored(Q, K, G, bc, scale, tile=KDA_TILE):
    """The same blocks as 16 x 16 tiles of products of scaled operands, as the kernel forms them:

    * block (m, j), j < m: reference b = the last token of tile m - 1; left k_t o e^{G_t - G_b}
      (t in tile m, a decay, <= 1), right k_s o e^{G_b - G_s} (s <= b, <= 1): both fit float16;
    * block (m, m): reference r = token 7 of the tile; left k_t o e^{G_t - G_r}, right
      k_s o e^{G_r - G_s}: factors between e^{-8 |g|max} and e^{8 |g|max}, inside float32 range
      (e^{+-80}) when every log-decay is >= KDA_G_MIN = -10; formed in float32.
    Returns (A, A_qk, the largest |exponent| used in a diagonal tile)."""
    C, dk = K.shape
    A = np.zeros((C, C))
    Aqk = np.zeros((C, C))
    big = 0.0
    for m in range(C // tile):
        tm = slice(tile * m, tile * (m + 1))
        r = tile * m + tile // 2 - 1
        e_l, e_r = G[tm] - G[r], G[r] - G[tm]
        big = max(big, float(np.max(np.abs(e_l))))
        L, Lq, Rt = K[tm] * np.exp(e_l), Q[tm] * np.exp(e_l), K[tm] * np.exp(e_r)
        A[tm, tm] = np.tril(bc[tm, None] * (L @ Rt.T), -1)
        Aqk[tm, tm] = np.tril(scale * (Lq @ Rt.T))
        if m > 0:
            b = tile * m - 1
            Lo, Loq = K[tm] * np.exp(G[tm] - G[b]), Q[tm] * np.exp(G[tm] - G[b])
            Ro = K[:tile * m] * np.exp(G[b] - G[:tile * m])
            A[tm, :tile * m] = bc[tm, None] * (Lo @ Ro.T)
            Aqk[tm, :tile * m] = scale * (Loq @ Ro.T)
    return A, Aqk, big


def kda_chunk_step(S, Q, K, V, gc, bc, scale, factored=False):
    """One chunk of the per-channel-decay WY form (gc [C][dk]); returns (O, S at the chunk end).
    factored: the blocks as the kernel forms them (chunk a multiple of KDA_TILE)."""
    G = np.cumsum(gc, axis=0)
    if factored:
        A, Aqk, _ = kda_blocks_factored(Q, K, G, bc, scale)
    else:
        A, Aqk = kda_blocks_exact(Q, K, G, bc, scale)
    Tm = inverse_unit_lower(-A)
    R = bc[:, None] * (V - (K * np.exp(G)) @ S.T)
    U = Tm @ R
    O = scale * (Q * np.exp(G)) @ S.T + Aqk @ U
    S = S * np.exp(G[-1])[None, :] + U.T @ (K * np.exp(G[-1] - G))
    return O, S


def _kda_chunk(x, b, h, kh, t0, C):
    q, k, v, g, beta = x
    T, dk = q.shape[2], q.shape[3]
    n = max(0, min(C, T - t0))
    Q, K, V, _, bc, _ = _chunk((q, k, v, np.zeros(beta.shape), beta), b, h, kh, t0, C)
    gc = np.zeros((C, dk))
    gc[:n] = g[b, h, t0:t0 + n]
    return Q, K, V, gc, bc, n


def kda_chunked_prefill(q, k, v, g, beta, s0, scale, chunk, head_map=0, factored=False, clamp=False, P=1):
    """Chunked per-channel-decay prefill in float64 (g [B][Hv][T][dk]); clamp: log-decays below
    KDA_G_MIN taken as KDA_G_MIN; P > 1: run as P segments through their affine maps, as the
    segmented prefill does. Returns (o, s_final)."""
    B, Hk, T, dk = q.shape
    Hv, dv = v.shape[1], v.shape[3]
    C = chunk
    g = np.maximum(g, KDA_G_MIN) if clamp else g
    x = (q, k, v, g, beta)
    bounds = segment_bounds(T, C, P)
    o = np.zeros((B, Hv, T, dv))
    S_out = np.zeros((B, Hv, dv, dk))
    for b in range(B):
        for h in range(Hv):
            kh = h % Hk if head_map == 0 else h // (Hv // Hk)
            S0 = np.zeros((dv, dk)) if s0 is None else np.array(s0[b, h], dtype=np.float64)

            def run(S, c0, c1, with_v=True, out=False):
                for c in range(c0, c1):
                    Q, K, V, gc, bc, n = _kda_chunk(x, b, h, kh, c * C, C)
                    O, S = kda_chunk_step(S, Q, K, V if with_v else np.zeros_like(V), gc, bc, scale, factored)
                    if out:
                        o[b, h, c * C:c * C + n] = O[:n]
                return S

            starts = [S0]
            if P > 1:
                starts.append(run(S0, *bounds[0]))
            for p in range(1, P - 1):
                N = run(np.zeros((dv, dk)), *bounds[p])
                M = run(np.eye(dk), *bounds[p], with_v=False)
                starts.append(starts[p] @ M + N)
            for p in range(P):
                S = run(starts[p], *bounds[p], out=True)
            S_out[b, h] = S
    return o, S_out
