"""Pins of the float64 oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function takes a loaded oracle and raises AssertionError when
the oracle disagrees with what mathematics or the pages fix. They are run on
the real oracle (test_oracle_pins.py) and on copies of it with planted
mistakes (test_oracle_mutants.py), where at least one pin must fail.

The independent references used here:

* dense brute-force unrolling of the recurrence into products of dk x dk
  transition matrices (numpy, float64);
* exact rational arithmetic (fractions.Fraction) on tiny inputs;
* the one-step formula of the tinygrad gated-delta decode test, which reads
  the output off the state before the update ("27b 935/47" compare page,
  ``test_gated_delta_decode_matches_reference``): with delta = (v - alpha*S k)
  * beta, core = alpha * S q + delta * (k . q) and S' = alpha*S + delta k^T;
* closed forms: beta = 0 (pure decay), delta-rule recall with orthonormal keys;
* exact invariants: padded steps (beta = 0, g = 0, q = k = v = 0) are no-ops
  (page "mergable fast RDNA3 Qwen 3.6", symbolic-length prefill entry),
  continuation splits, scale linearity, head-map relabelling, thread count;
* for the gated RMSNorm epilogue: unit root-mean-square rows, the eps closed
  form, quoted sigmoid values, per-column weights and row independence;
* for the input prologue: single-tap convolutions against quoted SiLU values,
  continuation splits, the q/k normalisation against the unnormalised v path,
  and one-hot channels landing in their head-major slots.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

TILED, GROUPED = 0, 1


def _rand_inputs(rng, B, Hk, Hv, T, d, s0=True, unit_keys=True):
    q = rng.standard_normal((B, Hk, T, d)).astype(np.float32)
    k = rng.standard_normal((B, Hk, T, d))
    if unit_keys:
        k = k / np.linalg.norm(k, axis=-1, keepdims=True)
    k = k.astype(np.float32)
    v = rng.standard_normal((B, Hv, T, d)).astype(np.float32)
    g = (-np.log1p(np.exp(rng.standard_normal((B, Hv, T))))).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((B, Hv, T))))).astype(np.float32)
    S0 = rng.normal(0, 0.3, (B, Hv, d, d)) if s0 else None
    return q, k, v, g, beta, S0


def _kh(h, Hk, Hv, head_map):
    return h % Hk if head_map == TILED else h // (Hv // Hk)


def _rel(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))) / max(np.max(np.abs(b)), 1e-300))


def pin_bruteforce_unroll(orc, seed=11):
    """S_t = S_0 P(1..t) + sum_s beta_s v_s k_s^T P(s+1..t), P(a..b) = A_a ... A_b,
    A_t = exp(g_t) (I - beta_t k_t k_t^T); o_t = S_t (scale q_t). Dense matrices, float64."""
    rng = np.random.default_rng(seed)
    B, Hk, Hv, T, d = 1, 2, 4, 10, 5
    scale = 0.37
    q, k, v, g, beta, S0 = _rand_inputs(rng, B, Hk, Hv, T, d)
    o, S = orc.prefill(q, k, v, g, beta, S0, scale=scale, head_map=TILED)
    I = np.eye(d)
    for h in range(Hv):
        kh = _kh(h, Hk, Hv, TILED)
        K = k[0, kh].astype(np.float64)
        A = [math.exp(float(g[0, h, t])) * (I - float(beta[0, h, t]) * np.outer(K[t], K[t])) for t in range(T)]
        for t in range(T):
            P = I.copy()
            for r in range(t + 1):
                P = P @ A[r]
            St = S0[0, h] @ P
            for s in range(t + 1):
                P = I.copy()
                for r in range(s + 1, t + 1):
                    P = P @ A[r]
                St = St + float(beta[0, h, s]) * np.outer(v[0, h, s].astype(np.float64), K[s]) @ P
            ot = St @ (scale * q[0, kh, t].astype(np.float64))
            assert _rel(o[0, h, t], ot) < 1e-12, ("unrolled output", h, t, _rel(o[0, h, t], ot))
            if t == T - 1:
                assert _rel(S[0, h], St) < 1e-12, ("unrolled final state", h, _rel(S[0, h], St))


def pin_exact_rational(orc, seed=12):
    """Tiny inputs in exact rational arithmetic. alpha is the double exp(g) that the C
    library returns (Python's math.exp calls the same libm), taken exactly as a Fraction."""
    rng = np.random.default_rng(seed)
    B, Hk, Hv, T, d = 1, 1, 2, 5, 3
    scale = 0.25
    q, k, v, g, beta, S0 = _rand_inputs(rng, B, Hk, Hv, T, d, unit_keys=False)
    S0 = S0.astype(np.float32).astype(np.float64)
    o, S = orc.prefill(q, k, v, g, beta, S0, scale=scale, head_map=TILED)
    F = Fraction
    for h in range(Hv):
        St = [[F(float(S0[0, h, i, j])) for j in range(d)] for i in range(d)]
        for t in range(T):
            a = F(math.exp(float(g[0, h, t])))
            bt = F(float(beta[0, h, t]))
            kk = [F(float(x)) for x in k[0, 0, t]]
            vv = [F(float(x)) for x in v[0, h, t]]
            qq = [F(scale) * F(float(x)) for x in q[0, 0, t]]
            # M = I - beta k k^T ; S <- a * S M + beta v k^T
            M = [[(F(1) if i == j else F(0)) - bt * kk[i] * kk[j] for j in range(d)] for i in range(d)]
            SM = [[sum(St[i][r] * M[r][j] for r in range(d)) for j in range(d)] for i in range(d)]
            St = [[a * SM[i][j] + bt * vv[i] * kk[j] for j in range(d)] for i in range(d)]
            ot = [sum(St[i][j] * qq[j] for j in range(d)) for i in range(d)]
            for i in range(d):
                err = abs(F(float(o[0, h, t, i])) - ot[i])
                assert err <= F(1, 10**13) * (1 + abs(ot[i])), ("rational output", h, t, i, float(err))
        for i in range(d):
            for j in range(d):
                err = abs(F(float(S[0, h, i, j])) - St[i][j])
                assert err <= F(1, 10**13) * (1 + abs(St[i][j])), ("rational state", h, i, j, float(err))


def pin_pages_one_step(orc, seed=13):
    """One decode step against the tinygrad decode test's formula (output from the state
    before the update): core = alpha*S q' + delta (k.q'), delta = beta (v - alpha S k)."""
    rng = np.random.default_rng(seed)
    B, Hk, Hv, d = 2, 2, 4, 16
    scale = 1.0 / math.sqrt(d)
    q = rng.standard_normal((B, Hk, d)).astype(np.float32)
    k = rng.standard_normal((B, Hk, d)).astype(np.float32)
    v = rng.standard_normal((B, Hv, d)).astype(np.float32)
    g = np.log(rng.uniform(0.9, 1.0, (B, Hv))).astype(np.float32)
    beta = rng.random((B, Hv), dtype=np.float32)
    S = rng.standard_normal((B, Hv, d, d))
    for head_map in (TILED, GROUPED):
        state = S.copy()
        o = orc.decode_step(q, k, v, g, beta, state, scale=scale, head_map=head_map)
        for b in range(B):
            for h in range(Hv):
                kh = _kh(h, Hk, Hv, head_map)
                kk, qq = k[b, kh].astype(np.float64), scale * q[b, kh].astype(np.float64)
                a = math.exp(float(g[b, h]))
                delta = (v[b, h] - a * (S[b, h] @ kk)) * float(beta[b, h])
                core = a * (S[b, h] @ qq) + delta * float(kk @ qq)
                nxt = a * S[b, h] + np.outer(delta, kk)
                assert _rel(o[b, h], core) < 1e-13, ("pages' core", head_map, b, h)
                assert _rel(state[b, h], nxt) < 1e-13, ("pages' next state", head_map, b, h)


def pin_padded_noop(orc, seed=14):
    """Inserting padded steps (beta = 0, g = 0, q = k = v = 0) anywhere changes nothing at
    the real positions and gives exactly zero outputs at the padded ones (bit-exact)."""
    rng = np.random.default_rng(seed)
    B, Hk, Hv, T, d = 1, 2, 4, 9, 8
    q, k, v, g, beta, S0 = _rand_inputs(rng, B, Hk, Hv, T, d)
    ref_o, ref_S = orc.prefill(q, k, v, g, beta, S0, scale=0.5)
    Tp = 14
    real = np.array([0, 1, 3, 4, 5, 8, 9, 10, 12])  # the 9 real tokens; padding in between and at the end
    qp, kp = np.zeros((B, Hk, Tp, d), np.float32), np.zeros((B, Hk, Tp, d), np.float32)
    vp = np.zeros((B, Hv, Tp, d), np.float32)
    gp, bp = np.zeros((B, Hv, Tp), np.float32), np.zeros((B, Hv, Tp), np.float32)
    qp[:, :, real], kp[:, :, real], vp[:, :, real] = q, k, v
    gp[:, :, real], bp[:, :, real] = g, beta
    o, S = orc.prefill(qp, kp, vp, gp, bp, S0, scale=0.5)
    assert np.array_equal(o[:, :, real], ref_o), "padded no-op: real outputs changed"
    pad = np.setdiff1d(np.arange(Tp), real)
    assert np.all(o[:, :, pad] == 0.0), "padded no-op: padded outputs are not zero"
    assert np.array_equal(S, ref_S), "padded no-op: final state changed"


def pin_continuation(orc, seed=15):
    """prefill(T) == prefill(m) followed by prefill(T - m) from the state at m (bit-exact)."""
    rng = np.random.default_rng(seed)
    B, Hk, Hv, T, d = 2, 1, 2, 40, 8
    q, k, v, g, beta, S0 = _rand_inputs(rng, B, Hk, Hv, T, d)
    full_o, full_S = orc.prefill(q, k, v, g, beta, S0, scale=0.3)
    for m in (1, 17, 31, T - 1):
        o1, S1 = orc.prefill(q[:, :, :m], k[:, :, :m], v[:, :, :m], g[:, :, :m], beta[:, :, :m], S0, scale=0.3)
        o2, S2 = orc.prefill(q[:, :, m:], k[:, :, m:], v[:, :, m:], g[:, :, m:], beta[:, :, m:], S1, scale=0.3)
        assert np.array_equal(np.concatenate([o1, o2], axis=2), full_o), ("continuation outputs", m)
        assert np.array_equal(S2, full_S), ("continuation state", m)


def pin_beta_zero(orc, seed=16):
    """beta = 0: o_t = exp(G_t) S_0 (scale q_t) and S_T = exp(G_T) S_0 with G_t = sum_{s<=t} g_s."""
    rng = np.random.default_rng(seed)
    B, Hk, Hv, T, d = 1, 2, 2, 30, 8
    q, k, v, g, beta, S0 = _rand_inputs(rng, B, Hk, Hv, T, d)
    beta[:] = 0.0
    o, S = orc.prefill(q, k, v, g, beta, S0, scale=0.7, head_map=TILED)
    G = np.cumsum(g.astype(np.float64), axis=-1)
    for h in range(Hv):
        kh = _kh(h, Hk, Hv, TILED)
        for t in range(T):
            expect = math.exp(G[0, h, t]) * (S0[0, h] @ (0.7 * q[0, kh, t].astype(np.float64)))
            assert _rel(o[0, h, t], expect) < 1e-13, ("beta=0 output", h, t)
        assert _rel(S[0, h], math.exp(G[0, h, -1]) * S0[0, h]) < 1e-13, ("beta=0 state", h)


def pin_recall(orc, seed=17):
    """beta = 1, g = 0 and orthonormal keys: after the scan S k_t = v_t for every written key,
    and columns of S_0 along unwritten directions survive. Exact for the unit basis."""
    rng = np.random.default_rng(seed)
    B, Hk, Hv, d = 1, 1, 2, 8
    T = 6
    q = rng.standard_normal((B, Hk, T, d)).astype(np.float32)
    v = rng.standard_normal((B, Hv, T, d)).astype(np.float32)
    g = np.zeros((B, Hv, T), np.float32)
    beta = np.ones((B, Hv, T), np.float32)
    S0 = rng.standard_normal((B, Hv, d, d))
    # unit basis vectors e_{perm[t]}: bit-exact recall
    perm = rng.permutation(d)[:T]
    k = np.zeros((B, Hk, T, d), np.float32)
    k[0, 0, np.arange(T), perm] = 1.0
    o, S = orc.prefill(q, k, v, g, beta, S0, scale=1.0)
    for h in range(Hv):
        for t in range(T):
            assert np.array_equal(S[0, h][:, perm[t]], v[0, h, t].astype(np.float64)), ("recall", h, t)
        rest = np.setdiff1d(np.arange(d), perm)
        assert np.array_equal(S[0, h][:, rest], S0[0, h][:, rest]), ("untouched columns", h)
    # a rotated orthonormal basis: recall up to rounding
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    k2 = np.zeros((B, Hk, T, d), np.float32)
    k2[0, 0] = Qm[:, :T].T.astype(np.float32)
    o, S = orc.prefill(q, k2, v, g, beta, S0, scale=1.0)
    # float32 keys are only orthonormal to ~1e-7, so recall holds to that accuracy
    for h in range(Hv):
        for t in range(T):
            got = S[0, h] @ k2[0, 0, t].astype(np.float64)
            assert _rel(got, v[0, h, t]) < 5e-6, ("rotated recall", h, t, _rel(got, v[0, h, t]))


def pin_scale_linear(orc, seed=18):
    """o(2 scale) = 2 o(scale) bit-exactly; the state does not depend on the scale."""
    rng = np.random.default_rng(seed)
    q, k, v, g, beta, S0 = _rand_inputs(rng, 1, 2, 4, 12, 8)
    o1, S1 = orc.prefill(q, k, v, g, beta, S0, scale=0.3)
    o2, S2 = orc.prefill(q, k, v, g, beta, S0, scale=0.6)
    assert np.array_equal(o2, 2.0 * o1), "scale linearity"
    assert np.array_equal(S1, S2), "state independent of scale"


def pin_head_map(orc, seed=19):
    """Tiled and grouped head maps differ only by a relabelling of the value heads."""
    rng = np.random.default_rng(seed)
    B, Hk, Hv, T, d = 2, 2, 6, 7, 4
    q, k, v, g, beta, S0 = _rand_inputs(rng, B, Hk, Hv, T, d)
    o_t, S_t = orc.prefill(q, k, v, g, beta, S0, scale=0.5, head_map=TILED)
    r = Hv // Hk
    # tiled value head h reads key head h % Hk; give it the grouped label kh * r + h // Hk
    perm = np.array([(h % Hk) * r + h // Hk for h in range(Hv)])
    vg, gg, bg, Sg = (np.empty_like(x) for x in (v, g, beta, S0))
    vg[:, perm], gg[:, perm], bg[:, perm], Sg[:, perm] = v, g, beta, S0
    o_g, S_g = orc.prefill(q, k, vg, gg, bg, Sg, scale=0.5, head_map=GROUPED)
    assert np.array_equal(o_g[:, perm], o_t), "head-map relabelling (outputs)"
    assert np.array_equal(S_g[:, perm], S_t), "head-map relabelling (states)"


def pin_threads(orc, seed=20):
    """One thread and many threads give bit-identical results."""
    rng = np.random.default_rng(seed)
    q, k, v, g, beta, S0 = _rand_inputs(rng, 2, 2, 4, 20, 16)
    o1, S1 = orc.prefill(q, k, v, g, beta, S0, scale=0.5, threads=1)
    o8, S8 = orc.prefill(q, k, v, g, beta, S0, scale=0.5, threads=8)
    assert np.array_equal(o1, o8) and np.array_equal(S1, S8), "thread-count invariance"


def pin_decode_matches_prefill(orc, seed=21):
    """T decode steps equal one prefill over the same T tokens (same float64 op sequence)."""
    rng = np.random.default_rng(seed)
    B, Hk, Hv, T, d = 2, 2, 4, 6, 8
    q, k, v, g, beta, S0 = _rand_inputs(rng, B, Hk, Hv, T, d)
    for head_map in (TILED, GROUPED):
        o_ref, S_ref = orc.prefill(q, k, v, g, beta, S0, scale=0.5, head_map=head_map)
        state = np.ascontiguousarray(S0.copy())
        for t in range(T):
            o = orc.decode_step(q[:, :, t], k[:, :, t], v[:, :, t], g[:, :, t], beta[:, :, t],
                                state, scale=0.5, head_map=head_map)
            assert np.array_equal(o, o_ref[:, :, t]), ("decode vs prefill output", head_map, t)
        assert np.array_equal(state, S_ref), ("decode vs prefill state", head_map)


def pin_pair_subset(orc, seed=22):
    """Computing a subset of (b, h) pairs gives the same rows as the full call."""
    rng = np.random.default_rng(seed)
    B, Hk, Hv, T, d = 2, 2, 4, 5, 8
    q, k, v, g, beta, S0 = _rand_inputs(rng, B, Hk, Hv, T, d)
    o, S = orc.prefill(q, k, v, g, beta, S0, scale=0.5, head_map=GROUPED)
    pairs = [7, 0, 5]
    op, Sp = orc.prefill(q, k, v, g, beta, S0, scale=0.5, head_map=GROUPED, pairs=pairs)
    for n, p in enumerate(pairs):
        assert np.array_equal(op[n], o[p // Hv, p % Hv]) and np.array_equal(Sp[n], S[p // Hv, p % Hv]), \
            ("pair subset", p)


# ---------------------------------------------------------------- gated RMSNorm epilogue
# The output epilogue of the gated delta kernels ("27b 935/47" page): y = x / sqrt(mean(x^2) +
# eps) * weight * silu(gate). Pinned by closed forms and exact invariants, and by sigmoid
# values quoted as constants (sigmoid(1) = 1 / (1 + 1/e) etc.).
_SIGMOID = {0.0: 0.5, 1.0: 0.7310585786300049, -1.0: 0.2689414213699951, 2.0: 0.8807970779778823,
            -3.0: 0.04742587317756678}


def pin_rmsnorm_unit_rms(orc, seed=23):
    """eps = 0, weight = 1, no gate: every output row has root-mean-square exactly 1, and
    doubling a row leaves its output unchanged bit for bit (powers of two scale exactly)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((5, 128)) * rng.uniform(0.1, 10.0, (5, 1))
    w = np.ones(128, np.float32)
    y = orc.gated_rmsnorm(x, w, eps=0.0)
    rms = np.sqrt(np.mean(y * y, axis=-1))
    assert np.max(np.abs(rms - 1.0)) < 1e-14, ("unit rms", rms)
    assert np.array_equal(orc.gated_rmsnorm(2.0 * x, w, eps=0.0), y), "scale invariance"
    assert np.all(np.sign(y) == np.sign(x)), "sign"


def pin_rmsnorm_eps(orc, seed=24):
    """weight = 1, no gate: mean(y^2) = m / (m + eps) with m = mean(x^2), for several eps."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((4, 64)) * 0.01
    m = np.mean(x * x, axis=-1)
    for eps in (1e-6, 1e-4, 3e-3):
        y = orc.gated_rmsnorm(x, np.ones(64, np.float32), eps=eps)
        got = np.mean(y * y, axis=-1)
        assert np.max(np.abs(got - m / (m + eps))) < 1e-13, ("eps", eps)


def pin_rmsnorm_gate_and_weight(orc, seed=25):
    """A constant row c (so the normalised value is c / sqrt(c^2 + eps)) times weight times
    silu(gate) = gate * sigmoid(gate), against quoted sigmoid values; weight acts per column,
    the same for every row, and rows are independent."""
    eps = 1e-6
    gates = np.array(sorted(_SIGMOID), dtype=np.float32)
    n = len(gates)
    c = np.array([0.5, -2.0, 3.0])
    x = np.repeat(c[:, None], n, axis=1)
    w = np.array([1.0, 2.0, -0.5, 4.0, 0.25][:n], np.float32)
    gate = np.tile(gates, (3, 1))
    y = orc.gated_rmsnorm(x, w, gate=gate, eps=eps)
    for r in range(3):
        for i, z in enumerate(gates):
            want = c[r] / math.sqrt(c[r] * c[r] + eps) * float(w[i]) * float(z) * _SIGMOID[float(z)]
            assert abs(y[r, i] - want) <= 1e-15 * max(1.0, abs(want)), ("gated value", r, i, y[r, i], want)
    rng = np.random.default_rng(seed)
    x2 = rng.standard_normal((6, 32))
    g2 = rng.standard_normal((6, 32)).astype(np.float32)
    w2 = rng.standard_normal(32).astype(np.float32)
    y2 = orc.gated_rmsnorm(x2, w2, gate=g2)
    perm = np.array([3, 0, 5, 1, 4, 2])
    assert np.array_equal(orc.gated_rmsnorm(x2[perm], w2, gate=g2[perm]), y2[perm]), "rows independent"
    w3 = np.full(32, 2.0, np.float32)
    y3 = orc.gated_rmsnorm(x2, w3, gate=g2)
    y1 = orc.gated_rmsnorm(x2, np.ones(32, np.float32), gate=g2)
    assert np.array_equal(y3, 2.0 * y1), "weight scales its column"


# ---------------------------------------------------------------- input prologue
# Causal depthwise convolution + SiLU and the q | k | v split with per-head L2 normalisation
# ("27b 935/47" page: causal_conv_silu and gdn_qkv tests).
def _silu_quoted(z):
    return z * _SIGMOID[float(z)]


def pin_prologue_taps(orc, seed=26):
    """Only the last tap set: y = silu(x) channel by channel (quoted sigmoid values), v heads
    unnormalised. Only the first tap set: y_t = silu(x_{t-3}), taking the state rows for t < 3."""
    Hk, Hv, d, K = 1, 2, 4, 4
    C = (2 * Hk + Hv) * d
    vals = np.array(sorted(_SIGMOID), dtype=np.float32)
    rng = np.random.default_rng(seed)
    x = rng.choice(vals, size=(1, 6, C)).astype(np.float32)
    w = np.zeros((C, K), np.float32)
    w[:, K - 1] = 1.0
    _, _, v, _ = orc.qkv_prologue(x, w, Hk, Hv, d, eps=0.0)
    for h in range(Hv):
        for t in range(6):
            for j in range(d):
                want = _silu_quoted(float(x[0, t, (2 * Hk + h) * d + j]))
                assert abs(v[0, h, t, j] - want) <= 1e-15 * max(1.0, abs(want)), ("last tap", h, t, j)
    w[:] = 0.0
    w[:, 0] = 1.0
    state = rng.choice(vals, size=(1, K - 1, C)).astype(np.float64)
    _, _, v, _ = orc.qkv_prologue(x, w, Hk, Hv, d, state=state, eps=0.0)
    for h in range(Hv):
        for t in range(6):
            for j in range(d):
                c = (2 * Hk + h) * d + j
                src = state[0, t, c] if t < K - 1 else x[0, t - (K - 1), c]
                want = _silu_quoted(float(src))
                assert abs(v[0, h, t, j] - want) <= 1e-15 * max(1.0, abs(want)), ("first tap", h, t, j)


def pin_prologue_continuation(orc, seed=27):
    """One call over T tokens equals a call over m tokens then one over T - m from the returned
    state, bit for bit; the returned state is the last K - 1 input rows."""
    rng = np.random.default_rng(seed)
    B, T, Hk, Hv, d, K = 2, 9, 2, 4, 8, 4
    C = (2 * Hk + Hv) * d
    x = rng.standard_normal((B, T, C)).astype(np.float32)
    w = rng.standard_normal((C, K)).astype(np.float32)
    s0 = rng.standard_normal((B, K - 1, C))
    q, k, v, st = orc.qkv_prologue(x, w, Hk, Hv, d, state=s0)
    assert np.array_equal(st, x[:, T - (K - 1):].astype(np.float64)), "state = last rows"
    for m in (1, 2, 5):
        q1, k1, v1, st1 = orc.qkv_prologue(x[:, :m], w, Hk, Hv, d, state=s0)
        q2, k2, v2, st2 = orc.qkv_prologue(x[:, m:], w, Hk, Hv, d, state=st1)
        for a_, b1, b2 in ((q, q1, q2), (k, k1, k2), (v, v1, v2)):
            assert np.array_equal(a_, np.concatenate([b1, b2], axis=2)), ("continuation", m)
        assert np.array_equal(st, st2), ("continued state", m)


def pin_prologue_norm_and_layout(orc, seed=28):
    """q and k heads are the v-style activations divided by their L2 norm: the same channel data
    placed in a q, a k and a v head gives q = k = v / |v| (eps = 0) and |q|^2 = s / (s + eps) with
    s = |v|^2 in general. A single nonzero channel lands in exactly its (tensor, head, t, j)."""
    rng = np.random.default_rng(seed)
    Hk, Hv, d, K, T = 1, 1, 16, 4, 5
    C = 3 * d
    head = rng.standard_normal((1, T, d)).astype(np.float32)
    x = np.concatenate([head, head, head], axis=-1)
    w = np.tile(rng.standard_normal((d, K)).astype(np.float32), (3, 1))
    q, k, v, _ = orc.qkv_prologue(x, w, Hk, Hv, d, eps=0.0)
    n = np.linalg.norm(v, axis=-1, keepdims=True)
    assert np.max(np.abs(q - v / n)) < 1e-15 and np.array_equal(q, k), "q, k = v / |v|"
    eps = 0.3
    q, _, v, _ = orc.qkv_prologue(x, w, Hk, Hv, d, eps=eps)
    s_ = np.sum(v * v, axis=-1)
    assert np.max(np.abs(np.sum(q * q, axis=-1) - s_ / (s_ + eps))) < 1e-14, "eps closed form"
    Hk, Hv, d = 2, 4, 4
    C = (2 * Hk + Hv) * d
    w = np.zeros((C, K), np.float32)
    w[:, K - 1] = 1.0
    for c, t in ((0, 0), (5, 3), (2 * d + 1, 1), (3 * d + 3, 4), (4 * d + 2, 2), (7 * d + 3, 0)):
        x = np.zeros((1, 5, C), np.float32)
        x[0, t, c] = 1.0
        q, k, v, _ = orc.qkv_prologue(x, w, Hk, Hv, d, eps=1e-300)  # eps > 0: all-zero heads stay 0
        hh, j = divmod(c, d)
        outs = {"q": q, "k": k, "v": v}
        name, h = ("q", hh) if hh < Hk else ("k", hh - Hk) if hh < 2 * Hk else ("v", hh - 2 * Hk)
        want = 1.0 if name != "v" else _SIGMOID[1.0]
        for nm, arr in outs.items():
            nz = np.argwhere(arr != 0.0)
            if nm == name:
                assert nz.tolist() == [[0, h, t, j]] and abs(arr[0, h, t, j] - want) < 1e-15, ("one-hot", c, t)
            else:
                assert nz.size == 0, ("leak", nm, c)


# ---------------------------------------------------------------- per-channel decay (KDA)
def _kda_g(rng, B, Hv, T, d):
    """One log-decay per key channel, -softplus(N(0, 1)) as for the scalar decay."""
    return (-np.log1p(np.exp(rng.standard_normal((B, Hv, T, d))))).astype(np.float32)


def pin_kda_uniform_is_gdn(orc, seed=29):
    """With every channel of g_t equal to one value, the per-channel recurrence is the gated
    delta rule: prefill and decode agree with the scalar-decay oracle to rounding."""
    rng = np.random.default_rng(seed)
    B, Hk, Hv, T, d = 2, 2, 4, 12, 6
    q, k, v, g, beta, S0 = _rand_inputs(rng, B, Hk, Hv, T, d)
    gc = np.repeat(g[..., None], d, axis=-1)
    for head_map in (TILED, GROUPED):
        o1, S1 = orc.prefill(q, k, v, g, beta, S0, scale=0.7, head_map=head_map)
        o2, S2 = orc.kda_prefill(q, k, v, gc, beta, S0, scale=0.7, head_map=head_map)
        assert _rel(o2, o1) < 1e-13 and _rel(S2, S1) < 1e-13, ("uniform decay", head_map)
        st1, st2 = S0.copy(), S0.copy()
        d1 = orc.decode_step(q[:, :, 0], k[:, :, 0], v[:, :, 0], g[:, :, 0], beta[:, :, 0], st1, scale=0.7,
                             head_map=head_map)
        d2 = orc.kda_decode_step(q[:, :, 0], k[:, :, 0], v[:, :, 0], gc[:, :, 0], beta[:, :, 0], st2, scale=0.7,
                                 head_map=head_map)
        assert _rel(d2, d1) < 1e-13 and _rel(st2, st1) < 1e-13, ("uniform decay decode", head_map)


def pin_kda_beta_zero(orc, seed=30):
    """beta = 0: S_t = S_0 diag(exp(G_t)) with G_t the running sum of g over tokens, per key
    channel (the decay scales the key columns), and o_t = S_t (scale q_t)."""
    rng = np.random.default_rng(seed)
    B, Hk, Hv, T, d = 1, 2, 4, 9, 5
    q, k, v, _, beta, S0 = _rand_inputs(rng, B, Hk, Hv, T, d)
    g = _kda_g(rng, B, Hv, T, d)
    beta = np.zeros_like(beta)
    o, S = orc.kda_prefill(q, k, v, g, beta, S0, scale=0.5)
    for h in range(Hv):
        kh = _kh(h, Hk, Hv, TILED)
        G = np.cumsum(g[0, h].astype(np.float64), axis=0)
        for t in range(T):
            St = S0[0, h] * np.exp(G[t])[None, :]
            assert _rel(o[0, h, t], St @ (0.5 * q[0, kh, t].astype(np.float64))) < 1e-13, ("beta=0 output", h, t)
        assert _rel(S[0, h], S0[0, h] * np.exp(G[-1])[None, :]) < 1e-13, ("beta=0 state", h)


def pin_kda_bruteforce_unroll(orc, seed=31):
    """S_t = S_0 P(1..t) + sum_s beta_s v_s k_s^T P(s+1..t) with A_t = diag(exp(g_t)) (I - beta_t
    k_t k_t^T): dense matrices in float64, the decay applied before the delta-rule erase."""
    rng = np.random.default_rng(seed)
    B, Hk, Hv, T, d = 1, 1, 2, 8, 5
    q, k, v, _, beta, S0 = _rand_inputs(rng, B, Hk, Hv, T, d)
    g = _kda_g(rng, B, Hv, T, d)
    o, S = orc.kda_prefill(q, k, v, g, beta, S0, scale=0.4)
    I = np.eye(d)
    for h in range(Hv):
        K = k[0, 0].astype(np.float64)
        A = [np.diag(np.exp(g[0, h, t].astype(np.float64))) @ (I - float(beta[0, h, t]) * np.outer(K[t], K[t]))
             for t in range(T)]
        for t in range(T):
            P = I.copy()
            for r in range(t + 1):
                P = P @ A[r]
            St = S0[0, h] @ P
            for s_ in range(t + 1):
                P = I.copy()
                for r in range(s_ + 1, t + 1):
                    P = P @ A[r]
                St = St + float(beta[0, h, s_]) * np.outer(v[0, h, s_].astype(np.float64), K[s_]) @ P
            assert _rel(o[0, h, t], St @ (0.4 * q[0, 0, t].astype(np.float64))) < 1e-12, ("kda unrolled", h, t)
            if t == T - 1:
                assert _rel(S[0, h], St) < 1e-12, ("kda unrolled state", h)


def pin_kda_channel_recall(orc, seed=32):
    """One-hot keys k_t = e_{j_t} with beta = 1: after step t column j_t of S holds v_t and every
    other column j has been multiplied by exp(g_t[j]) (recall with per-channel forgetting)."""
    rng = np.random.default_rng(seed)
    B, Hk, Hv, T, d = 1, 1, 2, 7, 6
    q, _, v, _, _, S0 = _rand_inputs(rng, B, Hk, Hv, T, d)
    g = _kda_g(rng, B, Hv, T, d)
    cols = rng.integers(0, d, size=T)
    k = np.zeros((B, Hk, T, d), dtype=np.float32)
    k[0, 0, np.arange(T), cols] = 1.0
    beta = np.ones((B, Hv, T), dtype=np.float32)
    for h in range(Hv):
        St = S0[0, h].copy()
        for t in range(T):
            _, S = orc.kda_prefill(q[:, :, :t + 1], k[:, :, :t + 1], v[:, :, :t + 1], g[:, :, :t + 1],
                                   beta[:, :, :t + 1], S0, scale=1.0)
            St = St * np.exp(g[0, h, t].astype(np.float64))[None, :]
            St[:, cols[t]] = v[0, h, t]
            assert _rel(S[0, h], St) < 1e-14, ("channel recall", h, t)


def pin_kda_continuation_and_decode(orc, seed=33):
    """A prefill split at any token continues bit for bit, and T decode steps equal the
    prefill's outputs and state bit for bit."""
    rng = np.random.default_rng(seed)
    B, Hk, Hv, T, d = 2, 1, 2, 9, 4
    q, k, v, _, beta, S0 = _rand_inputs(rng, B, Hk, Hv, T, d)
    g = _kda_g(rng, B, Hv, T, d)
    o, S = orc.kda_prefill(q, k, v, g, beta, S0, scale=0.6)
    for m in (1, 4, T - 1):
        o1, S1 = orc.kda_prefill(q[:, :, :m], k[:, :, :m], v[:, :, :m], g[:, :, :m], beta[:, :, :m], S0, scale=0.6)
        o2, S2 = orc.kda_prefill(q[:, :, m:], k[:, :, m:], v[:, :, m:], g[:, :, m:], beta[:, :, m:], S1, scale=0.6)
        assert np.array_equal(np.concatenate([o1, o2], axis=2), o) and np.array_equal(S2, S), ("split", m)
    st = S0.copy()
    for t in range(T):
        ot = orc.kda_decode_step(q[:, :, t], k[:, :, t], v[:, :, t], g[:, :, t], beta[:, :, t], st, scale=0.6)
        assert np.array_equal(ot, o[:, :, t]), ("decode output", t)
    assert np.array_equal(st, S), "decode state"


ALL_PINS = [pin_bruteforce_unroll, pin_exact_rational, pin_pages_one_step, pin_padded_noop,
            pin_continuation, pin_beta_zero, pin_recall, pin_scale_linear, pin_head_map,
            pin_threads, pin_decode_matches_prefill, pin_pair_subset,
            pin_rmsnorm_unit_rms, pin_rmsnorm_eps, pin_rmsnorm_gate_and_weight,
            pin_prologue_taps, pin_prologue_continuation, pin_prologue_norm_and_layout,
            pin_kda_uniform_is_gdn, pin_kda_beta_zero, pin_kda_bruteforce_unroll, pin_kda_channel_recall,
            pin_kda_continuation_and_decode]
