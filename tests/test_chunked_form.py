"""The chunked WY form that the prefill kernel implements equals the sequential oracle (CPU only)."""
import numpy as np
import pytest

from tests import chunked_model
from tests.oracle_pins import _rand_inputs


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / np.max(np.abs(b)))


@pytest.mark.parametrize("chunk", [4, 16, 64])
@pytest.mark.parametrize("head_map", [0, 1])
def test_chunked_equals_sequential(oracle_lib, chunk, head_map):
    rng = np.random.default_rng(100 + chunk)
    B, Hk, Hv, T, d = 2, 2, 4, 150, 16  # 150 is not a multiple of any chunk: ragged tail
    q, k, v, g, beta, S0 = _rand_inputs(rng, B, Hk, Hv, T, d)
    o_ref, S_ref = oracle_lib.prefill(q, k, v, g, beta, S0, scale=0.25, head_map=head_map)
    o, S = chunked_model.chunked_prefill(q, k, v, g, beta, S0, 0.25, chunk, head_map)
    assert _rel(o, o_ref) < 1e-12
    assert _rel(S, S_ref) < 1e-12


def test_chunked_short_sequence(oracle_lib):
    """T smaller than one chunk (the whole sequence is a masked tail)."""
    rng = np.random.default_rng(7)
    q, k, v, g, beta, S0 = _rand_inputs(rng, 1, 1, 2, 5, 8)
    o_ref, S_ref = oracle_lib.prefill(q, k, v, g, beta, S0, scale=0.5)
    o, S = chunked_model.chunked_prefill(q, k, v, g, beta, S0, 0.5, 64)
    assert _rel(o, o_ref) < 1e-12 and _rel(S, S_ref) < 1e-12


def test_inverse_unit_lower():
    rng = np.random.default_rng(3)
    for n in (1, 2, 16, 64):
        x = np.tril(rng.standard_normal((n, n)) * 0.3, -1)
        N = chunked_model.inverse_unit_lower(x)
        assert np.allclose((np.eye(n) - x) @ N, np.eye(n), atol=1e-13, rtol=0)
        assert np.array_equal(np.triu(N, 1), np.zeros((n, n))) and np.all(np.diag(N) == 1.0)


@pytest.mark.parametrize("P", [1, 2, 3, 5])
@pytest.mark.parametrize("chunk", [16, 32])
def test_segmented_equals_sequential(oracle_lib, P, chunk):
    """Segments run from starts chained through their affine maps S -> S M + N equal the
    sequential recurrence, outputs and final state, with a ragged last chunk."""
    rng = np.random.default_rng(200 + P + chunk)
    B, Hk, Hv, T, d = 1, 2, 4, 7 * chunk + 5, 8
    q, k, v, g, beta, S0 = _rand_inputs(rng, B, Hk, Hv, T, d)
    for head_map in (0, 1):
        o_ref, S_ref = oracle_lib.prefill(q, k, v, g, beta, S0, scale=0.3, head_map=head_map)
        o, S, starts = chunked_model.segmented_prefill(q, k, v, g, beta, S0, 0.3, chunk, P, head_map)
        assert _rel(o, o_ref) < 1e-11
        assert _rel(S, S_ref) < 1e-11
    # every segment start is the sequential state at that token (pinned against the oracle)
    for p, (c0, _) in enumerate(chunked_model.segment_bounds(T, chunk, P)):
        if c0 == 0:
            continue
        _, S_mid = oracle_lib.prefill(q[:, :, :c0 * chunk], k[:, :, :c0 * chunk], v[:, :, :c0 * chunk],
                                      g[:, :, :c0 * chunk], beta[:, :, :c0 * chunk], S0, scale=0.3, head_map=1)
        assert _rel(starts[:, :, p], S_mid) < 1e-11


def test_segment_map_of_identity_is_transition(oracle_lib):
    """The map M of a segment (identity rows, v = 0) is the product of the per-token transitions
    exp(g_t)(I - beta_t k_t k_t^T), built densely here."""
    rng = np.random.default_rng(9)
    q, k, v, g, beta, _ = _rand_inputs(rng, 1, 1, 1, 40, 6)
    M_dense = np.eye(6)
    for t in range(40):
        kt = k[0, 0, t].astype(np.float64)
        M_dense = M_dense @ (np.exp(float(g[0, 0, t])) * (np.eye(6) - float(beta[0, 0, t]) * np.outer(kt, kt)))
    S = np.eye(6)
    for t0 in range(0, 40, 16):
        Q, K, V, gc, bc, n = chunked_model._chunk((q, k, v, g, beta), 0, 0, 0, t0, 16)
        _, S = chunked_model.chunk_step(S, Q, K, np.zeros_like(V), gc, bc, 0.5)
    assert _rel(S, M_dense) < 1e-12


# ---- per-channel decay (KDA)

def _kda_inputs(rng, B, Hk, Hv, T, d, mult=1.0):
    q, k, v, _, beta, S0 = _rand_inputs(rng, B, Hk, Hv, T, d)
    g = -np.log1p(np.exp(rng.standard_normal((B, Hv, T, d)))) * mult
    return q, k, v, g.astype(np.float32), beta, S0


@pytest.mark.parametrize("chunk,factored", [(4, False), (16, False), (32, False), (16, True), (32, True), (64, True)])
def test_kda_chunked_equals_sequential(oracle_lib, chunk, factored):
    """The per-channel-decay WY form, with the blocks from pairwise decays or from the kernel's
    scaled tiles (references at tile boundaries and mid-tile), equals the sequential oracle."""
    rng = np.random.default_rng(200 + chunk)
    q, k, v, g, beta, S0 = _kda_inputs(rng, 2, 2, 4, 150, 16)  # ragged tail
    o_ref, S_ref = oracle_lib.kda_prefill(q, k, v, g, beta, S0, scale=0.25, head_map=1)
    o, S = chunked_model.kda_chunked_prefill(q, k, v, g, beta, S0, 0.25, chunk, head_map=1, factored=factored)
    assert _rel(o, o_ref) < 1e-12 and _rel(S, S_ref) < 1e-12


def test_kda_segmented_equals_sequential(oracle_lib):
    rng = np.random.default_rng(210)
    q, k, v, g, beta, S0 = _kda_inputs(rng, 1, 2, 4, 300, 16)
    o_ref, S_ref = oracle_lib.kda_prefill(q, k, v, g, beta, S0, scale=0.3)
    for P in (2, 3, 5):
        o, S = chunked_model.kda_chunked_prefill(q, k, v, g, beta, S0, 0.3, 32, factored=True, P=P)
        assert _rel(o, o_ref) < 1e-11 and _rel(S, S_ref) < 1e-11, P


def test_kda_factor_range():
    """With every log-decay >= KDA_G_MIN the diagonal tiles' factors stay within e^{+-80}
    (float32 range with margin); without the clamp a strong decay leaves it."""
    rng = np.random.default_rng(211)
    K = rng.standard_normal((32, 16)); Q = rng.standard_normal((32, 16)); bc = rng.random(32)
    g = -np.abs(rng.standard_normal((32, 16))) * 30.0  # up to ~-100 per step
    g[0, 0] = -1000.0
    _, _, big = chunked_model.kda_blocks_factored(Q, K, np.cumsum(g, axis=0), bc, 0.5)
    assert big > 80
    gcl = np.maximum(g, chunked_model.KDA_G_MIN)
    _, _, big = chunked_model.kda_blocks_factored(Q, K, np.cumsum(gcl, axis=0), bc, 0.5)
    assert big <= 8 * -chunked_model.KDA_G_MIN


def test_kda_clamp_is_within_bound(oracle_lib):
    """Strong decay (g x 10, steps below -10 common): the clamped chunked form stays within
    e^{-10} of the state's size from the exact recurrence, far inside the 2e-3 bar."""
    rng = np.random.default_rng(212)
    q, k, v, g, beta, S0 = _kda_inputs(rng, 1, 1, 2, 96, 16, mult=10.0)
    assert (g < chunked_model.KDA_G_MIN).mean() > 0.2
    o_ref, S_ref = oracle_lib.kda_prefill(q, k, v, g, beta, S0, scale=0.25)
    o, S = chunked_model.kda_chunked_prefill(q, k, v, g, beta, S0, 0.25, 32, factored=True, clamp=True)
    assert _rel(o, o_ref) < 1e-4 and _rel(S, S_ref) < 1e-4
