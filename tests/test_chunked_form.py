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
