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
