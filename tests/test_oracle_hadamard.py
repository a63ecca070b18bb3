"""Pins of the oracle's Walsh-Hadamard transform (CPU only).

Sylvester Hadamard matrix: deterministic, self-inverse up to d, needs no
storage (PolarQuant page, Technical summary sec. 2 and sec. 3)."""
import numpy as np
import pytest

import oracle as O


def sylvester(n):
    """Independent construction: H_1 = [1], H_2n = [[H, H], [H, -H]]."""
    H = np.ones((1, 1), dtype=np.int64)
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


@pytest.mark.parametrize("n", [2, 4, 8, 16, 32, 64, 128])
def test_orthogonality_exact(n):
    H = O.hadamard_matrix(n)
    assert np.array_equal(H @ H.T, n * np.eye(n, dtype=np.int64))
    assert np.array_equal(H, H.T)
    assert np.array_equal(H, sylvester(n))


def test_fwht_equals_dense_and_is_self_inverse():
    rng = np.random.default_rng(11)
    for n in (8, 128):
        xi = rng.integers(-50, 50, n).astype(np.float64)  # exact in fp64
        assert np.array_equal(O.fwht(xi), O.hadamard_dense(xi))
        assert np.array_equal(O.fwht(xi), sylvester(n) @ xi)
        x = rng.standard_normal(n)
        np.testing.assert_allclose(O.fwht(x), sylvester(n) @ x, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(O.fwht(O.fwht(x)), n * x, rtol=1e-12, atol=1e-12)


def test_norm_preservation_with_random_signs():
    rng = np.random.default_rng(3)
    u = rng.standard_normal(128)
    u /= np.linalg.norm(u)
    D = np.where(rng.integers(0, 2, 128) == 1, 1.0, -1.0)
    y = O.fwht(D * u)
    assert abs(np.linalg.norm(y) - np.sqrt(128.0)) < 1e-12
    # rotating then de-rotating (H is its own inverse up to d) is the identity
    back = D * O.fwht(y) / 128.0
    np.testing.assert_allclose(back, u, atol=1e-14)
