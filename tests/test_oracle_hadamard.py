"""Pins of the oracle's Walsh-Hadamard transform (H_B of Eq. 8 and Eq. 12 in the
TACO paper, section 4.2.2: orthogonal after the 1/sqrt(B) factor, symmetric,
applied as an in-place FWHT).

Pinned against: hand-written Sylvester matrices (tests/golden), scipy's
``linalg.hadamard`` (a library routine, Sylvester construction), the closed
forms H H^T = n I and H = H^T, and Parseval's identity.
"""
import numpy as np
import pytest
from scipy.linalg import hadamard

from conftest import read_golden

SIZES = [2, 4, 8, 16, 32, 64, 128, 256, 512]


def dense_from_fwht(oracle_mod, n):
    """Columns of H obtained by transforming the basis vectors."""
    return oracle_mod.fwht(np.eye(n)).T      # row j of FWHT(I) = H e_j = column j


def test_matches_handwritten_sylvester(oracle_mod):
    rows = read_golden("hadamard_sylvester.txt")
    i = 0
    while i < len(rows):
        assert rows[i][0] == "n"
        n = int(rows[i][1])
        want = np.array([[float(v) for v in r] for r in rows[i + 1:i + 1 + n]])
        assert np.array_equal(dense_from_fwht(oracle_mod, n), want), n
        i += 1 + n


@pytest.mark.parametrize("n", SIZES)
def test_matches_scipy_and_is_orthogonal(oracle_mod, n):
    H = dense_from_fwht(oracle_mod, n)
    assert np.array_equal(H, hadamard(n).astype(np.float64))
    assert np.array_equal(H, H.T)
    assert np.array_equal(H @ H.T, n * np.eye(n))


@pytest.mark.parametrize("n", SIZES)
def test_fwht_equals_dense_product_and_parseval(oracle_mod, n):
    rng = np.random.default_rng(n)
    v = rng.standard_normal((16, n))
    got = oracle_mod.fwht(v)
    want = v @ hadamard(n).astype(np.float64).T
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12 * n)
    np.testing.assert_allclose((got ** 2).sum(1), n * (v ** 2).sum(1), rtol=1e-12)
    # Applying it twice multiplies by n (H^-1 = H / n).
    np.testing.assert_allclose(oracle_mod.fwht(got), n * v, rtol=0, atol=1e-10 * n)
