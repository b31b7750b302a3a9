"""Pins of the oracle's Hadamard rotation (paper notes, section 2.3, the Indexer excerpt: indexer queries and keys
are Hadamard-rotated before FP4 quantisation), checked against things other than its own formula: scipy's
Sylvester construction, hand-computed small cases, closed forms and the algebra of an orthonormal involution."""
import numpy as np
import pytest
import scipy.linalg

from oracle import oracle as orc


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128, 256, 1024])
def test_matches_scipy_sylvester_matrix(n):
    g = np.random.default_rng(n)
    x = g.standard_normal((3, n))
    ref = x @ scipy.linalg.hadamard(n).T / np.sqrt(n)
    np.testing.assert_allclose(orc.hadamard_rotate(x), ref, rtol=0, atol=1e-12 * np.sqrt(n))


def test_small_cases_by_hand():
    r2 = 1.0 / np.sqrt(2.0)
    np.testing.assert_allclose(orc.hadamard_rotate(np.array([3.0, 1.0])), [4.0 * r2, 2.0 * r2], atol=1e-15)
    # order 4: rows (1 1 1 1), (1 -1 1 -1), (1 1 -1 -1), (1 -1 -1 1), scaled by 1/2
    np.testing.assert_allclose(orc.hadamard_rotate(np.array([1.0, 2.0, 3.0, 4.0])), [5.0, -1.0, -2.0, 0.0],
                               atol=1e-15)


@pytest.mark.parametrize("n", [16, 128])
def test_closed_forms(n):
    e0 = np.zeros(n)
    e0[0] = 1.0
    np.testing.assert_allclose(orc.hadamard_rotate(e0), np.full(n, 1.0 / np.sqrt(n)), atol=1e-15)
    ones = np.ones(n)
    np.testing.assert_allclose(orc.hadamard_rotate(ones), np.sqrt(n) * e0, atol=1e-12)
    # e_j maps to the j-th Walsh function: signs (-1)^popcount(i & j)
    j = n // 2 + 3
    ej = np.zeros(n)
    ej[j] = 1.0
    signs = np.array([(-1.0) ** bin(i & j).count("1") for i in range(n)])
    np.testing.assert_allclose(orc.hadamard_rotate(ej), signs / np.sqrt(n), atol=1e-15)


def test_involution_and_dot_products():
    g = np.random.default_rng(7)
    q, k = g.standard_normal((2, 5, 128))
    Hq, Hk = orc.hadamard_rotate(q), orc.hadamard_rotate(k)
    np.testing.assert_allclose(orc.hadamard_rotate(Hq), q, atol=1e-12)  # H is symmetric and orthonormal
    np.testing.assert_allclose(np.sum(Hq * Hk, -1), np.sum(q * k, -1), atol=1e-11)
    np.testing.assert_allclose(np.linalg.norm(Hq, axis=-1), np.linalg.norm(q, axis=-1), atol=1e-12)


def test_rejects_non_power_of_two():
    with pytest.raises(AssertionError):
        orc.hadamard_rotate(np.ones(96))
