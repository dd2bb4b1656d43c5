"""Pins of the oracle FWHT / RHT against Sylvester Hadamard matrices and identities.

glq 0.5.1 (PyPI project page), "How it works", item 2 (random sign flips, then a
fast Walsh-Hadamard transform).  scipy.linalg.hadamard builds the Sylvester
matrix by repeated Kronecker products, an independent construction.
"""
import numpy as np
import pytest
import scipy.linalg

from oracle import hadamard


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 64, 256, 1024, 4096])
def test_fwht_equals_sylvester_matrix(n):
    rng = np.random.default_rng(n)
    v = rng.standard_normal((3, n))
    H = scipy.linalg.hadamard(n).astype(np.float64)
    np.testing.assert_allclose(hadamard.fwht(v), v @ H.T, rtol=0, atol=1e-9 * np.sqrt(n))


def test_h2():
    assert hadamard.fwht(np.eye(2)).tolist() == [[1.0, 1.0], [1.0, -1.0]]


@pytest.mark.parametrize("n", [8, 32, 512])
def test_entries_follow_popcount_formula(n):
    H = hadamard.fwht(np.eye(n))        # row j = H e_j = column j (H symmetric)
    i = np.arange(n)
    pc = np.array([[bin(a & b).count("1") for b in i] for a in i])
    assert np.array_equal(H, (-1.0) ** pc)


@pytest.mark.parametrize("n", [8, 256, 2048, 4096])
def test_hht_is_n_identity(n):
    H = hadamard.fwht(np.eye(n))
    assert np.array_equal(H @ H.T, n * np.eye(n))


@pytest.mark.parametrize("n", [16384, 32768, 65536])
def test_involution_large(n):
    # H^2 = n I, checked on random vectors at the large padded sizes
    v = np.random.default_rng(1).standard_normal((2, n))
    np.testing.assert_allclose(hadamard.fwht(hadamard.fwht(v)), n * v, rtol=0, atol=1e-7 * n)


@pytest.mark.parametrize("n1,n2", [(2, 16384), (4, 8), (32, 1024), (64, 512)])
def test_kronecker_split(n1, n2):
    # H_{n1 n2} = H_{n1} (x) H_{n2}: index i = a * n2 + c; transform c, then a
    v = np.random.default_rng(n1).standard_normal(n1 * n2)
    two = hadamard.fwht(hadamard.fwht(v.reshape(n1, n2)).T).T.reshape(-1)
    np.testing.assert_allclose(two, hadamard.fwht(v), rtol=0, atol=1e-9 * n1 * n2)


def test_rht_preserves_norm_and_inverts():
    rng = np.random.default_rng(3)
    n, n_pad = 960, 1024
    x = rng.standard_normal((4, n))
    s = (2 * rng.integers(0, 2, n_pad) - 1).astype(np.int8)
    u = hadamard.rht_in(x, s, n_pad)
    np.testing.assert_allclose(np.linalg.norm(u, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    back = s * hadamard.fwht(u) / np.sqrt(n_pad)
    np.testing.assert_allclose(back[:, :n], x, atol=1e-12)
    np.testing.assert_allclose(back[:, n:], 0, atol=1e-12)


def test_rht_out_matches_dense():
    rng = np.random.default_rng(4)
    m, m_pad = 200, 256
    z = rng.standard_normal((3, m_pad))
    s = (2 * rng.integers(0, 2, m_pad) - 1).astype(np.int8)
    H = scipy.linalg.hadamard(m_pad).astype(np.float64)
    want = ((z @ H.T) * s / np.sqrt(m_pad))[:, :m]
    np.testing.assert_allclose(hadamard.rht_out(z, s, m), want, atol=1e-12)


def test_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        hadamard.fwht(np.zeros(12))
