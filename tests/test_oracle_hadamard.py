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


# ---- block-diagonal transforms (glq 0.5.1, "Bit widths": non-power-of-two sizes
# split into power-of-two blocks, the example 2688 = 2048 + 512 + 128) -------------------
def test_block_split_of_the_pages_example():
    assert hadamard.pow2_blocks(2688) == [2048, 512, 128]


def test_block_split_is_the_binary_expansion():
    # distinct powers of two, largest first, summing to n: the unique such set
    for n in range(1, 5000):
        bl = hadamard.pow2_blocks(n)
        assert sum(bl) == n
        assert all(b & (b - 1) == 0 for b in bl)
        assert all(bl[i] > bl[i + 1] for i in range(len(bl) - 1))
    assert hadamard.pow2_blocks(4096) == [4096]
    assert hadamard.pow2_blocks(11008) == [8192, 2048, 512, 256]
    assert hadamard.pow2_blocks(5120) == [4096, 1024]


def dense_block_diag(n):
    bl = hadamard.pow2_blocks(n)
    return scipy.linalg.block_diag(*[scipy.linalg.hadamard(b).astype(np.float64) / np.sqrt(b) for b in bl])


@pytest.mark.parametrize("n", [1, 3, 7, 24, 100, 960])
def test_block_rht_matches_dense(n):
    rng = np.random.default_rng(n)
    x = rng.standard_normal((3, n))
    s_in = (2 * rng.integers(0, 2, size=n) - 1).astype(np.int8)
    D = dense_block_diag(n)
    np.testing.assert_allclose(hadamard.rht_in_blocks(x, s_in), (x * s_in) @ D.T, rtol=0, atol=1e-12)
    np.testing.assert_allclose(hadamard.rht_out_blocks(x, s_in), s_in * (x @ D.T), rtol=0, atol=1e-12)


@pytest.mark.parametrize("n", [64, 1024])
def test_block_rht_of_a_power_of_two_is_the_full_rht(n):
    rng = np.random.default_rng(n + 1)
    x = rng.standard_normal((2, n))
    s = (2 * rng.integers(0, 2, size=n) - 1).astype(np.int8)
    assert np.array_equal(hadamard.rht_in_blocks(x, s), hadamard.rht_in(x, s, n))
    assert np.array_equal(hadamard.rht_out_blocks(x, s), hadamard.rht_out(x, s, n))


def test_block_rht_orthonormal():
    rng = np.random.default_rng(7)
    n = 2688
    x = rng.standard_normal((2, n))
    s = (2 * rng.integers(0, 2, size=n) - 1).astype(np.int8)
    u = hadamard.rht_in_blocks(x, s)
    np.testing.assert_allclose(np.linalg.norm(u, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    # each orthonormal block is its own inverse: out(in(x)) with the same signs is x
    np.testing.assert_allclose(hadamard.rht_out_blocks(u, s), x, rtol=0, atol=1e-12)


def test_block_rht_rejects_wrong_sign_length():
    with pytest.raises(ValueError):
        hadamard.rht_in_blocks(np.zeros((1, 24)), np.ones(32, dtype=np.int8))
