"""Pins of the oracle's E8 codebook against facts fixed outside the oracle.

glq 0.5.1 (PyPI project page), "How it works", item 1; "Inference kernels"
(1 MB codebook).  Shell sizes come from the E8 theta series
1 + 240 sum_k sigma_3(k) q^(2k) (Conway & Sloane), computed here by divisor sums.
"""
import os

import numpy as np
import pytest

from oracle import e8

HERE = os.path.dirname(os.path.abspath(__file__))


def sigma3(k):
    return sum(d ** 3 for d in range(1, k + 1) if k % d == 0)


def theta_shell(norm2):
    return 1 if norm2 == 0 else 240 * sigma3(norm2 // 2)


def load_pins(name):
    rows = []
    with open(os.path.join(HERE, "golden", name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            p = line.split()
            rows.append((int(p[0]), [float(t) for t in p[1:]]))
    return rows


def test_size_and_fp16_bytes():
    bits = e8.codebook_fp16_bits()
    assert bits.shape == (65536, 8)
    assert bits.dtype == np.uint16
    assert bits.nbytes == 1 << 20          # the "1 MB" codebook


def test_membership_in_e8(oracle_codebook):
    t = 2 * oracle_codebook
    assert np.array_equal(t, np.round(t))
    t = t.astype(np.int64)
    parity = t % 2
    all_int = (parity == 0).all(1)
    all_half = (parity == 1).all(1)
    assert (all_int | all_half).all()
    # sum(v) even <=> sum(t) = 0 mod 4
    assert (t.sum(1) % 4 == 0).all()


def test_unique_entries(oracle_codebook):
    assert len(np.unique(oracle_codebook, axis=0)) == 65536


def test_shell_counts_match_theta_series(oracle_codebook):
    norm2 = np.round((oracle_codebook ** 2).sum(1)).astype(int)
    counts = {int(k): int(c) for k, c in zip(*np.unique(norm2, return_counts=True))}
    assert counts[2] == 240 and counts[4] == 2160          # stated shell sizes
    full = {k: theta_shell(k) for k in (0, 2, 4, 6, 8, 10)}
    for k, c in full.items():
        assert counts[k] == c
    assert sum(full.values()) == 56881
    assert counts[12] == 65536 - 56881
    assert set(counts) == {0, 2, 4, 6, 8, 10, 12}          # first seven shells


def test_enumerated_ball_is_complete():
    t = e8.e8_ball_doubled(12)
    norm2 = (t * t).sum(1) // 4
    for k in (0, 2, 4, 6, 8, 10, 12):
        assert int((norm2 == k).sum()) == theta_shell(k)


def test_minimum_distance_is_two(oracle_codebook):
    rng = np.random.default_rng(7)
    sel = oracle_codebook[rng.choice(65536, 3000, replace=False)]
    d2 = ((sel[:, None, :] - sel[None, :, :]) ** 2).sum(-1)
    d2 = d2[~np.eye(len(sel), dtype=bool)]
    assert d2.min() == 2.0
    # every nonzero point has norm^2 >= 2 (E8 minimal norm)
    n2 = (oracle_codebook[1:] ** 2).sum(1)
    assert n2.min() == 2.0


def test_hand_derived_index_pins(oracle_codebook):
    for idx, v in load_pins("e8_index_pins.txt"):
        assert oracle_codebook[idx].tolist() == v, idx


def test_full_shells_are_negation_symmetric(oracle_codebook):
    # a full shell is closed under v -> -v, which reverses lexicographic order
    start = 0
    for k in (0, 2, 4, 6, 8, 10):
        size = theta_shell(k)
        shell = oracle_codebook[start:start + size]
        assert np.array_equal(shell, -shell[::-1])
        start += size


def test_residual_8bit_table():
    r = e8.residual_codebook(8)
    assert r.shape == (256, 8)
    n2 = (r ** 2).sum(1)
    assert n2[0] == 0 and (n2[1:241] == 2).all() and (n2[241:] == 4).all()
    assert np.abs(r).max() == 2.0
    assert np.array_equal(e8.residual_codebook(16), e8.codebook())


def test_max_doubled_coordinate_is_six(oracle_codebook):
    assert np.abs(2 * oracle_codebook).max() == 6
