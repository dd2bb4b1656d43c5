"""Pins of the E8 KV-cache decode attention oracle (oracle/kv.py).

Glq v0.5.0 release notes, "Highlights": compressed K/V expanded inside the
attention tile loop, a length-8 Hadamard transform inverting the rotation;
glq 0.5.1, "KV cache compression" (E8 lattice cache, the e8_relaxed:2 recipe).
Each pin holds independently of the oracle's own code: hand-derived groups, the
scipy Hadamard matrix, closed forms of softmax attention (one token, equal
scores, the hard-max limit) and invariances (page placement, grouped heads).
"""
import os

import numpy as np
import pytest
import scipy.linalg

import synth
from oracle import e8, kv

HERE = os.path.dirname(os.path.abspath(__file__))


def test_h8_is_the_orthonormal_sylvester_matrix():
    H = kv.h8_normalized()
    np.testing.assert_allclose(H, scipy.linalg.hadamard(8) / np.sqrt(8.0), rtol=0, atol=1e-15)
    np.testing.assert_allclose(H @ H.T, np.eye(8), rtol=0, atol=1e-14)


def golden_groups():
    rows = []
    for line in open(os.path.join(HERE, "golden", "kv_dequant_groups.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        left, right = line.split("|")
        st, i0, i1 = left.split()
        rows.append((int(st), int(i0), None if i1 == "-" else int(i1), np.array([float(v) for v in right.split()])))
    return rows


def test_hand_derived_groups():
    rows = golden_groups()
    assert len(rows) == 3
    for stages, i0, i1, h8e in rows:
        s = np.float32(1.75)
        idx0 = np.array([[i0]], dtype=np.uint16)
        idx1 = None if stages == 1 else np.array([[i1]], dtype=np.uint16)
        x = kv.dequant_vectors(idx0, idx1, np.array([s]), 0.25)
        np.testing.assert_allclose(x[0], float(s) * h8e / np.sqrt(8.0), rtol=0, atol=1e-14)


def test_dequant_vector_norm_is_the_codeword_norm():
    # H8 / sqrt(8) is orthonormal: |x_g| = s |e_g| group by group
    rng = np.random.default_rng(4)
    idx0 = rng.integers(0, 65536, size=(5, 16), dtype=np.uint16)
    idx1 = rng.integers(0, 65536, size=(5, 16), dtype=np.uint16)
    s = rng.uniform(0.5, 2, size=5)
    x = kv.dequant_vectors(idx0, idx1, s, 0.25).reshape(5, 16, 8)
    c = e8.codebook()
    e = c[idx0.astype(np.int64)] + 0.25 * c[idx1.astype(np.int64)]
    np.testing.assert_allclose(np.linalg.norm(x, axis=-1), s[:, None] * np.linalg.norm(e, axis=-1), rtol=1e-13)


def _attn(cache, q, sm_scale=None):
    D = cache.head_dim
    return kv.attention_decode(q, cache.k_idx0, cache.k_idx1, cache.k_scale, cache.v_idx0, cache.v_idx1,
                               cache.v_scale, cache.resid_scale, cache.block_table, cache.seq_lens,
                               cache.page_size, 1.0 / np.sqrt(D) if sm_scale is None else sm_scale)


def _v_of(cache, b, h, t):
    page = cache.block_table[b][t // cache.page_size]
    slot = t % cache.page_size
    i1 = None if cache.v_idx1 is None else cache.v_idx1[page, slot, h][None]
    return kv.dequant_vectors(cache.v_idx0[page, slot, h][None], i1, cache.v_scale[page, slot, h][None],
                              cache.resid_scale)[0]


@pytest.mark.parametrize("stages", [1, 2])
def test_one_token_returns_its_value(stages):
    cache = synth.make_kv([1, 1], 2, 64, stages, 16, seed=stages)
    q, _ = synth.make_q(2, 4, 64, "f32", 1)
    out = _attn(cache, q)
    for b in range(2):
        for hq in range(4):
            np.testing.assert_allclose(out[b, hq], _v_of(cache, b, hq // 2, 0), rtol=0, atol=1e-13)


def test_zero_query_averages_the_values():
    cache = synth.make_kv([37], 1, 64, 2, 16, seed=5)
    out = _attn(cache, np.zeros((1, 1, 64)))
    want = np.mean([_v_of(cache, 0, 0, t) for t in range(37)], axis=0)
    np.testing.assert_allclose(out[0, 0], want, rtol=0, atol=1e-13)


def test_hard_max_limit_picks_the_best_key():
    # sm_scale -> infinity: softmax -> one-hot at argmax_t q . K_t
    cache = synth.make_kv([50], 1, 64, 2, 16, seed=6)
    q, _ = synth.make_q(1, 1, 64, "f32", 2)
    keys = []
    for t in range(50):
        page = cache.block_table[0][t // 16]
        keys.append(kv.dequant_vectors(cache.k_idx0[page, t % 16, 0][None], cache.k_idx1[page, t % 16, 0][None],
                                       cache.k_scale[page, t % 16, 0][None], 0.25)[0])
    sc = np.array(keys) @ q[0, 0]
    order = np.argsort(sc)
    assert sc[order[-1]] - sc[order[-2]] > 1e-3     # a unique maximum for this seed
    out = _attn(cache, q, sm_scale=1e6)
    np.testing.assert_allclose(out[0, 0], _v_of(cache, 0, 0, int(order[-1])), rtol=0, atol=1e-12)


def test_page_placement_does_not_matter():
    # the same logical tokens in other physical pages give the same output
    cache = synth.make_kv([40, 23], 2, 64, 2, 8, seed=7)
    q, _ = synth.make_q(2, 4, 64, "f32", 3)
    out = _attn(cache, q)
    perm = np.random.default_rng(0).permutation(cache.pages)
    moved = synth.KVCache(cache.num_kv_heads, cache.head_dim, cache.page_size, cache.stages,
                          np.empty_like(cache.k_idx0), np.empty_like(cache.k_idx1),
                          np.empty_like(cache.v_idx0), np.empty_like(cache.v_idx1),
                          np.empty_like(cache.k_scale), np.empty_like(cache.v_scale),
                          perm[cache.block_table].astype(np.int32), cache.seq_lens)
    for name in ("k_idx0", "k_idx1", "v_idx0", "v_idx1", "k_scale", "v_scale"):
        getattr(moved, name)[perm] = getattr(cache, name)
    assert np.array_equal(_attn(moved, q), out)


def test_grouped_heads_equal_repeated_kv_heads():
    # 4 query heads on 2 KV heads = 4 query heads on 4 KV heads holding each KV head twice
    cache = synth.make_kv([30], 2, 64, 1, 16, seed=8)
    q, _ = synth.make_q(1, 4, 64, "f32", 4)
    rep = lambda a: None if a is None else np.repeat(a, 2, axis=2)
    wide = synth.KVCache(4, 64, 16, 1, rep(cache.k_idx0), None, rep(cache.v_idx0), None, rep(cache.k_scale),
                         rep(cache.v_scale), cache.block_table, cache.seq_lens)
    np.testing.assert_allclose(_attn(cache, q), _attn(wide, q), rtol=0, atol=1e-14)
