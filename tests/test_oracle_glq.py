"""Pins of the oracle dequantizer and linear against independent forms.

glq 0.5.1 (PyPI project page): "How it works" items 1, 2, 4; table "Bit widths";
"Inference kernels" (Y = X dequant(W)^T, glq_dequant_matmul arguments).
The fused form is checked against the dense conjugated weight
W = (S_out H_m W~ H_n S_in / sqrt(n_pad m_pad))[:m, :n] built from
scipy.linalg.hadamard, an independent construction of the transforms.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg
import torch

import synth
from oracle import e8, glq, hadamard

HERE = os.path.dirname(os.path.abspath(__file__))


def dense_reference(x, layer):
    """y = x W^T with W the dense RHT-conjugated weight (independent construction)."""
    n, m, n_pad, m_pad = layer.n, layer.m, layer.n_pad, layer.m_pad
    c0 = e8.codebook()
    W = c0[layer.idx0.astype(np.int64)].reshape(m_pad, n_pad)
    if layer.resid_bits:
        c1 = e8.residual_codebook(layer.resid_bits)
        W = W + 0.25 * c1[layer.idx1.astype(np.int64)].reshape(m_pad, n_pad)
    W = float(np.float32(0.02)) * W       # the layer scale is an fp32 argument
    Hn = scipy.linalg.hadamard(n_pad).astype(np.float64)
    Hm = scipy.linalg.hadamard(m_pad).astype(np.float64)
    Wc = (np.diag(layer.sign_out.astype(np.float64)) @ Hm @ W @ Hn
          @ np.diag(layer.sign_in.astype(np.float64))) / np.sqrt(n_pad * m_pad)
    return x @ Wc[:m, :n].T


def oracle_linear(x, layer):
    return glq.linear(x, layer.sign_in, layer.sign_out, layer.n_pad, layer.m,
                      layer.idx0, layer.idx1, layer.resid_bits, layer.wscale, layer.resid_scale)


@pytest.mark.parametrize("resid_bits", [0, 8, 16])
@pytest.mark.parametrize("n,m,n_pad,m_pad", [(8, 8, 8, 8), (13, 40, 16, 64), (100, 70, 128, 128),
                                             (256, 200, 256, 256), (60, 256, 64, 256)])
def test_fused_equals_dense_conjugated(resid_bits, n, m, n_pad, m_pad):
    layer = synth.random_layer(n, m, resid_bits, seed=n * 1000 + m + resid_bits, n_pad=n_pad, m_pad=m_pad)
    x = np.random.default_rng(n + m).standard_normal((3, n))
    y = oracle_linear(x, layer)
    want = dense_reference(x, layer)
    assert y.shape == (3, m)
    np.testing.assert_allclose(y, want, rtol=0, atol=1e-12 * max(1.0, np.abs(want).max()))


def dense_block_reference(x, layer):
    """y = x W^T with W = S_out D_m W~ D_n S_in, D the block-diagonal orthonormal
    Hadamard matrix built from scipy.linalg.block_diag of scipy.linalg.hadamard."""
    n, m = layer.n, layer.m
    c0 = e8.codebook()
    W = c0[layer.idx0.astype(np.int64)].reshape(m, n)
    if layer.resid_bits:
        c1 = e8.residual_codebook(layer.resid_bits)
        W = W + 0.25 * c1[layer.idx1.astype(np.int64)].reshape(m, n)
    W = float(np.float32(0.02)) * W

    def D(k):
        return scipy.linalg.block_diag(*[scipy.linalg.hadamard(b).astype(np.float64) / np.sqrt(b)
                                         for b in hadamard.pow2_blocks(k)])
    Wc = np.diag(layer.sign_out.astype(np.float64)) @ D(m) @ W @ D(n) @ np.diag(layer.sign_in.astype(np.float64))
    return x @ Wc.T


@pytest.mark.parametrize("resid_bits", [0, 8, 16])
@pytest.mark.parametrize("n,m", [(24, 40), (8, 56), (96, 64), (200, 328)])
def test_block_diag_linear_equals_dense(resid_bits, n, m):
    layer = synth.block_layer(n, m, resid_bits, seed=n + 7 * m + resid_bits)
    assert layer.n_pad == n and layer.m_pad == m and layer.idx0.shape == (m, n // 8)
    x = np.random.default_rng(n * m).standard_normal((3, n))
    y = glq.linear(x, layer.sign_in, layer.sign_out, n, m, layer.idx0, layer.idx1, resid_bits,
                   layer.wscale, layer.resid_scale, block_diag=True)
    want = dense_block_reference(x, layer)
    np.testing.assert_allclose(y, want, rtol=0, atol=1e-12 * max(1.0, np.abs(want).max()))


def test_zero_indices_give_zero_output():
    layer = synth.random_layer(64, 64, 16, seed=5)
    layer.idx0[:] = 0
    layer.idx1[:] = 0
    x = np.random.default_rng(0).standard_normal((2, 64))
    assert np.array_equal(oracle_linear(x, layer), np.zeros((2, 64)))


def test_hand_computed_8x8():
    rows = []
    with open(os.path.join(HERE, "golden", "linear_8x8.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                p = line.split()
                rows.append((int(p[0]), [float(t) for t in p[1:]]))
    for s0, want in rows:
        sign_out = np.ones(8, dtype=np.int8)
        sign_out[0] = s0
        idx0 = np.ones((8, 1), dtype=np.uint16)
        x = np.zeros((1, 8))
        x[0, 0] = 1.0
        y = glq.linear(x, np.ones(8, np.int8), sign_out, 8, 8, idx0, None, 0, 0.02, 0.25)
        # s is the fp32 nearest to 0.02, a relative change of 4.5e-8
        np.testing.assert_allclose(y[0], want, rtol=1e-7, atol=1e-15)


def test_linearity():
    layer = synth.random_layer(96, 80, 8, seed=11)
    rng = np.random.default_rng(12)
    x1, x2 = rng.standard_normal((2, 96)), rng.standard_normal((2, 96))
    a, b = 0.7, -1.3
    lhs = oracle_linear(a * x1 + b * x2, layer)
    rhs = a * oracle_linear(x1, layer) + b * oracle_linear(x2, layer)
    np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-13)


def test_dequant_hand_group():
    # idx0 = 1 -> (-1,-1,0..), 16-bit residual idx1 = 241 -> (-2,0,..): e = (-1.5,-1,0,..)
    idx0 = np.array([[1]], dtype=np.uint16)
    idx1 = np.array([[241]], dtype=np.uint16)
    w = glq.dequant_rows(idx0, idx1, 16, 0.02, 0.25)
    s = float(np.float32(0.02))
    np.testing.assert_array_equal(w[0], np.array([-1.5, -1, 0, 0, 0, 0, 0, 0]) * s)
    # 8-bit residual idx1 = 242 -> (-1.5, -0.5 x6, 0.5)
    idx1 = np.array([[242]], dtype=np.uint8)
    w = glq.dequant_rows(idx0, idx1, 8, 0.02, 0.25)
    np.testing.assert_array_equal(w[0], np.array([-1.375, -1.125, -0.125, -0.125, -0.125, -0.125, -0.125, 0.125]) * s)


@pytest.mark.parametrize("resid_bits", [0, 8, 16])
def test_dequant_fp32_is_single_rounding_of_exact_value(resid_bits):
    layer = synth.random_layer(64, 16, resid_bits, seed=21)
    w32 = glq.dequant_fp32(layer.idx0, layer.idx1, resid_bits, 0.02, 0.25)
    c0 = e8.codebook()
    c1 = e8.residual_codebook(resid_bits) if resid_bits else None
    s = Fraction(float(np.float32(0.02)))
    rng = np.random.default_rng(1)
    for _ in range(200):
        o, k = int(rng.integers(16)), int(rng.integers(64))
        g, j = divmod(k, 8)
        e = Fraction(c0[layer.idx0[o, g]][j])
        if resid_bits:
            e += Fraction(1, 4) * Fraction(c1[layer.idx1[o, g]][j])
        exact = s * e
        # nearest fp32 to the exact rational, ties to even: compare with the two neighbours
        got = Fraction(float(w32[o, k]))
        up = Fraction(float(np.nextafter(w32[o, k], np.float32(np.inf))))
        dn = Fraction(float(np.nextafter(w32[o, k], np.float32(-np.inf))))
        assert abs(got - exact) <= abs(up - exact) and abs(got - exact) <= abs(dn - exact)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(2)
    v = (rng.standard_normal(10000) * 0.05).astype(np.float32)
    v[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]   # ties
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(glq.fp32_to_bf16_bits(v), want)


def test_matmul_row_blocks_agree():
    layer = synth.random_layer(256, 512, 16, seed=31)
    u = np.random.default_rng(3).standard_normal((2, 256))
    a = glq.matmul_z(u, layer.idx0, layer.idx1, 16, 0.02, 0.25, row_block=512)
    b = glq.matmul_z(u, layer.idx0, layer.idx1, 16, 0.02, 0.25, row_block=96)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_workload_shapes():
    w = synth.WORKLOADS
    assert [(l.n_pad, l.m_pad) for l in w["smollm3_block"].layers] == [
        (2048, 2048), (2048, 512), (2048, 512), (2048, 2048), (2048, 16384), (2048, 16384), (16384, 2048)]
    assert [(l.n_pad, l.m_pad) for l in w["devstral_mlp"].layers] == [(8192, 32768), (8192, 32768), (32768, 8192)]
    assert (w["smollm2_up"].layers[0].n_pad, w["smollm2_up"].layers[0].m_pad) == (1024, 4096)


# ---- 5-8 bpw: further residual stages ("Bit widths") ---------------------------------
def test_recipe_table_matches_bit_widths():
    # 16-bit primary + the stages' bits = 8 bpw bits per 8-weight group
    for bpw, (r, extra) in synth.RECIPES.items():
        assert 16 + r + sum(extra) == 8 * bpw
    assert synth.RECIPES[5] == (16, (8,)) and synth.RECIPES[7] == (16, (16, 8))


def test_dequant_hand_group_multistage():
    with open(os.path.join(HERE, "golden", "dequant_multistage_group.txt")) as f:
        rows = [line.split() for line in f if line.strip() and not line.startswith("#")]
    assert len(rows) == 4
    s = float(np.float32(0.02))
    for p in rows:
        bpw, idx = int(p[0]), p[1:5]
        want = np.array([float(t) for t in p[5:]])
        r, extra_bits = synth.RECIPES[bpw]
        i = lambda v, bits: np.array([[int(v)]], dtype=np.uint8 if bits == 8 else np.uint16)
        extra = [(i(idx[2 + j], b), b, 0.25 ** (j + 2)) for j, b in enumerate(extra_bits)]
        w = glq.dequant_rows(i(idx[0], 16), i(idx[1], r), r, 0.02, 0.25, extra=extra)
        np.testing.assert_array_equal(w[0], want * s)
        w32 = glq.dequant_fp32(i(idx[0], 16), i(idx[1], r), r, 0.02, 0.25, extra=extra)
        assert np.array_equal(w32[0], (want * s).astype(np.float32))


@pytest.mark.parametrize("bpw", [5, 6, 7, 8])
def test_dequant_fp32_multistage_single_rounding(bpw):
    layer = synth.recipe_layer(64, 16, bpw, seed=30 + bpw)
    ex = layer.oracle_extra()
    w32 = glq.dequant_fp32(layer.idx0, layer.idx1, layer.resid_bits, 0.02, 0.25, extra=ex)
    c0 = e8.codebook()
    s = Fraction(float(np.float32(0.02)))
    rng = np.random.default_rng(bpw)
    for _ in range(200):
        o, k = int(rng.integers(16)), int(rng.integers(64))
        g, j = divmod(k, 8)
        e = Fraction(c0[layer.idx0[o, g]][j]) + Fraction(1, 4) * Fraction(
            e8.residual_codebook(layer.resid_bits)[layer.idx1[o, g]][j])
        for st, (idx, bits, scale) in enumerate(ex):
            assert Fraction(scale) == Fraction(1, 4 ** (st + 2))
            e += Fraction(scale) * Fraction(e8.residual_codebook(bits)[idx[o, g]][j])
        exact = s * e
        got = Fraction(float(w32[o, k]))
        up = Fraction(float(np.nextafter(w32[o, k], np.float32(np.inf))))
        dn = Fraction(float(np.nextafter(w32[o, k], np.float32(-np.inf))))
        assert abs(got - exact) <= abs(up - exact) and abs(got - exact) <= abs(dn - exact)


@pytest.mark.parametrize("bpw", [5, 8])
def test_multistage_fused_equals_dense_conjugated(bpw):
    layer = synth.recipe_layer(100, 70, bpw, seed=40 + bpw, n_pad=128, m_pad=128)
    x = np.random.default_rng(bpw).standard_normal((3, 100))
    y = glq.linear(x, layer.sign_in, layer.sign_out, layer.n_pad, layer.m, layer.idx0, layer.idx1,
                   layer.resid_bits, layer.wscale, layer.resid_scale, extra=layer.oracle_extra())
    w = glq.dequant_rows(layer.idx0, layer.idx1, layer.resid_bits, layer.wscale, layer.resid_scale,
                         extra=layer.oracle_extra())
    h_n, h_m = scipy.linalg.hadamard(128), scipy.linalg.hadamard(128)
    dense = (np.diag(layer.sign_out.astype(float)) @ h_m @ w @ h_n @ np.diag(layer.sign_in.astype(float))
             / np.sqrt(128 * 128))[:70, :100]
    want = x @ dense.T
    np.testing.assert_allclose(y, want, rtol=0, atol=1e-12 * max(1.0, np.abs(want).max()))


def test_multistage_zero_indices_give_zero_output():
    layer = synth.recipe_layer(64, 64, 8, seed=5)
    layer.idx0[:] = 0
    layer.idx1[:] = 0
    for _, idx, _ in layer.extra:
        idx[:] = 0
    x = np.random.default_rng(0).standard_normal((2, 64))
    y = glq.linear(x, layer.sign_in, layer.sign_out, layer.n_pad, layer.m, layer.idx0, layer.idx1,
                   layer.resid_bits, layer.wscale, layer.resid_scale, extra=layer.oracle_extra())
    assert np.array_equal(y, np.zeros((2, 64)))
