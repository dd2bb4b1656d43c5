"""GPU parity of the prefill matmul (B > 16, fp16 MFMA against codeword
fragments dequantized from the LDS codebook) against the fp64 oracle.

glq 0.5.1, "Inference kernels" (Y = X dequant(W)^T on the matrix units without
forming W).  The matmul is called on its own with fp16 u, which the oracle takes
exactly; the dequantized weights 2e = 2c0 + s_r 2c1 are exact in fp16 for
s_r = 1/4, so the only rounding is the fp32 accumulation: the bound is a
relative Frobenius error of 1e-5.  The whole linear (fp16 u from the input
transform) keeps the 5e-3 prefill bound.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import glq as og
from gpu_util import rel_frob, say, to_f64

pytestmark = pytest.mark.gpu
glq = pytest.importorskip("e8_lattice_codebook_amd")
DEV = "cuda:0"

# (n, m, n_pad, m_pad): one 256-output tile, 8 tiles (the XCD-grouped tile order)
# and 16 tiles
SHAPES = [(256, 250, 256, 256), (1000, 2000, 1024, 2048), (2048, 4000, 2048, 4096)]


@pytest.mark.parametrize("resid_bits", [0, 8, 16])
@pytest.mark.parametrize("n,m,n_pad,m_pad", SHAPES)
def test_prefill_matmul(gpu_codebooks, resid_bits, n, m, n_pad, m_pad):
    layer = synth.random_layer(n, m, resid_bits, seed=3 * n + m + resid_bits, n_pad=n_pad, m_pad=m_pad)
    ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks)
    for M in (17, 130, 300):
        say("prefill matmul", n_pad, m_pad, resid_bits, M)
        u16 = np.random.default_rng(M).standard_normal((M, n_pad)).astype(np.float16)
        z = glq.e8_matmul(ql, torch.from_numpy(u16).to(DEV))
        torch.cuda.synchronize()
        assert z.shape == (1, M, m_pad)
        want = og.matmul_z(u16.astype(np.float64), layer.idx0, layer.idx1, resid_bits, layer.wscale,
                           layer.resid_scale)
        err = rel_frob(to_f64(z[0]), want)
        say("  rel_frob", err)
        assert err <= 1e-5, (M, err)


@pytest.mark.parametrize("M", [17, 257])
def test_prefill_linear(gpu_codebooks, M):
    n, m = 2000, 3000
    layer = synth.random_layer(n, m, 8, seed=M, n_pad=2048, m_pad=4096)
    ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks)
    x = torch.randn(M, n, dtype=torch.bfloat16)
    y = glq.e8rht_linear(ql, x.to(DEV), torch.float32)
    torch.cuda.synchronize()
    want = og.linear(x.to(torch.float64).numpy(), layer.sign_in, layer.sign_out, layer.n_pad, layer.m, layer.idx0,
                     layer.idx1, 8, layer.wscale, layer.resid_scale)
    assert rel_frob(to_f64(y), want) <= 5e-3


@pytest.mark.parametrize("M", [17, 300])
def test_fragment_order_path_matches_row_order(gpu_codebooks, M):
    # the linear's prefill steps (input transform into fragment order, then the
    # shared-tile matmul for slot codes or the per-wave matmul for codebook indices)
    # and the per-wave matmul on the same fp16 u in row order: the same exact
    # products, summed in other orders (fp32), all within 1e-5 of the oracle; the
    # per-wave kernel gives the same bits on either order of u
    layer = synth.random_layer(2000, 3000, 8, seed=M + 1, n_pad=2048, m_pad=4096)
    ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks)
    qs = ql.to_slot_codes()
    assert glq.e8_matmul_prefill_supported(qs) and glq.e8_matmul_prefill_supported(ql)
    x = torch.randn(M, 2000, device=DEV, dtype=torch.bfloat16)
    uf = glq.input_rht_prefill(x, ql.n_pad, ql.sign_in)
    zs = glq.e8_matmul_prefill(qs, uf, M)
    zi = glq.e8_matmul_prefill(ql, uf, M)
    u16 = glq.input_rht(x, ql.n_pad, ql.sign_in, torch.float16)
    zr = glq.e8_matmul(ql, u16)
    torch.cuda.synchronize()
    assert torch.equal(zi, zr)
    want = og.matmul_z(to_f64(u16), layer.idx0, layer.idx1, 8, layer.wscale, layer.resid_scale)
    assert rel_frob(to_f64(zs[0]), want) <= 1e-5
    assert rel_frob(to_f64(zr[0]), want) <= 1e-5


# Slot-code layers at many tiles per compute unit (m_pad 8192: 32 output tiles of
# 256; M = 1000 gives 8 token tiles of 128, the last with 104 tokens and a token
# block of 8; M = 2049 gives 17, the last with one token).
@pytest.mark.parametrize("resid_bits", [0, 8, 16])
@pytest.mark.parametrize("M", [1000, 2049])
def test_prefill_large_slot_codes(gpu_codebooks, resid_bits, M):
    layer = synth.random_layer(1000, 8000, resid_bits, seed=M + resid_bits, n_pad=1024, m_pad=8192)
    ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks)
    qs = ql.to_slot_codes()
    x = torch.from_numpy(np.random.default_rng(M).standard_normal((M, 1000)).astype(np.float32)).to(DEV)
    say("prefill large", resid_bits, M)
    uf = glq.input_rht_prefill(x, 1024, ql.sign_in)
    zw = glq.e8_matmul_prefill(qs, uf, M)
    u16 = glq.input_rht(x, 1024, ql.sign_in, torch.float16)
    torch.cuda.synchronize()
    want = og.matmul_z(to_f64(u16), layer.idx0, layer.idx1, resid_bits, layer.wscale, layer.resid_scale)
    err = rel_frob(to_f64(zw[0]), want)
    say("  rel_frob", err)
    assert err <= 1e-5, err
    # repeat calls are bit-identical; the whole linear keeps the prefill bound
    assert torch.equal(glq.e8_matmul_prefill(qs, uf, M), zw)
    y = glq.e8rht_linear(qs, x, torch.float32)
    torch.cuda.synchronize()
    wy = og.linear(x.double().cpu().numpy(), layer.sign_in, layer.sign_out, 1024, 8000, layer.idx0, layer.idx1,
                   resid_bits, layer.wscale, layer.resid_scale)
    assert rel_frob(to_f64(y), wy) <= 5e-3


@pytest.mark.parametrize("bpw", [5, 8])
def test_prefill_large_slot_codes_recipes(gpu_codebooks, bpw):
    # 5-8 bpw: the second pass adds its partial products to z
    resid_bits, extra_bits = synth.RECIPES[bpw]
    layer = synth.random_layer(1024, 8192, resid_bits, seed=bpw, n_pad=1024, m_pad=8192, extra_bits=extra_bits)
    qs = glq.QuantizedLayer.from_synth(layer, gpu_codebooks).to_slot_codes()
    x = torch.from_numpy(np.random.default_rng(bpw).standard_normal((1000, 1024)).astype(np.float32)).to(DEV)
    y = glq.e8rht_linear(qs, x, torch.float32)
    torch.cuda.synchronize()
    want = og.linear(x.double().cpu().numpy(), layer.sign_in, layer.sign_out, 1024, 8192, layer.idx0, layer.idx1,
                     resid_bits, layer.wscale, layer.resid_scale, extra=layer.oracle_extra())
    assert rel_frob(to_f64(y), want) <= 5e-3


@pytest.mark.parametrize("M,n,n_pad", [(33, 2000, 2048), (5, 2600, 2688)])
def test_fragment_order_layout(M, n, n_pad):
    # the documented placement of element (b, i): group g = i / 8, k-step
    # ks = 4 (g / 16) + g % 4, quarter q = (g / 4) % 4, half index
    # (((b / 16) KS + ks) 4 + q) 128 + (b % 16) 8 + i % 8 with KS = n_pad / 32; rows
    # past M are not compared
    sign = synth.random_layer(n, 256, 0, seed=M, n_pad=n_pad, m_pad=256).sign_in
    x = torch.randn(M, n, device=DEV, dtype=torch.bfloat16)
    st = torch.from_numpy(sign).to(DEV)
    uf = glq.input_rht_prefill(x, n_pad, st).view(torch.float16).cpu().numpy()
    u = glq.input_rht(x, n_pad, st, torch.float16).cpu().numpy()
    KS = n_pad // 32
    b, i = np.meshgrid(np.arange(M), np.arange(n_pad), indexing="ij")
    g = i // 8
    ks, q = 4 * (g // 16) + g % 4, (g // 4) % 4
    pos = (((b // 16) * KS + ks) * 4 + q) * 128 + (b % 16) * 8 + i % 8
    assert np.array_equal(uf[pos].view(np.uint16), u.view(np.uint16))
