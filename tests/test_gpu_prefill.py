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
def test_fragment_order_path_equals_row_order(gpu_codebooks, M):
    # the linear's prefill steps (input transform into fragment order, matmul on it)
    # give bit for bit the matmul on the same fp16 u in row order
    layer = synth.random_layer(2000, 3000, 8, seed=M + 1, n_pad=2048, m_pad=4096)
    ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks)
    assert glq.e8_matmul_prefill_supported(ql)
    x = torch.randn(M, 2000, device=DEV, dtype=torch.bfloat16)
    uf = glq.input_rht_prefill(x, ql.n_pad, ql.sign_in)
    zf = glq.e8_matmul_prefill(ql, uf, M)
    u16 = glq.input_rht(x, ql.n_pad, ql.sign_in, torch.float16)
    zr = glq.e8_matmul(ql, u16)
    torch.cuda.synchronize()
    assert torch.equal(zf, zr)
