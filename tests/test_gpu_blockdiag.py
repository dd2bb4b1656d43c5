"""GPU parity of block-diagonal (unpadded) transforms and layers against the fp64 oracle.

glq 0.5.1, table "Bit widths" and the note below it: sizes that are not powers of
two use a block-diagonal transform (2688 = 2048 + 512 + 128) so that nothing is
padded.  A transform length that is a multiple of 64 but not a power of two is
transformed block by block over its binary expansion, largest block first, each
block orthonormal.  The matmul then runs over the unpadded K = n and m rows.

Tolerances are those of the padded layers: 1e-6 relative Frobenius for fp32
transforms, one rounding for fp16 / bf16 outputs, 1e-3 for the decode linear
(16-bit fixed-point activations) and 5e-3 for the fp16 MFMA prefill linear.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import glq as og, hadamard
from gpu_util import TORCH_DT, fragment_buffer, oracle_prefill_u16, rel_frob, same_products, say, to_f64, x_tensor

pytestmark = pytest.mark.gpu
glq = pytest.importorskip("e8_lattice_codebook_amd")
DEV = "cuda:0"
REL = {"f32": 1e-6, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}


# lengths: 4 blocks down to 64; the pages' 2688; 8192 + 2048 + 512 + 256; a block
# above 16384 (two-pass) with a small one; 16384 + 64
@pytest.mark.parametrize("n,B", [(960, 3), (2688, 1), (5120, 2), (11008, 5), (33792, 2), (16448, 1), (192, 4)])
@pytest.mark.parametrize("xdt,udt", [("f32", "f32"), ("bf16", "f32"), ("f16", "f16"), ("bf16", "bf16")])
def test_input_rht_blocks(n, B, xdt, udt):
    say("input_rht blocks", n, B, xdt, udt)
    x64, raw = synth.make_x(n, B, xdt, 91, n)
    sign = synth.block_layer(n, 64, 0, seed=n).sign_in
    u = glq.input_rht(x_tensor(raw, xdt, DEV), n, torch.from_numpy(sign).to(DEV), TORCH_DT[udt])
    torch.cuda.synchronize()
    want = hadamard.rht_in_blocks(x64, sign)
    assert u.shape == (B, n)
    assert rel_frob(to_f64(u), want) <= REL[udt]


def test_input_rht_blocks_padded():
    # x shorter than a block-diagonal n_pad: zero-padded into the last block
    n, n_pad = 2600, 2688
    x64, raw = synth.make_x(n, 2, "f32", 5, n)
    sign = synth.block_layer(n_pad, 64, 0, seed=1).sign_in
    u = glq.input_rht(x_tensor(raw, "f32", DEV), n_pad, torch.from_numpy(sign).to(DEV))
    torch.cuda.synchronize()
    xp = np.zeros((2, n_pad))
    xp[:, :n] = x64
    assert rel_frob(to_f64(u), hadamard.rht_in_blocks(xp, sign)) <= 1e-6


@pytest.mark.parametrize("m,m_pad,B,S", [(960, 960, 1, 1), (2688, 2688, 3, 2), (11008, 11008, 2, 5),
                                         (33792, 33792, 1, 3), (4160, 4160, 5, 8), (2600, 2688, 2, 1)])
@pytest.mark.parametrize("ydt", ["f32", "bf16"])
def test_output_rht_blocks(m, m_pad, B, S, ydt):
    say("output_rht blocks", m, m_pad, B, S, ydt)
    rng = np.random.default_rng(m + S)
    z = rng.standard_normal((S, B, m_pad)).astype(np.float32)
    sign = (2 * rng.integers(0, 2, m_pad) - 1).astype(np.int8)
    y = glq.output_rht(torch.from_numpy(z).to(DEV), m, torch.from_numpy(sign).to(DEV), TORCH_DT[ydt])
    torch.cuda.synchronize()
    want = hadamard.rht_out_blocks(z.astype(np.float64).sum(0), sign)[:, :m]
    assert y.shape == (B, m)
    assert rel_frob(to_f64(y), want) <= REL[ydt]


def _oracle(layer, x):
    return og.linear(x.to(torch.float64).cpu().numpy(), layer.sign_in, layer.sign_out, layer.n, layer.m,
                     layer.idx0, layer.idx1, layer.resid_bits, layer.wscale, layer.resid_scale,
                     extra=layer.oracle_extra(), block_diag=True)


# (n, m): input blocks 4096 + 1024; output blocks 2048 + 512; four output blocks
# (8192 + 2048 + 512 + 256) from one input block; four input blocks; blocks down
# to 64 on both sides; an output of 4096 + 64 (row blocks of 64 rows, a part-idle
# lane in the cross-block launch); a power of two (one block) on both sides
SHAPES = [(5120, 4096), (5120, 2560), (2048, 11008), (11008, 2048), (960, 2688), (1024, 4160), (2048, 2048)]


@pytest.mark.parametrize("resid_bits", [0, 8, 16])
@pytest.mark.parametrize("n,m", SHAPES)
@pytest.mark.parametrize("B", [1, 5, 130])
def test_linear_blocks(gpu_codebooks, resid_bits, n, m, B):
    layer = synth.block_layer(n, m, resid_bits, seed=n + m + B + resid_bits)
    x = torch.from_numpy(np.random.default_rng(B + n).standard_normal((B, n)).astype(np.float32))
    x = x.to(torch.bfloat16)
    say("block linear", n, m, B, resid_bits)
    ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks)
    y = glq.e8rht_linear(ql, x.to(DEV), torch.float32)
    ys = glq.e8rht_linear(ql.to_slot_codes(), x.to(DEV), torch.float32)
    torch.cuda.synchronize()
    assert y.shape == (B, m)
    assert same_products(y, ys, B > 16)
    err = rel_frob(to_f64(y), _oracle(layer, x))
    say("  rel_frob", err)
    assert err <= (1e-3 if B <= 16 else 5e-3), err


@pytest.mark.parametrize("B", [1, 16, 40])
def test_linear_blocks_small_and_fallback(gpu_codebooks, B):
    # n = 192 (128 + 64): one lane per row on the B = 1 path; the prefill
    # matmul takes the kernel that gathers from the int8 tables (n / 32 groups of
    # k-steps is not a multiple of 4)
    layer = synth.block_layer(192, 320, 8, seed=B)
    x = torch.from_numpy(np.random.default_rng(B).standard_normal((B, 192)).astype(np.float32))
    ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks)
    y = glq.e8rht_linear(ql, x.to(DEV), torch.float32)
    torch.cuda.synchronize()
    assert rel_frob(to_f64(y), _oracle(layer, x)) <= (1e-3 if B <= 16 else 5e-3)


@pytest.mark.parametrize("bpw", [5, 8])
@pytest.mark.parametrize("B", [1, 5, 130])
def test_linear_blocks_recipes(gpu_codebooks, bpw, B):
    resid_bits, extra_bits = synth.RECIPES[bpw]
    layer = synth.block_layer(2688, 2560, resid_bits, seed=bpw * 100 + B, extra_bits=extra_bits)
    x = torch.from_numpy(np.random.default_rng(B).standard_normal((B, 2688)).astype(np.float32)).to(torch.bfloat16)
    say("block recipe linear", bpw, B)
    ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks)
    y = glq.e8rht_linear(ql, x.to(DEV), torch.float32)
    ys = glq.e8rht_linear(ql.to_slot_codes(), x.to(DEV), torch.float32)
    torch.cuda.synchronize()
    assert same_products(y, ys, B > 16)
    assert rel_frob(to_f64(y), _oracle(layer, x)) <= (1e-3 if B <= 16 else 5e-3)


@pytest.mark.parametrize("B", [1, 5, 16])
def test_decode_matmul_unpadded_k(gpu_codebooks, B):
    layer = synth.block_layer(5120, 1536, 16, seed=B)
    ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks)
    u = np.random.default_rng(B).standard_normal((B, 5120)).astype(np.float32)
    parts = glq.e8_matmul(ql, torch.from_numpy(u).to(DEV))
    torch.cuda.synchronize()
    want = og.matmul_z(u.astype(np.float64), layer.idx0, layer.idx1, 16, layer.wscale, layer.resid_scale)
    assert rel_frob(to_f64(parts).sum(0), want) <= 1e-4


@pytest.mark.parametrize("M", [17, 300])
def test_prefill_fragment_order_unpadded(gpu_codebooks, M):
    # fragment order over K = 2688 (84 k-steps of 32, 21 index blocks): the
    # linear's prefill steps for slot codes and the row-order matmul on the same fp16
    # u are both within fp32 accumulation of the oracle
    layer = synth.block_layer(2688, 2560, 8, seed=M)
    ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks)
    qs = ql.to_slot_codes()
    assert glq.e8_matmul_prefill_supported(qs)
    x = np.random.default_rng(M).standard_normal((M, 2688))
    u16, e = oracle_prefill_u16(x, layer.sign_in, 2688)
    zf = glq.e8_matmul_prefill(qs, fragment_buffer(u16, e, DEV), M)
    zr = glq.e8_matmul(ql, torch.from_numpy(u16).to(DEV))
    torch.cuda.synchronize()
    want = og.matmul_z(u16.astype(np.float64), layer.idx0, layer.idx1, 8, layer.wscale, layer.resid_scale)
    sc = np.exp2(e)[:, None]
    assert rel_frob(to_f64(zf[0]), want * sc) <= 1e-5
    assert rel_frob(to_f64(zr[0]), want) <= 1e-5
