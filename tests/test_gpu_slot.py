"""GPU parity of layers whose 16-bit indices are relabelled as slot codes.

glq_slot_codes maps each codebook index to a slot code once, at load time; the
kernels then read a codeword from the slot image with one LDS access instead of
two.  The codewords, hence the integer dot products and fp16 MFMA operands, are
the same as with codebook indices, so every decode path must give bit for bit the
output of the index-format layer, which is itself checked against the fp64
oracle (glq 0.5.1, "How it works" items 1-4, "Inference kernels").  The prefill
of a slot-code layer runs the shared-tile kernel, whose fp32 sums run in another
order: within 1e-5 of the index-format output.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import glq as og
from gpu_util import rel_frob, same_products, say, to_f64

pytestmark = pytest.mark.gpu
glq = pytest.importorskip("e8_lattice_codebook_amd")
DEV = "cuda:0"
IMAGE_MAX = 39680


def code_of_table(codebooks):
    pack = codebooks.primary.cpu().numpy().view(np.uint8)
    img_off = (256 + 65536 * 8 + 255) // 256 * 256
    code_off = img_off + 2 * IMAGE_MAX * 4
    return pack[code_off:code_off + 65536 * 2].view(np.uint16)


def test_slot_codes_kernel(gpu_codebooks):
    code_of = code_of_table(gpu_codebooks)
    assert np.array_equal(np.sort(code_of), np.arange(65536))
    rng = np.random.default_rng(11)
    for count, off in [(65536, 0), (1000003, 0), (4097, 1), (7, 3), (0, 0)]:
        say("slot codes", count, off)
        idx = rng.integers(0, 65536, size=count + off, dtype=np.uint16)
        d = torch.from_numpy(idx.view(np.int16)).to(DEV)
        got = glq.slot_codes(d[off:], gpu_codebooks)
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy().view(np.uint16), code_of[idx[off:]])
    # in place
    idx = rng.integers(0, 65536, size=4096, dtype=np.uint16)
    d = torch.from_numpy(idx.view(np.int16)).to(DEV)
    glq.slot_codes(d, gpu_codebooks, out=d)
    torch.cuda.synchronize()
    assert np.array_equal(d.cpu().numpy().view(np.uint16), code_of[idx])


@pytest.mark.parametrize("resid_bits", [0, 8, 16])
def test_dequant_slot_layer(gpu_codebooks, resid_bits):
    layer = synth.random_layer(1024, 512, resid_bits, seed=40 + resid_bits)
    ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks)
    qs = ql.to_slot_codes()
    assert qs.index_format == glq.INDEX_SLOT
    ws = glq.e8_dequant(qs, torch.float32)
    torch.cuda.synchronize()
    want = og.dequant_fp32(layer.idx0, layer.idx1, resid_bits, layer.wscale, layer.resid_scale)
    assert np.array_equal(ws.cpu().numpy().view(np.uint32), want.view(np.uint32))


def _both(layer, codebooks, x, y_dtype=torch.float32):
    ql = glq.QuantizedLayer.from_synth(layer, codebooks)
    qs = ql.to_slot_codes()
    yi = glq.e8rht_linear(ql, x, y_dtype)
    ys = glq.e8rht_linear(qs, x, y_dtype)
    torch.cuda.synchronize()
    return yi, ys


def _oracle(layer, x):
    return og.linear(x.to(torch.float64).cpu().numpy(), layer.sign_in, layer.sign_out, layer.n_pad, layer.m,
                     layer.idx0, layer.idx1, layer.resid_bits, layer.wscale, layer.resid_scale)


# (n, m, n_pad, m_pad, B): B = 1 two-launch path (64 lanes per row, fewer, split
# counts 1..8), B = 5 staged decode, B = 130 prefill (the shared-tile kernel for
# slot codes), B = 40 with n_pad 64 on the prefill kernel that gathers from the
# int8 table (both formats)
CASES = [(5120, 700, 8192, 1024, 1), (32768, 64, 32768, 64, 1), (60, 3000, 64, 4096, 1), (100, 8000, 128, 8192, 1),
         (3000, 2000, 4096, 2048, 5), (2000, 3000, 2048, 4096, 130), (60, 200, 64, 256, 40)]


@pytest.mark.parametrize("resid_bits", [0, 8, 16])
@pytest.mark.parametrize("n,m,n_pad,m_pad,B", CASES)
def test_linear_slot_equals_index(gpu_codebooks, resid_bits, n, m, n_pad, m_pad, B):
    layer = synth.random_layer(n, m, resid_bits, seed=n + m + B + resid_bits, n_pad=n_pad, m_pad=m_pad)
    x = torch.from_numpy(np.random.default_rng(B).standard_normal((B, n)).astype(np.float32)).to(torch.bfloat16)
    say("slot linear", n, m, n_pad, m_pad, B, resid_bits)
    yi, ys = _both(layer, gpu_codebooks, x.to(DEV))
    assert same_products(yi, ys, B > 16 and n_pad >= 256)
    tol = 1e-3 if B <= 16 else 5e-3
    assert rel_frob(to_f64(ys), _oracle(layer, x)) <= tol


def test_linear_slot_bf16_output(gpu_codebooks):
    layer = synth.random_layer(5120, 3000, 16, seed=9, n_pad=8192, m_pad=4096)
    x = torch.randn(1, 5120, dtype=torch.bfloat16)
    yi, ys = _both(layer, gpu_codebooks, x.to(DEV), torch.bfloat16)
    assert torch.equal(yi.view(torch.int16), ys.view(torch.int16))
