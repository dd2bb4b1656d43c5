"""GPU parity of the 5-8 bpw layers (further residual stages) against the fp64 oracle.

glq 0.5.1, table "Bit widths": 5 to 8 bits per weight add a third and fourth
stage to the 16-bit primary and 16-bit residual stage (16+16+8, 16+16+16,
16+16+16+8, 16+16+16+16), each stage k scaled by s_k.  The library runs such a
layer as two passes shaped like 2-4 bpw layers whose partial outputs add, so
every matmul path is covered here: dequant (bit-exact fp32 rule
e = RN32(e + s_k c_k) stage by stage), the B = 1 two-launch path, the staged
B <= 16 path, the prefill kernel on the LDS codebook and the prefill kernel that
gathers from the int8 tables.  Slot-code layers must match index layers bit for
bit on every path.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import glq as og
from gpu_util import fragment_buffer, oracle_prefill_u16, rel_frob, same_products, say, to_f64, u16_as_f64

pytestmark = pytest.mark.gpu
glq = pytest.importorskip("e8_lattice_codebook_amd")
DEV = "cuda:0"
BPWS = [5, 6, 7, 8]


def _want32(layer):
    return og.dequant_fp32(layer.idx0, layer.idx1, layer.resid_bits, layer.wscale, layer.resid_scale,
                           extra=layer.oracle_extra())


@pytest.mark.parametrize("bpw", BPWS)
def test_dequant_recipe(gpu_codebooks, bpw):
    layer = synth.recipe_layer(1000, 700, bpw, seed=50 + bpw, n_pad=1024, m_pad=1024)
    ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks)
    want32 = _want32(layer)
    for q, name in ((ql, "index"), (ql.to_slot_codes(), "slot")):
        say("dequant recipe", bpw, name)
        w = glq.e8_dequant(q, torch.float32)
        w16 = glq.e8_dequant(q, torch.float16)
        torch.cuda.synchronize()
        assert np.array_equal(w.cpu().numpy().view(np.uint32), want32.view(np.uint32)), (bpw, name)
        assert np.array_equal(w16.cpu().numpy().view(np.uint16), want32.astype(np.float16).view(np.uint16))


def _oracle_linear(layer, x):
    return og.linear(x.to(torch.float64).cpu().numpy(), layer.sign_in, layer.sign_out, layer.n_pad, layer.m,
                     layer.idx0, layer.idx1, layer.resid_bits, layer.wscale, layer.resid_scale,
                     extra=layer.oracle_extra())


# (n, m, n_pad, m_pad, B): B = 1 two-launch path (full 64-lane rows, fewer lanes
# per row), B = 5 staged decode, B = 130 prefill (the shared-tile kernel for slot
# codes), B = 40 with n_pad 64 on the prefill kernel that gathers from the int8 tables
CASES = [(5120, 700, 8192, 1024, 1), (60, 3000, 64, 4096, 1), (3000, 2000, 4096, 2048, 5),
         (2000, 3000, 2048, 4096, 130), (60, 200, 64, 256, 40)]


@pytest.mark.parametrize("bpw", BPWS)
@pytest.mark.parametrize("n,m,n_pad,m_pad,B", CASES)
def test_linear_recipe(gpu_codebooks, bpw, n, m, n_pad, m_pad, B):
    layer = synth.recipe_layer(n, m, bpw, seed=7 * bpw + n + B, n_pad=n_pad, m_pad=m_pad)
    x = torch.from_numpy(np.random.default_rng(B + bpw).standard_normal((B, n)).astype(np.float32))
    x = x.to(torch.bfloat16)
    say("recipe linear", bpw, n, m, n_pad, m_pad, B)
    ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks)
    yi = glq.e8rht_linear(ql, x.to(DEV), torch.float32)
    ys = glq.e8rht_linear(ql.to_slot_codes(), x.to(DEV), torch.float32)
    torch.cuda.synchronize()
    assert same_products(yi, ys, B > 16 and n_pad >= 256)
    err = rel_frob(to_f64(yi), _oracle_linear(layer, x))
    say("  rel_frob", err)
    # the bounds of the 2-4 bpw paths: the extra stages only refine the weights
    assert err <= (1e-3 if B <= 16 else 5e-3), err


@pytest.mark.parametrize("bpw", BPWS)
@pytest.mark.parametrize("B", [1, 5, 16])
def test_decode_matmul_recipe(gpu_codebooks, bpw, B):
    layer = synth.recipe_layer(3000, 1500, bpw, seed=B * 10 + bpw, n_pad=4096, m_pad=2048)
    ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks)
    u = np.random.default_rng(B).standard_normal((B, layer.n_pad)).astype(np.float32)
    say("recipe matmul", bpw, B)
    parts = glq.e8_matmul(ql, torch.from_numpy(u).to(DEV))
    torch.cuda.synchronize()
    want = og.matmul_z(u.astype(np.float64), layer.idx0, layer.idx1, layer.resid_bits, layer.wscale,
                       layer.resid_scale, extra=layer.oracle_extra())
    # u rounded to 16-bit fixed point per 64 columns, as for 2-4 bpw: bound 1e-4
    assert rel_frob(to_f64(parts).sum(0), want) <= 1e-4


@pytest.mark.parametrize("bpw", BPWS)
def test_prefill_matmul_recipe(gpu_codebooks, bpw):
    # 2e of each pass (2c + s 2c' with s a power of two) is exact in fp16, so the
    # only rounding is the fp32 accumulation of the two passes: bound 1e-5
    layer = synth.recipe_layer(1000, 2000, bpw, seed=bpw, n_pad=1024, m_pad=2048)
    ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks)
    for M in (17, 300):
        say("recipe prefill matmul", bpw, M)
        u16 = np.random.default_rng(M).standard_normal((M, layer.n_pad)).astype(np.float16)
        z = glq.e8_matmul(ql, torch.from_numpy(u16).to(DEV))
        torch.cuda.synchronize()
        want = og.matmul_z(u16.astype(np.float64), layer.idx0, layer.idx1, layer.resid_bits, layer.wscale,
                           layer.resid_scale, extra=layer.oracle_extra())
        err = rel_frob(to_f64(z[0]), want)
        say("  rel_frob", err)
        assert err <= 1e-5, (M, err)
        # the linear's prefill steps for slot codes (fragment-order u, shared-tile
        # kernel, both passes) within fp32 accumulation of the oracle
        x = np.random.default_rng(M + 1).standard_normal((M, 1000))
        uq, e = oracle_prefill_u16(x, layer.sign_in, ql.n_pad)
        zf = glq.e8_matmul_prefill(ql.to_slot_codes(), fragment_buffer(uq, e, DEV), M)
        torch.cuda.synchronize()
        wf = og.matmul_z(u16_as_f64(uq, e), layer.idx0, layer.idx1, layer.resid_bits, layer.wscale,
                         layer.resid_scale, extra=layer.oracle_extra())
        assert rel_frob(to_f64(zf[0]), wf) <= 1e-5
