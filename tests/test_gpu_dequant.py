"""GPU dequantization and codebook pack, bit-exact against the oracle.

glq 0.5.1, "How it works", item 1 (16-bit primary index, 8- or 16-bit residual),
table "Bit widths"; the fp32 rule is w = RN32(s * e) with e = c0 + s_r c1 exact,
fp16 / bf16 outputs round that fp32 value once more to nearest-even.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import e8, glq as og
from gpu_util import layer_from, say

pytestmark = pytest.mark.gpu
glq = pytest.importorskip("e8_lattice_codebook_amd")


def test_device_pack_holds_doubled_codebook(gpu_codebooks):
    want = (2 * e8.codebook()).astype(np.int8).reshape(-1)
    got = gpu_codebooks.primary.cpu().numpy().view(np.int8)[256:256 + 65536 * 8]
    assert np.array_equal(got, want)
    got8 = gpu_codebooks.resid8.cpu().numpy().view(np.int8)[256:256 + 256 * 8]
    assert np.array_equal(got8, want[:256 * 8])


def _check_layer(layer, codebooks, rows=None, dtypes=("f32", "f16", "bf16")):
    ql = glq.QuantizedLayer.from_synth(layer, codebooks)
    want32 = og.dequant_fp32(layer.idx0, layer.idx1, layer.resid_bits, layer.wscale, layer.resid_scale, rows=rows)
    for dt in dtypes:
        say("dequant", layer.m_pad, layer.n_pad, layer.resid_bits, dt)
        w = glq.e8_dequant(ql, {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dt])
        torch.cuda.synchronize()
        sel = w if rows is None else w[torch.as_tensor(rows, device=w.device)]
        if dt == "f32":
            got = sel.cpu().numpy()
            assert np.array_equal(got.view(np.uint32), want32.view(np.uint32))
        elif dt == "f16":
            got = sel.cpu().numpy()
            assert np.array_equal(got.view(np.uint16), want32.astype(np.float16).view(np.uint16))
        else:
            got = sel.view(torch.int16).cpu().numpy().view(np.uint16)
            assert np.array_equal(got, og.fp32_to_bf16_bits(want32))
        del w


@pytest.mark.parametrize("resid_bits", [0, 8, 16])
@pytest.mark.parametrize("n_pad,m_pad", [(8, 8), (64, 16), (256, 256), (1024, 40 * 0 + 512)])
def test_dequant_small(gpu_codebooks, resid_bits, n_pad, m_pad):
    layer = synth.random_layer(n_pad, m_pad, resid_bits, seed=n_pad + m_pad + resid_bits)
    _check_layer(layer, gpu_codebooks)


@pytest.mark.parametrize("key,k", [("tiny", 0), ("smollm2_up", 0), ("smollm3_block", 0), ("smollm3_block", 1),
                                   ("smollm3_block", 4), ("smollm3_block", 6), ("prefill_gateup", 0)])
def test_dequant_workloads_full(gpu_codebooks, key, k):
    _check_layer(layer_from(key, k), gpu_codebooks)


@pytest.mark.parametrize("k", [0, 2])
def test_dequant_devstral_sampled_rows(gpu_codebooks, k):
    # 32768 x 8192 and 8192 x 32768: the kernel writes all of W~; 3 row blocks
    # (first, a middle one, last) are compared bit for bit
    layer = layer_from("devstral_mlp", k)
    m = layer.m_pad
    rows = np.concatenate([np.arange(0, 64), np.arange(m // 2 - 37, m // 2 + 27), np.arange(m - 64, m)])
    _check_layer(layer, gpu_codebooks, rows=rows, dtypes=("f32", "bf16"))
