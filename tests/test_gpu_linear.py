"""GPU parity of the E8RHTLinear forward and of the decode matmul against the
fp64 oracle (dequantize-then-matmul between the two transforms).

glq 0.5.1, "How it works" and "Inference kernels" (Y = X dequant(W)^T without
forming W; split-K with a fixed-order reduction).  Tolerances: relative
Frobenius error of fp32 y over all [B, m] <= 1e-3 for the decode path (fp32
accumulation) and <= 5e-3 for the prefill path (fp16 MFMA operands, fp32
accumulation); fp16 / bf16 outputs equal the nearest-even rounding of the
library's own fp32 output.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import glq as og, hadamard
from gpu_util import (TORCH_DT, fp32_to_bf16_rn, fp32_to_f16_rn, fragment_buffer, layer_from, oracle_prefill_u16,
                      rel_frob, say, to_f64, u16_as_f64, x_tensor)

pytestmark = pytest.mark.gpu
glq = pytest.importorskip("e8_lattice_codebook_amd")

DECODE_TOL = 1e-3
PREFILL_TOL = 5e-3

CASES = []
for key, w in synth.WORKLOADS.items():
    for k in range(len(w.layers)):
        CASES.append((key, k))


@pytest.mark.parametrize("key,k", CASES)
def test_linear_workloads(gpu_codebooks, key, k):
    # every layer of every workload at each of its batch sizes, in both index formats
    # (codebook indices, and the slot codes the benchmark times), against one oracle pass
    w = synth.WORKLOADS[key]
    layer = layer_from(key, k)
    qi = glq.QuantizedLayer.from_synth(layer, gpu_codebooks)
    qs = qi.to_slot_codes()
    xs = {B: synth.make_x(layer.n, B, w.act_dtype, w.seed, k) for B in w.batches}
    # one oracle pass for all batch sizes of the layer
    u = np.concatenate([hadamard.rht_in(xs[B][0], layer.sign_in, layer.n_pad) for B in w.batches])
    z = og.matmul_z(u, layer.idx0, layer.idx1, layer.resid_bits, layer.wscale, layer.resid_scale)
    y_all = hadamard.rht_out(z, layer.sign_out, layer.m)
    off = 0
    for B in w.batches:
        want = y_all[off:off + B]
        off += B
        x = x_tensor(xs[B][1], w.act_dtype, "cuda:0")
        for fmt, ql in (("index", qi), ("slot", qs)):
            say("linear", key, k, "B", B, fmt)
            y32 = glq.e8rht_linear(ql, x, torch.float32)
            torch.cuda.synchronize()
            got = to_f64(y32)
            err = rel_frob(got, want)
            tol = DECODE_TOL if B <= 16 else PREFILL_TOL
            say("  rel_frob", err)
            assert err <= tol, (key, k, B, fmt, err)
            # output dtype: one nearest-even rounding of the fp32 result
            for dt, rn in (("f16", fp32_to_f16_rn), ("bf16", fp32_to_bf16_rn)):
                yd = glq.e8rht_linear(ql, x, TORCH_DT[dt])
                torch.cuda.synchronize()
                assert np.array_equal(to_f64(yd), rn(got.astype(np.float32))), (key, k, B, fmt, dt)


def test_prefill_matmul_full_shape(gpu_codebooks):
    # the timed prefill shape (SmolLM3-3B gate, 2048 -> 11008 padded to 16384, 3 bpw,
    # M = 2048): the matmul alone on an operand built on the CPU from the oracle's
    # transform (fp16 with the row exponents), in both index formats (the shared-tile
    # kernel for slot codes, the per-wave kernel for codebook indices).  The only
    # rounding is the fp32 accumulation: relative Frobenius error <= 1e-5 over z, and
    # <= 1e-4 in every 16 x 16 block of z (one MFMA tile: a wrong tile adds about 1).
    key, k = "prefill_gateup", 0
    w = synth.WORKLOADS[key]
    layer = layer_from(key, k)
    qi = glq.QuantizedLayer.from_synth(layer, gpu_codebooks)
    qs = qi.to_slot_codes()
    B = w.batches[0]
    x64, _ = synth.make_x(layer.n, B, w.act_dtype, w.seed, k)
    u16, e = oracle_prefill_u16(x64, layer.sign_in, layer.n_pad)
    uf = fragment_buffer(u16, e, "cuda:0")
    want = og.matmul_z(u16_as_f64(u16, e), layer.idx0, layer.idx1, layer.resid_bits, layer.wscale,
                       layer.resid_scale)
    wb = want.reshape(B // 16, 16, layer.m_pad // 16, 16)
    wn = np.sqrt((wb ** 2).sum(axis=(1, 3)))
    for fmt, ql in (("index", qi), ("slot", qs)):
        say("prefill matmul full shape", fmt)
        z = glq.e8_matmul_prefill(ql, uf, B)
        torch.cuda.synchronize()
        got = to_f64(z[0])
        err = rel_frob(got, want)
        d = (got - want).reshape(wb.shape)
        blk = np.sqrt((d ** 2).sum(axis=(1, 3))) / np.maximum(wn, 1e-30)
        say("  rel_frob", err, "worst 16x16 block", float(blk.max()))
        assert err <= 1e-5, (fmt, err)
        assert float(blk.max()) <= 1e-4, (fmt, float(blk.max()), np.unravel_index(blk.argmax(), blk.shape))


@pytest.mark.parametrize("key,k,B", [("smollm3_block", 6, 1), ("devstral_mlp", 2, 4), ("smollm2_up", 0, 5),
                                     ("tiny", 0, 1), ("devstral_mlp", 0, 16)])
def test_decode_matmul(gpu_codebooks, key, k, B):
    layer = layer_from(key, k)
    ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks)
    rng = np.random.default_rng(B + k)
    u = rng.standard_normal((B, layer.n_pad)).astype(np.float32)
    say("matmul", key, k, B)
    parts = glq.e8_matmul(ql, torch.from_numpy(u).to("cuda:0"))
    torch.cuda.synchronize()
    assert parts.shape == (glq.e8_matmul_splits(ql, B), B, layer.m_pad)
    want = og.matmul_z(u.astype(np.float64), layer.idx0, layer.idx1, layer.resid_bits, layer.wscale,
                       layer.resid_scale)
    err = rel_frob(to_f64(parts).sum(0), want)
    # u is rounded to 16-bit fixed point per 64 columns (step max|u| / 30583): for
    # Gaussian-like u the step is ~1.5e-4 of rms(u) and the rounding error, uniform
    # within half a step, gives a relative error of ~4e-5 in z; the dot products
    # and the fp32 reduction add ~1e-7.  Bound: 1e-4.
    assert err <= 1e-4, err


def test_decode_with_separate_residual_codebook(gpu_codebooks):
    # a 16-bit residual stage whose pack is a different buffer from the primary
    # pack: the decode matmul gathers codewords from the int8 tables in global memory
    layer = layer_from("smollm2_up", 0)
    ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks)
    other = glq.codebook_pack(gpu_codebooks.fp16, "cuda:0")
    ql.desc.cb2_pack = other.data_ptr()
    w = synth.WORKLOADS["smollm2_up"]
    for B in (1, 5):
        x64, raw = synth.make_x(layer.n, B, w.act_dtype, w.seed, 0)
        y = glq.e8rht_linear(ql, x_tensor(raw, w.act_dtype, "cuda:0"), torch.float32)
        torch.cuda.synchronize()
        want = og.linear(x64, layer.sign_in, layer.sign_out, layer.n_pad, layer.m, layer.idx0, layer.idx1,
                         layer.resid_bits, layer.wscale, layer.resid_scale)
        assert rel_frob(to_f64(y), want) <= DECODE_TOL
    del other
