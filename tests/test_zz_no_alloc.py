"""glq_e8rht_linear_noalloc against glq_e8rht_linear (the same kernels on the same
inputs, with the library's static device scratch as the workspace instead of a
caller's buffer): bit-identical outputs, on consecutive calls of decreasing size
(each reuses what the previous call left in the scratch), on the decode, staged
and prefill paths; a call whose workspace would exceed the scratch is refused
before anything is launched and leaves y untouched."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from gpu_util import layer_from, say, x_tensor

pytestmark = pytest.mark.gpu
glq = pytest.importorskip("e8_lattice_codebook_amd")
DEV = "cuda:0"


def _pair(ql, x, y_dtype=torch.float32):
    want = glq.e8rht_linear(ql, x, y_dtype)
    got = glq.e8rht_linear_noalloc(ql, x, y_dtype)
    torch.cuda.synchronize()
    return want, got


def test_noalloc_matches_linear(gpu_codebooks):
    # largest first: the Devstral gate layer at B = 16 (about 35 MiB of scratch), then
    # B = 4, then the SmolLM3 q layer at B = 1 (the two-launch path), then a prefill
    # call of 40 tokens, then the tiny layer
    cases = [("devstral_mlp", 0, 16), ("devstral_mlp", 2, 4), ("smollm3_block", 0, 1), ("smollm3_block", 4, 40),
             ("tiny", 0, 1)]
    for key, k, B in cases:
        w = synth.WORKLOADS[key]
        layer = layer_from(key, k)
        ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks).to_slot_codes()
        assert glq.linear_workspace_bytes(ql, B) <= glq.NOALLOC_SCRATCH_BYTES
        _, raw = synth.make_x(layer.n, B, w.act_dtype, w.seed, k)
        x = x_tensor(raw, w.act_dtype, DEV)
        say("noalloc", key, k, B)
        for _ in range(2):  # twice in a row on the same inputs
            want, got = _pair(ql, x)
            assert torch.equal(want, got), (key, k, B)
        want, got = _pair(ql, x, torch.bfloat16)
        assert torch.equal(want.view(torch.int16), got.view(torch.int16))


def test_noalloc_refuses_oversized_calls(gpu_codebooks):
    # the SmolLM3 gate prefill at 2048 tokens needs about 136 MiB: refused, y untouched
    key, k = "prefill_gateup", 0
    w = synth.WORKLOADS[key]
    layer = layer_from(key, k)
    ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks).to_slot_codes()
    B = 2048
    assert glq.linear_workspace_bytes(ql, B) > glq.NOALLOC_SCRATCH_BYTES
    _, raw = synth.make_x(layer.n, B, w.act_dtype, w.seed, k)
    x = x_tensor(raw, w.act_dtype, DEV)
    y = torch.full((B, layer.m), 7.0, device=DEV)
    with pytest.raises(glq.GLQError) as e:
        glq.e8rht_linear_noalloc(ql, x, out=y)
    assert e.value.name == "GLQ_ERR_WORKSPACE"
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
    # and a valid call right after it still matches the linear
    layer = layer_from("smollm2_up", 0)
    ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks).to_slot_codes()
    _, raw = synth.make_x(layer.n, 5, "f16", 1002, 0)
    want, got = _pair(ql, x_tensor(raw, "f16", DEV))
    assert torch.equal(want, got)
