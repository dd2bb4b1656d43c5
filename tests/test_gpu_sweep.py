"""Small-shape sweep of the E8RHTLinear forward against the oracle: every recipe,
power-of-two pads 8..1024 with ragged n < n_pad and m < m_pad, batch sizes
across the decode / prefill boundary (B = 16 / 17), plus determinism and HIP
graph replay of the call.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import glq as og
from gpu_util import rel_frob, say, to_f64

pytestmark = pytest.mark.gpu
glq = pytest.importorskip("e8_lattice_codebook_amd")

SHAPES = [(8, 8, 8, 8), (5, 3, 8, 8), (8, 16, 8, 16), (40, 8, 64, 8), (100, 70, 128, 128), (256, 200, 256, 256),
          (1000, 24, 1024, 32), (17, 1000, 32, 1024), (512, 512, 512, 512)]


@pytest.mark.parametrize("resid_bits", [0, 8, 16])
@pytest.mark.parametrize("n,m,n_pad,m_pad", SHAPES)
def test_sweep(gpu_codebooks, resid_bits, n, m, n_pad, m_pad):
    layer = synth.random_layer(n, m, resid_bits, seed=n * 7 + m * 3 + resid_bits, n_pad=n_pad, m_pad=m_pad)
    ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks)
    for B in (1, 2, 3, 5, 8, 9, 16, 17, 33):
        say("sweep", n, m, n_pad, m_pad, resid_bits, B)
        x = np.random.default_rng(B).standard_normal((B, n)).astype(np.float32)
        y = glq.e8rht_linear(ql, torch.from_numpy(x).to("cuda:0"), torch.float32)
        torch.cuda.synchronize()
        want = og.linear(x.astype(np.float64), layer.sign_in, layer.sign_out, n_pad, m, layer.idx0, layer.idx1,
                         resid_bits, layer.wscale, layer.resid_scale)
        err = rel_frob(to_f64(y), want)
        assert err <= (1e-3 if B <= 16 else 5e-3), (B, err)


def test_zero_indices_give_exact_zero(gpu_codebooks):
    layer = synth.random_layer(200, 300, 16, seed=9)
    layer.idx0[:] = 0
    layer.idx1[:] = 0
    ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks)
    for B in (1, 20):
        x = torch.randn(B, 200, device="cuda:0")
        y = glq.e8rht_linear(ql, x, torch.float32)
        torch.cuda.synchronize()
        assert torch.count_nonzero(y).item() == 0


@pytest.mark.parametrize("key,k,B", [("devstral_mlp", 2, 1), ("smollm3_block", 4, 5), ("prefill_gateup", 0, 2048)])
def test_repeat_bit_identical(gpu_codebooks, key, k, B):
    w = synth.WORKLOADS[key]
    layer = synth.make_layer(w.layers[k], w.resid_bits, w.seed, k)
    ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks)
    x = torch.randn(B, layer.n, device="cuda:0", dtype=torch.float16)
    say("repeat", key, k, B)
    a = glq.e8rht_linear(ql, x, torch.float32)
    b = glq.e8rht_linear(ql, x, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("B", [1, 4, 24])
def test_hip_graph_replay(gpu_codebooks, B):
    # the call allocates nothing and never synchronizes, so it captures; every
    # replay must equal the eager result
    layer = synth.random_layer(5120, 4000, 16, seed=B, n_pad=8192, m_pad=4096)
    ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks)
    dev = "cuda:0"
    x = torch.randn(B, 5120, device=dev, dtype=torch.bfloat16)
    ws = glq.linear_workspace(ql, B, dev)
    y = torch.empty(B, 4000, device=dev, dtype=torch.float32)
    eager = glq.e8rht_linear(ql, x, torch.float32, workspace=ws).clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        glq.e8rht_linear(ql, x, torch.float32, workspace=ws, out=y)  # warm on the side stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            glq.e8rht_linear(ql, x, torch.float32, workspace=ws, out=y)
    torch.cuda.synchronize()
    for _ in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager)
        _ = (x.float() * 2).sum().item()   # eager work between replays
