"""GPU parity of the B = 1 forward (input RHT chunk per workgroup, LDS-codebook
matmul and row-block output transform; then the fixed-order split reduction and
the cross-block output transform) against the fp64 oracle.

glq 0.5.1, "How it works" items 1-4 and "Inference kernels".  Tolerance: the
decode bound, relative Frobenius error of fp32 y <= 1e-3 (16-bit fixed-point
activations, exact integer dot products, fp32 transforms).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import glq as og
from gpu_util import rel_frob, say, to_f64

pytestmark = pytest.mark.gpu
glq = pytest.importorskip("e8_lattice_codebook_amd")

TOL = 1e-3
DEV = "cuda:0"


def oracle_y(layer, x64):
    return og.linear(x64, layer.sign_in, layer.sign_out, layer.n_pad, layer.m, layer.idx0, layer.idx1,
                     layer.resid_bits, layer.wscale, layer.resid_scale)


def rounded_x(n, dtype, seed):
    """x [1, n] drawn in fp32, rounded once to dtype; returns (float64 copy, device tensor)."""
    x = torch.from_numpy(np.random.default_rng(seed).standard_normal((1, n)).astype(np.float32)).to(dtype)
    return x.to(torch.float64).numpy(), x.to(DEV)


# (n, m, n_pad, m_pad): one split with 64 lanes per row, two, four and eight
# splits, fewer than 64 lanes per row, and the largest m_pad of the one-launch path;
# workgroup row blocks of 16 (LDS passes), 512 and 1024 rows (one-wave transform);
# cross-block transforms from 1 (m_pad 64: a single block) to 128 blocks
SHAPES = [(4000, 1000, 4096, 1024), (5120, 700, 8192, 1024), (11008, 300, 16384, 512),
          (32768, 64, 32768, 64), (2000, 2048, 2048, 2048), (60, 30000, 64, 32768), (100, 8000, 128, 8192)]


@pytest.mark.parametrize("resid_bits", [0, 8, 16])
@pytest.mark.parametrize("n,m,n_pad,m_pad", SHAPES)
def test_fused_shapes(gpu_codebooks, resid_bits, n, m, n_pad, m_pad):
    layer = synth.random_layer(n, m, resid_bits, seed=n + m + resid_bits, n_pad=n_pad, m_pad=m_pad)
    ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks)
    for dt in (torch.float32, torch.float16, torch.bfloat16):
        say("fused", n, m, n_pad, m_pad, resid_bits, dt)
        x64, x = rounded_x(n, dt, seed=n + resid_bits)
        y = glq.e8rht_linear(ql, x, torch.float32)
        torch.cuda.synchronize()
        err = rel_frob(to_f64(y), oracle_y(layer, x64))
        say("  rel_frob", err)
        assert err <= TOL, (dt, err)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_fused_unaligned_ragged_x(gpu_codebooks, dt):
    # x starts one element into its buffer (no 4-element loads) and n % 4 != 0
    n, m = 4093, 900
    layer = synth.random_layer(n, m, 16, seed=77, n_pad=8192, m_pad=1024)
    ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks)
    x64, xd = rounded_x(n + 1, dt, seed=5)
    x = xd[:, 1:]
    assert x.data_ptr() % 8 != 0
    y = glq.e8rht_linear(ql, x, torch.float32)
    torch.cuda.synchronize()
    assert rel_frob(to_f64(y), oracle_y(layer, x64[:, 1:])) <= TOL


def test_workspace_shared(gpu_codebooks):
    # one workspace (uninitialized) serves B = 1 and staged calls of several layers
    layers = [synth.random_layer(5120, 3000, 16, seed=1, n_pad=8192, m_pad=4096),
              synth.random_layer(3000, 2000, 8, seed=2, n_pad=4096, m_pad=2048),
              synth.random_layer(700, 500, 0, seed=3, n_pad=1024, m_pad=512)]
    qls = [glq.QuantizedLayer.from_synth(l, gpu_codebooks) for l in layers]
    nbytes = max(glq.linear_workspace_bytes(q, B) for q in qls for B in (1, 5))
    ws = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device=DEV)
    for rep in range(2):
        for l, q in zip(layers, qls):
            for B in (1, 5, 1):
                say("shared workspace", rep, l.n, l.m, B)
                x = np.random.default_rng(B + rep).standard_normal((B, l.n)).astype(np.float32)
                y = glq.e8rht_linear(q, torch.from_numpy(x).to(DEV), torch.float32, workspace=ws)
                torch.cuda.synchronize()
                assert rel_frob(to_f64(y), oracle_y(l, x.astype(np.float64))) <= TOL


def test_large_m_pad(gpu_codebooks):
    # m_pad 65536: 64 row blocks of 1024 rows, a 64-point cross-block transform
    layer = synth.random_layer(64, 40000, 16, seed=4, n_pad=64, m_pad=65536)
    ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks)
    x64, x = rounded_x(64, torch.float32, seed=6)
    y = glq.e8rht_linear(ql, x, torch.float32)
    torch.cuda.synchronize()
    assert rel_frob(to_f64(y), oracle_y(layer, x64)) <= TOL


def test_fused_unaligned_signs(gpu_codebooks):
    # sign_in / sign_out / y one element into their buffers: the element-wise paths
    n, m = 3000, 2000
    layer = synth.random_layer(n, m, 8, seed=88, n_pad=4096, m_pad=2048)
    ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks)
    si = torch.zeros(layer.n_pad + 1, dtype=torch.int8, device=DEV)
    so = torch.zeros(layer.m_pad + 1, dtype=torch.int8, device=DEV)
    si[1:] = torch.from_numpy(layer.sign_in).to(DEV)
    so[1:] = torch.from_numpy(layer.sign_out).to(DEV)
    ql.desc.sign_in = si.data_ptr() + 1
    ql.desc.sign_out = so.data_ptr() + 1
    x64, x = rounded_x(n, torch.bfloat16, seed=9)
    want = oracle_y(layer, x64)
    y = glq.e8rht_linear(ql, x, torch.float32)
    torch.cuda.synchronize()
    assert rel_frob(to_f64(y), want) <= TOL
    # y one element into its buffer: the element-wise output stores
    yb = torch.empty(1, m + 1, dtype=torch.bfloat16, device=DEV)
    yv = yb[:, 1:]
    glq.e8rht_linear(ql, x, torch.bfloat16, out=yv)
    torch.cuda.synchronize()
    assert rel_frob(to_f64(yv), want) <= 5e-3  # bf16 output rounding
