"""GPU parity of the input and output randomized Hadamard transforms against
the fp64 oracle (glq 0.5.1, "How it works", item 2; Glq v0.3.2 release notes,
"What changed": input_rht / output_rht, a separate path above 16384).

Tolerance: fp32 butterflies over log2(N) stages; the error is a few fp32 ulps of
the row norm, bounded here by 1e-6 relative Frobenius.  fp16 / bf16 outputs are
within one unit of rounding of the fp64 result (2^-11 and 2^-8 relative).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import hadamard
from gpu_util import TORCH_DT, rel_frob, say, to_f64, x_tensor

pytestmark = pytest.mark.gpu
glq = pytest.importorskip("e8_lattice_codebook_amd")

REL = {"f32": 1e-6, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}


@pytest.mark.parametrize("n,n_pad,B", [(8, 8, 1), (5, 8, 3), (16, 16, 2), (100, 128, 1), (256, 256, 1),
                                       (960, 1024, 5), (2048, 2048, 1), (4000, 4096, 2), (11008, 16384, 5),
                                       (16384, 16384, 1), (32768, 32768, 1), (20000, 32768, 4),
                                       (5120, 65536, 2), (1 << 20, 1 << 20, 1)])
@pytest.mark.parametrize("xdt,udt", [("f32", "f32"), ("f16", "f32"), ("bf16", "f32"), ("bf16", "f16"),
                                     ("f16", "bf16")])
def test_input_rht(n, n_pad, B, xdt, udt):
    if n_pad >= 1 << 20 and (xdt, udt) != ("f32", "f32"):
        pytest.skip("one dtype pair at the maximum size")
    say("input_rht", n, n_pad, B, xdt, udt)
    x64, raw = synth.make_x(n, B, xdt, 77, n_pad)
    sign = synth.make_layer(synth.LayerShape("s", n, 8, n_pad, 8), 0, 5, 0).sign_in
    dev = "cuda:0"
    u = glq.input_rht(x_tensor(raw, xdt, dev), n_pad, torch.from_numpy(sign).to(dev), TORCH_DT[udt])
    torch.cuda.synchronize()
    want = hadamard.rht_in(x64, sign, n_pad)
    got = to_f64(u)
    assert got.shape == (B, n_pad)
    err = rel_frob(got, want)
    assert err <= REL[udt], err


@pytest.mark.parametrize("m,m_pad,B,S", [(8, 8, 1, 1), (3, 8, 2, 2), (200, 256, 1, 1), (2560, 4096, 5, 1),
                                         (512, 512, 5, 4), (11008, 16384, 1, 2), (32768, 32768, 4, 2),
                                         (30000, 32768, 1, 8), (5120, 8192, 16, 8), (1000, 131072, 1, 1)])
@pytest.mark.parametrize("ydt", ["f32", "f16", "bf16"])
def test_output_rht(m, m_pad, B, S, ydt):
    say("output_rht", m, m_pad, B, S, ydt)
    rng = np.random.default_rng(m + m_pad + S)
    z = rng.standard_normal((S, B, m_pad)).astype(np.float32)
    sign = (2 * rng.integers(0, 2, m_pad) - 1).astype(np.int8)
    dev = "cuda:0"
    y = glq.output_rht(torch.from_numpy(z).to(dev), m, torch.from_numpy(sign).to(dev), TORCH_DT[ydt])
    torch.cuda.synchronize()
    want = hadamard.rht_out(z.astype(np.float64).sum(0), sign, m)
    got = to_f64(y)
    assert got.shape == (B, m)
    err = rel_frob(got, want)
    assert err <= REL[ydt], err


@pytest.mark.parametrize("m,m_pad,B,S", [(4000, 4096, 600, 3), (11008, 16384, 300, 2), (32768, 32768, 260, 1)])
@pytest.mark.parametrize("ydt", ["f32", "bf16"])
def test_output_rht_more_rows_than_workgroups(m, m_pad, B, S, ydt):
    # more rows than one workgroup per CU: each workgroup takes several rows in turn,
    # loading the next row's split sum while it transforms the current one
    test_output_rht(m, m_pad, B, S, ydt)


def test_output_split_order_is_fixed():
    # the same partials give bit-identical outputs on repeated calls
    dev = "cuda:0"
    rng = np.random.default_rng(3)
    z = torch.from_numpy(rng.standard_normal((8, 2, 4096)).astype(np.float32)).to(dev)
    sign = torch.from_numpy((2 * rng.integers(0, 2, 4096) - 1).astype(np.int8)).to(dev)
    a = glq.output_rht(z, 4000, sign)
    b = glq.output_rht(z, 4000, sign)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
