"""GPU parity of the E8RHTLinear forward on inputs at the edges of the number range.

glq 0.5.1, "How it works" items 2-4 and "Inference kernels": the layer is linear in
x, so y(2^k x) = 2^k y(x) exactly in the oracle.  The library's reduced-precision
steps (16-bit fixed point per 64 columns or 15-bit per row for B <= 16, fp16 operands for
B > 16)
carry power-of-two scales, so its result scales the same way while y stays in the
fp32 range: checked against the library's own unscaled output (relative Frobenius
<= 1e-6, which leaves room only for subnormal rounding of the smallest outputs) and
against the oracle at the path's tolerance.  Zero rows give zero outputs, outlier
channels keep the tolerance, and a NaN or infinity in a row of x makes that row of
y NaN (the oracle's y is NaN there too) without touching the other rows.

Paths: B = 1 (the two-launch decode), B = 3 on a layer of 2^20 groups (2048 -> 4096:
the staged integer decode, 16-bit fixed point per 64 columns), B = 5 on that layer and
B = 2, 3, 5 and 16 on a layer of 2^22 groups (2048 -> 16384) (the decode on the int8
matrix units, 15-bit fixed point per row), M = 40 (prefill, the shared-tile kernel of
slot codes and the per-wave kernel of codebook indices), M = 160 (prefill with the
persistent one-row-per-workgroup output transform).
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

N, M_OUT = 2048, 3000
PATHS = [(1, "index"), (3, "index"), (5, "index"), (1, "slot"), (3, "slot"), (5, "slot"), (40, "slot"), (40, "index"),
         (2, "slot-big"), (3, "index-big"), (5, "slot-big"), (16, "index-big"), (160, "slot")]
_LAYERS = {}


def _layer(gpu_codebooks, fmt, resid_bits=8):
    big = fmt.endswith("-big")
    key = (big, resid_bits)
    if key not in _LAYERS:
        if big:  # 2048 -> 16384: 2^22 groups, the int8 matrix-unit decode for 2 <= B <= 16
            _LAYERS[key] = synth.random_layer(N, 16000, resid_bits, seed=78 + resid_bits, n_pad=2048, m_pad=16384)
        else:
            _LAYERS[key] = synth.random_layer(N, M_OUT, resid_bits, seed=77 + resid_bits, n_pad=2048, m_pad=4096)
    layer = _LAYERS[key]
    ql = glq.QuantizedLayer.from_synth(layer, gpu_codebooks)
    return layer, (ql.to_slot_codes() if fmt.startswith("slot") else ql)


def _tol(B):
    return 1e-3 if B <= 16 else 5e-3


def _oracle(layer, x64):
    return og.linear(x64, layer.sign_in, layer.sign_out, layer.n_pad, layer.m, layer.idx0, layer.idx1,
                     layer.resid_bits, layer.wscale, layer.resid_scale)


def _run(ql, x32):
    y = glq.e8rht_linear(ql, torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(DEV), torch.float32)
    torch.cuda.synchronize()
    return to_f64(y)


@pytest.mark.parametrize("B,fmt", PATHS)
def test_power_of_two_scaling(gpu_codebooks, B, fmt):
    layer, ql = _layer(gpu_codebooks, fmt)
    x = np.random.default_rng(B).standard_normal((B, N))
    # no element below 2^-5 in magnitude, so that x 2^-120 is still a normal fp32 number
    # and every scaled input is exactly 2^k x
    x = np.where(np.abs(x) < 2.0 ** -5, np.copysign(2.0 ** -5, x), x).astype(np.float32)
    y0 = _run(ql, x)
    want = _oracle(layer, x.astype(np.float64))
    assert rel_frob(y0, want) <= _tol(B)
    for k in (-120, -60, 60):
        say("scaling", B, fmt, k)
        xk = np.ldexp(x, k)  # exact in fp32
        yk = _run(ql, xk)
        assert np.all(np.isfinite(yk)), k
        back = np.ldexp(yk, -k)
        err = rel_frob(back, y0)
        say("  vs unscaled", err)
        assert err <= 1e-6, (k, err)
        assert rel_frob(back, want) <= _tol(B), k


@pytest.mark.parametrize("B,fmt", PATHS)
def test_row_scales_zero_rows_and_outliers(gpu_codebooks, B, fmt):
    # rows of very different magnitudes (2^-100 .. 2^100 for the larger batches), an
    # all-zero row, and three outlier channels at 1000 sigma
    layer, ql = _layer(gpu_codebooks, fmt)
    rng = np.random.default_rng(100 + B)
    x = rng.standard_normal((B, N))
    x[:, [5, 700, 2047]] *= 1000.0
    if B > 1:
        x *= np.exp2(rng.integers(-100, 101, size=(B, 1)))
        x[1] = 0.0
    x = x.astype(np.float32)
    y = _run(ql, x)
    want = _oracle(layer, x.astype(np.float64))
    if B > 1:
        assert np.all(y[1] == 0.0)
    for b in range(B):  # each row against its own norm
        if b == 1 and B > 1:
            continue
        err = rel_frob(y[b], want[b])
        assert err <= _tol(B), (b, err)


@pytest.mark.parametrize("B,fmt", PATHS)
def test_non_finite_rows(gpu_codebooks, B, fmt):
    layer, ql = _layer(gpu_codebooks, fmt)
    x = np.random.default_rng(200 + B).standard_normal((B, N)).astype(np.float32)
    for bad in (np.nan, np.inf, -np.inf):
        xb = x.copy()
        xb[0, 11] = bad
        if B > 1:
            xb[B - 1, 1000] = np.nan
        say("non-finite", B, fmt, bad)
        y = _run(ql, xb)
        assert np.all(np.isnan(y[0])), bad
        want = _oracle(layer, xb.astype(np.float64))
        assert not np.any(np.isfinite(want[0]))
        if B > 1:
            assert np.all(np.isnan(y[B - 1]))
        if B > 2:  # the rows between the two bad ones
            good = slice(1, B - 1)
            assert np.all(np.isfinite(y[good]))
            assert rel_frob(y[good], want[good]) <= _tol(B)
