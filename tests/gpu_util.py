"""Shared helpers of the GPU parity tests (device setup, error measures)."""
import sys

import numpy as np
import torch

import synth


def rel_frob(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / (den if den > 0 else 1.0))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def x_tensor(raw, dtype, device):
    """Device tensor from synth.make_x's raw array (float32 / float16 / bf16 bits)."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(raw)).to(device)
    if dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(raw)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).to(device)
    return t.view(torch.bfloat16)


TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def same_products(y_index, y_slot, prefill):
    """Slot codes name the same codewords as codebook indices, so both formats form
    the same exact products.  The decode paths and the row-order prefill kernel run
    the same kernel on both: bit-equal outputs.  The prefill of a slot-code layer
    runs the shared-tile kernel (another fp32 summation order): within 1e-5."""
    if not prefill:
        return bool(torch.equal(y_index, y_slot))
    return rel_frob(to_f64(y_slot), to_f64(y_index)) <= 1e-5


def to_f64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def fp32_to_f16_rn(y32):
    return np.asarray(y32, dtype=np.float32).astype(np.float16).astype(np.float64)


def fp32_to_bf16_rn(y32):
    from oracle import glq as og
    return og.bf16_bits_to_f64(og.fp32_to_bf16_bits(np.asarray(y32, dtype=np.float32)))


def layer_from(workload_key, k):
    w = synth.WORKLOADS[workload_key]
    return synth.make_layer(w.layers[k], w.resid_bits, w.seed, k)


# ---- fp16 prefill operands built on the CPU from the oracle's transform ----------------
# The library's prefill path stores u[b] * 2^-e[b] in fp16 with
# e[b] = (frexp exponent of max |x[b]|) + ceil(log2 sqrt(n)) - 14 (0 for a zero row,
# 0x7FFFFFFF for a row with a NaN or an infinity), the placement of include/glq.h's
# fragment order, and the int32 exponents after it at a 256-byte boundary.
ROW_EXP_NAN = 0x7FFFFFFF


def row_exponents(x64, n):
    x64 = np.asarray(x64, dtype=np.float64)
    c = 0
    while (1 << (2 * c)) < n:
        c += 1
    finite = np.isfinite(x64).all(axis=1)
    mx = np.where(finite, np.abs(np.where(np.isfinite(x64), x64, 0.0)).max(axis=1), 0.0)
    fe = np.frexp(mx)[1]
    e = np.where(mx > 0, fe + c - 14, 0).astype(np.int64)
    return np.where(finite, e, ROW_EXP_NAN).astype(np.int32)


def oracle_prefill_u16(x64, sign_in, n_pad):
    """(fp16 u [B][n_pad] as the library stores it, row exponents) from the oracle's fp64 u."""
    from oracle import hadamard
    x64 = np.asarray(x64, dtype=np.float64)
    e = row_exponents(x64, x64.shape[1])
    if hadamard.is_pow2(n_pad):
        u = hadamard.rht_in(x64, sign_in, n_pad)
    else:  # block-diagonal over the binary expansion of n_pad, zeros past n
        xp = np.zeros((x64.shape[0], n_pad))
        xp[:, :x64.shape[1]] = x64
        u = hadamard.rht_in_blocks(xp, sign_in)
    return (u * np.ldexp(1.0, -e.astype(np.int64))[:, None]).astype(np.float16), e


def fragment_positions(M, n_pad):
    KS = n_pad // 32
    b, i = np.meshgrid(np.arange(M), np.arange(n_pad), indexing="ij")
    g = i // 8
    ks, q = 4 * (g // 16) + g % 4, (g // 4) % 4
    return (((b // 16) * KS + ks) * 4 + q) * 128 + (b % 16) * 8 + i % 8


def fragment_buffer(u16, rexp, device):
    """The fragment-order operand buffer (fp16 values, then the row exponents) of u16 [M][n_pad]."""
    M, n_pad = u16.shape
    Mp = (M + 15) // 16 * 16
    r256 = lambda v: (v + 255) // 256 * 256
    off = r256(Mp * n_pad * 2)
    buf = np.zeros(off + r256(Mp * 4), dtype=np.uint8)
    halves = buf[:Mp * n_pad * 2].view(np.uint16)
    halves[fragment_positions(M, n_pad)] = np.asarray(u16, dtype=np.float16).view(np.uint16)
    e = np.zeros(Mp, dtype=np.int32)
    e[:M] = rexp
    buf[off:off + Mp * 4] = e.view(np.uint8)
    return torch.from_numpy(buf).to(device)


def unpack_fragment_buffer(buf, M, n_pad):
    """(fp16 u [M][n_pad], int32 row exponents [M]) read back from a fragment-order buffer."""
    raw = buf.cpu().numpy().view(np.uint8)
    Mp = (M + 15) // 16 * 16
    off = (Mp * n_pad * 2 + 255) // 256 * 256
    halves = raw[:Mp * n_pad * 2].view(np.float16)
    return halves[fragment_positions(M, n_pad)], raw[off:off + Mp * 4].view(np.int32)[:M].copy()


def u16_as_f64(u16, rexp):
    return np.asarray(u16, dtype=np.float64) * np.ldexp(1.0, np.asarray(rexp, dtype=np.int64))[:, None]
