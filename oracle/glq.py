"""Dequantization and the E8RHTLinear forward (oracle; test infrastructure only).

glq 0.5.1 (PyPI project page):
  * "How it works", item 1: an 8-weight group is one 16-bit index into the E8
    codebook; 3-8 bpw add 8-bit (256-entry) or 16-bit residual stages that
    refine the primary reconstruction.
  * table "Bit widths": 2 bpw = 16b primary; 3 bpw = 16b + 8b; 4 bpw = 16b + 16b;
    one global scale per layer, no group size.
  * "Inference kernels": Y = X @ dequant(W)^T with N/8 codebook blocks per
    output row; the two-stage call passes Wscale, Qidxs2, codebook2 and
    inv_resid_scale; the CPU path dequantizes and then multiplies.

Reading (design notes): W~[o][8g + j] = s * (C0[I0[o, g]][j] + s_r * C1[I1[o, g]][j]),
with the residual term absent at 2 bpw; 5-8 bpw ("Bit widths": 16b + 16b + 8b,
16b + 16b + 16b, 16b + 16b + 16b + 8b, 16b x 4) add sum_k s_k C_k[I_k[o, g]][j] over
the further stages k, each with its own scale s_k (the `extra` argument); a group is 8 consecutive input columns of
one output row and I0/I1 are row-major [m_pad, n_pad / 8].  The layer forward is
  y = RHT_out(RHT_in(x) @ W~^T)
with RHT_in / RHT_out from oracle.hadamard.  Everything is float64 except
dequant_fp32, which states the one fp32 rounding the GPU dequantizer must match
bit for bit.
"""

import numpy as np

from . import e8, hadamard


def _tables(resid_bits):
    c0 = e8.codebook(e8.ENTRIES)
    c1 = e8.residual_codebook(resid_bits) if resid_bits else None
    return c0, c1


def _extra_terms(extra, rows):
    """sum_k s_k C_k[I_k] over the further residual stages, float64 [rows, groups, 8]."""
    total = None
    for idx, bits, scale in extra:
        i = np.asarray(idx)
        if rows is not None:
            i = i[rows]
        t = np.float64(np.float32(scale)) * e8.residual_codebook(bits)[i.astype(np.int64)]
        total = t if total is None else total + t
    return total


def dequant_rows(idx0, idx1, resid_bits, wscale, resid_scale, rows=None, tables=None, extra=()):
    """W~ rows as float64 [len(rows), n_pad] (all rows when rows is None).

    Exact: codeword values are in Z/2 and s, s_r are the fp32 values given, so
    the only inexact step is the float64 product s * e, which is also exact for
    fp32 s and e with 8 * e in Z (fewer than 53 significant bits).
    """
    c0, c1 = tables if tables is not None else _tables(resid_bits)
    i0 = np.asarray(idx0)
    if rows is not None:
        i0 = i0[rows]
    m_rows, groups = i0.shape
    e = c0[i0.astype(np.int64)]                       # [rows, groups, 8]
    if resid_bits:
        i1 = np.asarray(idx1)
        if rows is not None:
            i1 = i1[rows]
        e = e + np.float64(np.float32(resid_scale)) * c1[i1.astype(np.int64)]
    if extra:
        e = e + _extra_terms(extra, rows)
    w = np.float64(np.float32(wscale)) * e
    return w.reshape(m_rows, groups * 8)


def dequant_fp32(idx0, idx1, resid_bits, wscale, resid_scale, rows=None, extra=()):
    """The fp32 dequantized weights, rounded once: w32 = RN32(s32 * e), e exact.

    e = c0 + s_r * c1 is exact in fp32 (8 e is an integer of at most 6 bits when
    s_r is a power of two such as 1/4; in general e is first rounded to fp32),
    then the product with s is rounded to nearest-even once.  Further stages k are
    added in order, each sum rounded to fp32: e = RN32(e + s_k c_k) (exact for
    power-of-two scales).
    """
    c0, c1 = _tables(resid_bits)
    i0 = np.asarray(idx0)
    if rows is not None:
        i0 = i0[rows]
    e = c0[i0.astype(np.int64)]
    if resid_bits:
        i1 = np.asarray(idx1)
        if rows is not None:
            i1 = i1[rows]
        e = e + np.float64(np.float32(resid_scale)) * c1[i1.astype(np.int64)]
    e32 = e.astype(np.float32).astype(np.float64)
    for idx, bits, scale in extra:
        i = np.asarray(idx)
        if rows is not None:
            i = i[rows]
        ck = e8.residual_codebook(bits)[i.astype(np.int64)]
        e32 = (e32 + np.float64(np.float32(scale)) * ck).astype(np.float32).astype(np.float64)
    w32 = (np.float64(np.float32(wscale)) * e32).astype(np.float32)
    return w32.reshape(i0.shape[0], i0.shape[1] * 8)


def fp32_to_bf16_bits(w32):
    """Round fp32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns.

    Finite inputs only.  Pinned against torch's CPU float32 -> bfloat16 cast.
    """
    bits = np.asarray(w32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    return ((bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f64(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def matmul_z(u, idx0, idx1, resid_bits, wscale, resid_scale, row_block=2048, extra=()):
    """z = u @ W~^T, float64 [B, m_pad], with W~ formed in row blocks of row_block rows."""
    u = np.asarray(u, dtype=np.float64)
    m_pad = np.asarray(idx0).shape[0]
    tables = _tables(resid_bits)
    z = np.empty((u.shape[0], m_pad), dtype=np.float64)
    for r0 in range(0, m_pad, row_block):
        rows = np.arange(r0, min(m_pad, r0 + row_block))
        w = dequant_rows(idx0, idx1, resid_bits, wscale, resid_scale, rows=rows, tables=tables, extra=extra)
        z[:, rows] = u @ w.T
    return z


def linear(x, sign_in, sign_out, n_pad, m, idx0, idx1, resid_bits, wscale, resid_scale, extra=(), block_diag=False):
    """E8RHTLinear forward in float64: y [B, m] from x [B, n].

    Dequantize-then-matmul, the page's CPU path, between the two transforms.
    block_diag: the transforms are block-diagonal over the power-of-two blocks of
    n and m (oracle.hadamard.rht_in_blocks / rht_out_blocks); then n_pad == n and
    the index arrays have m rows.
    """
    if block_diag:
        if np.asarray(x).shape[-1] != n_pad or np.asarray(idx0).shape[0] != m:
            raise ValueError("a block-diagonal layer is unpadded")
        u = hadamard.rht_in_blocks(x, sign_in)
        z = matmul_z(u, idx0, idx1, resid_bits, wscale, resid_scale, extra=extra)
        return hadamard.rht_out_blocks(z, sign_out)
    u = hadamard.rht_in(x, sign_in, n_pad)
    z = matmul_z(u, idx0, idx1, resid_bits, wscale, resid_scale, extra=extra)
    return hadamard.rht_out(z, sign_out, m)
