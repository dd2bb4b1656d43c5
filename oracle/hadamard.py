"""Fast Walsh-Hadamard transform and the randomized Hadamard transform (oracle).

glq 0.5.1 (PyPI project page), "How it works", item 2: the randomized Hadamard
transform (RHT) is random sign flips followed by a fast Walsh-Hadamard
transform; it is applied to the weights offline and therefore to the
activations on the way into the layer and to the layer output on the way out
(the separate input_rht / output_rht operations named in the Glq v0.3.2 release
notes, "What changed").

Readings (listed in the design notes): natural (Sylvester) order, i.e.
H[i][j] = (-1)^popcount(i & j); each transform is orthonormal (divided by
sqrt of its padded length); input: sign then H; output: H then sign; inputs are
zero-padded from n to n_pad and outputs truncated from m_pad to m.

Block-diagonal form (glq 0.5.1, table "Bit widths" and the paragraph under it:
sizes that are not powers of two are split into power-of-two blocks, 2688 as
2048 + 512 + 128, so nothing is padded).  Readings: the blocks are the powers of
two of the length's binary expansion, largest first, at consecutive offsets;
each block is transformed on its own, orthonormal (divided by the square root
of the block length); the sign vectors have the unpadded lengths.
All arithmetic is float64.
"""

import numpy as np


def is_pow2(n):
    return n >= 1 and (n & (n - 1)) == 0


def fwht(v):
    """Unnormalized Walsh-Hadamard transform along the last axis, H_n @ v.

    In-place butterflies (a, b) -> (a + b, a - b) at spans h = 1, 2, 4, ...
    Pinned against scipy.linalg.hadamard (Sylvester construction) and the
    identity H H^T = n I in the tests.
    """
    a = np.array(v, dtype=np.float64, copy=True)
    n = a.shape[-1]
    if not is_pow2(n):
        raise ValueError("FWHT length must be a power of two")
    h = 1
    while h < n:
        a = a.reshape(a.shape[:-1] + (n // (2 * h), 2, h))
        lo = a[..., 0, :].copy()
        hi = a[..., 1, :].copy()
        a[..., 0, :] = lo + hi
        a[..., 1, :] = lo - hi
        a = a.reshape(a.shape[:-3] + (n,))
        h *= 2
    return a


def rht_in(x, sign_in, n_pad):
    """Input RHT: u = H_{n_pad} (s_in * [x, 0...]) / sqrt(n_pad), rows of x [B, n]."""
    x = np.asarray(x, dtype=np.float64)
    B, n = x.shape
    if n > n_pad:
        raise ValueError("n > n_pad")
    xp = np.zeros((B, n_pad), dtype=np.float64)
    xp[:, :n] = x
    s = np.asarray(sign_in, dtype=np.float64)
    return fwht(xp * s[None, :]) / np.sqrt(n_pad)


def rht_out(z, sign_out, m):
    """Output RHT: y = (s_out * H_{m_pad} z / sqrt(m_pad))[:, :m], rows of z [B, m_pad]."""
    z = np.asarray(z, dtype=np.float64)
    m_pad = z.shape[-1]
    s = np.asarray(sign_out, dtype=np.float64)
    return (s[None, :] * fwht(z) / np.sqrt(m_pad))[:, :m]


def pow2_blocks(n):
    """Block lengths of the block-diagonal transform of length n, largest first:
    the powers of two whose sum is n (its binary expansion)."""
    if n < 1:
        raise ValueError("length must be positive")
    out = []
    bit = 1 << (int(n).bit_length() - 1)
    while bit:
        if n & bit:
            out.append(bit)
        bit >>= 1
    return out


def block_fwht(v):
    """Orthonormal block-diagonal transform along the last axis: block b of length
    L (at its offset) becomes H_L v_b / sqrt(L)."""
    a = np.asarray(v, dtype=np.float64)
    out = np.empty_like(a)
    off = 0
    for L in pow2_blocks(a.shape[-1]):
        out[..., off:off + L] = fwht(a[..., off:off + L]) / np.sqrt(L)
        off += L
    return out


def rht_in_blocks(x, sign_in):
    """Block-diagonal input RHT: u = D_n (s_in * x), rows of x [B, n], no padding."""
    x = np.asarray(x, dtype=np.float64)
    s = np.asarray(sign_in, dtype=np.float64)
    if s.shape[-1] != x.shape[-1]:
        raise ValueError("sign_in must have n entries")
    return block_fwht(x * s[None, :])


def rht_out_blocks(z, sign_out):
    """Block-diagonal output RHT: y = s_out * D_m z, rows of z [B, m], no padding."""
    z = np.asarray(z, dtype=np.float64)
    s = np.asarray(sign_out, dtype=np.float64)
    if s.shape[-1] != z.shape[-1]:
        raise ValueError("sign_out must have m entries")
    return s[None, :] * block_fwht(z)
