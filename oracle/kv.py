"""E8 lattice KV cache and decode attention (oracle; test infrastructure only).

Glq v0.5.0 release notes, "Highlights" and "Scope"; glq 0.5.1 (PyPI project page),
"KV cache compression" -> "E8 lattice cache" and "Inline-dequant E8 KV": the paged
K/V cache is compressed with the same E8 lattice quantizer as the weights to about
a quarter of its fp16 size (the 4 bpw recipe e8_relaxed:2), and a decode attention
kernel expands it inside its tile loop, inverting the per-group rotation with a
radix-2 Hadamard transform of length 8 and spreading long contexts over
workgroups (flash-decoding).

Readings (listed in the design notes; the pages fix none of these details):
  * a cached K or V vector of head_dim D is D/8 groups of 8; group g is rotated by
    the orthonormal 8-point Hadamard H8 / sqrt(8) before quantization, so it is
    read back as  x_g = s * H8 e_g / sqrt(8)  with one fp32 scale s per (token,
    head) vector;
  * e_g = C[i0] (e8_relaxed:1, 2 bpw) or C[i0] + s_r C[i1] (e8_relaxed:2, 4 bpw),
    both 16-bit indices into the 65,536-entry weight codebook, s_r a parameter
    (0.25 in the synthetic caches);
  * pages of page_size tokens; token t of sequence b is slot t mod page_size of
    physical page block_table[b][t // page_size];
  * grouped-query attention: query head hq reads KV head hq // (num_q_heads /
    num_kv_heads);
  * out = softmax(sm_scale * q K^T) V over the sequence's seq_len tokens, one query
    token per sequence (decode).
All arithmetic is float64.
"""

import numpy as np

from . import e8, hadamard


def h8_normalized():
    """H8 / sqrt(8), Sylvester order (the orthonormal 8-point Hadamard)."""
    return hadamard.fwht(np.eye(8)) / np.sqrt(8.0)


def dequant_vectors(idx0, idx1, scale, resid_scale):
    """Cached vectors from their indices, float64 [..., D].

    idx0, idx1: [..., D/8] codebook indices of the stages (idx1 None for one
    stage); scale: [...] per-vector scales.
    """
    c = e8.codebook(e8.ENTRIES)
    e = c[np.asarray(idx0).astype(np.int64)]                       # [..., G8, 8]
    if idx1 is not None:
        e = e + np.float64(np.float32(resid_scale)) * c[np.asarray(idx1).astype(np.int64)]
    x = e @ h8_normalized().T                                      # H8 e / sqrt(8) per group
    x = x.reshape(x.shape[:-2] + (x.shape[-2] * 8,))
    return np.asarray(scale, dtype=np.float64)[..., None] * x


def gather_sequence(cache, block_table_row, seq_len, page_size):
    """Rows 0 .. seq_len-1 of one sequence from a paged array [pages, page_size, ...]."""
    t = np.arange(seq_len)
    pages = np.asarray(block_table_row)[t // page_size]
    return np.asarray(cache)[pages, t % page_size]


def attention_decode(q, k_idx0, k_idx1, k_scale, v_idx0, v_idx1, v_scale, resid_scale, block_table, seq_lens,
                     page_size, sm_scale):
    """Decode attention over an E8-compressed paged cache, float64 [B, Hq, D].

    q: [B, Hq, D]; k_idx*/v_idx*: [pages, page_size, Hkv, D/8] (idx1 None for one
    stage); k_scale/v_scale: [pages, page_size, Hkv]; block_table: [B, max_pages];
    seq_lens: [B] (each >= 1).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = np.asarray(k_idx0).shape[2]
    G = Hq // Hkv
    out = np.empty((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        row = block_table[b]
        gi = lambda a: None if a is None else gather_sequence(a, row, L, page_size)
        K = dequant_vectors(gi(k_idx0), gi(k_idx1), gi(k_scale), resid_scale)   # [L, Hkv, D]
        V = dequant_vectors(gi(v_idx0), gi(v_idx1), gi(v_scale), resid_scale)
        for hq in range(Hq):
            h = hq // G
            s = sm_scale * (K[:, h, :] @ q[b, hq])
            p = np.exp(s - s.max())
            out[b, hq] = (p @ V[:, h, :]) / p.sum()
    return out
