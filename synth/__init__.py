"""Seeded synthetic E8RHTLinear layers and activations.

Shared by the tests and the benchmark, for both the GPU library and the CPU
oracle.  It holds the workload shapes and the random draws only: no codebook,
no transform, no dequantization.

Recipe (numpy PCG64, numpy.random.default_rng):
  * a workload has an integer seed; layer k of it draws from
    default_rng([seed, k]) in this order: sign_in (n_pad), sign_out (m_pad),
    idx0 (m_pad x n_pad/8), idx1 (same shape, when the recipe has a residual);
  * signs are 2 * integers(0, 2) - 1 as int8 (Rademacher +-1);
  * indices are uniform: integers(0, 65536) as uint16, integers(0, 256) as uint8
    for an 8-bit residual;
  * activations for batch size B draw from default_rng([seed, k, B]):
    standard_normal((B, n)) in float64, rounded once (nearest-even) to the
    activation dtype; both sides consume the rounded values;
  * weight scale s = 0.02, residual scale s_r = 0.25 for every layer.

Shapes are the checkpoints' layer shapes (SmolLM2-360M, SmolLM3-3B,
Devstral-Small 24B) with dimensions padded to the next power of two.
"""

from dataclasses import dataclass, field

import numpy as np

WSCALE = 0.02
RESID_SCALE = 0.25


def next_pow2(n):
    p = 1
    while p < n:
        p *= 2
    return p


@dataclass(frozen=True)
class LayerShape:
    name: str
    n: int
    m: int
    n_pad: int = 0
    m_pad: int = 0

    def padded(self):
        return LayerShape(self.name, self.n, self.m,
                          self.n_pad or next_pow2(self.n), self.m_pad or next_pow2(self.m))


@dataclass(frozen=True)
class Workload:
    key: str
    title: str
    seed: int
    resid_bits: int          # 0: 2 bpw, 8: 3 bpw (16 + 8), 16: 4 bpw (16 + 16)
    act_dtype: str           # "f32" | "f16" | "bf16"
    batches: tuple
    layers: tuple = field(default_factory=tuple)

    @property
    def bpw(self):
        return {0: 2, 8: 3, 16: 4}[self.resid_bits]


def _L(name, n, m):
    return LayerShape(name, n, m).padded()


WORKLOADS = {
    "tiny": Workload("tiny", "tiny E8RHTLinear 256->256, fp32, 2 bpw", 1001, 0, "f32", (1,),
                     (_L("tiny", 256, 256),)),
    "smollm2_up": Workload("smollm2_up", "SmolLM2-360M MLP up-projection 960->2560, 4 bpw, fp16",
                           1002, 16, "f16", (1, 5), (_L("up", 960, 2560),)),
    "smollm3_block": Workload("smollm3_block", "SmolLM3-3B decoder block (7 linears), 3 bpw, fp16",
                              1003, 8, "f16", (1, 5),
                              (_L("q", 2048, 2048), _L("k", 2048, 512), _L("v", 2048, 512),
                               _L("o", 2048, 2048), _L("gate", 2048, 11008), _L("up", 2048, 11008),
                               _L("down", 11008, 2048))),
    "devstral_mlp": Workload("devstral_mlp", "Devstral-Small 24B MLP (gate, up, down), 4 bpw, bf16",
                             1004, 16, "bf16", (1, 4, 16),
                             (_L("gate", 5120, 32768), _L("up", 5120, 32768), _L("down", 32768, 5120))),
    "prefill_gateup": Workload("prefill_gateup", "prefill 2048->11008, M=2048 tokens, 3 bpw, bf16",
                               1005, 8, "bf16", (2048,), (_L("gate", 2048, 11008),)),
}


@dataclass
class Layer:
    """One synthetic quantized layer (host numpy arrays)."""
    shape: LayerShape
    resid_bits: int
    sign_in: np.ndarray      # int8 [n_pad]
    sign_out: np.ndarray     # int8 [m_pad]
    idx0: np.ndarray         # uint16 [m_pad, n_pad/8]
    idx1: object             # uint8/uint16 [m_pad, n_pad/8] or None
    wscale: float = WSCALE
    resid_scale: float = RESID_SCALE
    extra: tuple = ()        # further residual stages (5-8 bpw): (bits, index array, scale) each
    block_diag: bool = False  # unpadded, block-diagonal transforms (n_pad == n, m_pad == m)

    @property
    def n(self):
        return self.shape.n

    @property
    def m(self):
        return self.shape.m

    @property
    def n_pad(self):
        return self.shape.n_pad

    @property
    def m_pad(self):
        return self.shape.m_pad

    def index_bytes(self):
        return self.idx0.nbytes + (0 if self.idx1 is None else self.idx1.nbytes) + sum(e[1].nbytes for e in self.extra)

    @property
    def bpw(self):
        return 2 + self.resid_bits // 8 + sum(b // 8 for b, _, _ in self.extra)

    def oracle_extra(self):
        """The extra stages as the oracle takes them: (index array, bits, scale)."""
        return tuple((idx, bits, scale) for bits, idx, scale in self.extra)


# bpw -> (bits of the first residual stage, bits of the further stages), glq 0.5.1,
# table "Bit widths"
RECIPES = {2: (0, ()), 3: (8, ()), 4: (16, ()), 5: (16, (8,)), 6: (16, (16,)), 7: (16, (16, 8)), 8: (16, (16, 16))}


def make_layer(shape, resid_bits, seed, k, rows=None, extra_bits=(), block_diag=False):
    """Draw layer k of a workload with the given seed.

    extra_bits: bits (8 or 16) of residual stages 2, 3 (5-8 bpw), drawn after the
    other arrays; stage j is scaled by RESID_SCALE ** j (a reading: each stage
    refines the previous one's error by the same factor).

    rows: optionally keep only the first `rows` rows of the index arrays, used
    nowhere on the measured path (the draw order is unchanged).

    block_diag: the layer is unpadded (n_pad = n, m_pad = m) for block-diagonal
    transforms; the draws keep their order, with the unpadded lengths.
    """
    shape = LayerShape(shape.name, shape.n, shape.m, shape.n, shape.m) if block_diag else shape.padded()
    rng = np.random.default_rng([seed, k])
    sign_in = (2 * rng.integers(0, 2, size=shape.n_pad) - 1).astype(np.int8)
    sign_out = (2 * rng.integers(0, 2, size=shape.m_pad) - 1).astype(np.int8)
    gshape = (shape.m_pad, shape.n_pad // 8)
    idx0 = rng.integers(0, 65536, size=gshape, dtype=np.uint16)
    idx1 = None
    if resid_bits == 8:
        idx1 = rng.integers(0, 256, size=gshape, dtype=np.uint8)
    elif resid_bits == 16:
        idx1 = rng.integers(0, 65536, size=gshape, dtype=np.uint16)
    elif resid_bits != 0:
        raise ValueError("resid_bits must be 0, 8 or 16")
    extra = []
    for j, bits in enumerate(extra_bits):
        if bits not in (8, 16) or resid_bits == 0:
            raise ValueError("extra stages are 8 or 16 bits, after a residual stage")
        idx = rng.integers(0, 256 if bits == 8 else 65536, size=gshape, dtype=np.uint8 if bits == 8 else np.uint16)
        extra.append((bits, idx, float(np.float32(RESID_SCALE ** (j + 2)))))
    return Layer(shape, resid_bits, sign_in, sign_out, idx0, idx1, extra=tuple(extra), block_diag=block_diag)


def round_to_dtype(x64, dtype):
    """Round float64 values once, nearest-even, to 'f32' | 'f16' | 'bf16'.

    Returns (values as float64, raw array in that dtype: float32, float16, or
    uint16 bf16 bit patterns).
    """
    x64 = np.asarray(x64, dtype=np.float64)
    if dtype == "f32":
        r = x64.astype(np.float32)
        return r.astype(np.float64), r
    if dtype == "f16":
        r = x64.astype(np.float16)
        return r.astype(np.float64), r
    if dtype == "bf16":
        # one rounding to 8 significant bits, ties to even (normal range only)
        mant, expo = np.frexp(x64)
        vals = np.ldexp(np.round(np.ldexp(mant, 8)), expo - 8)
        bits = (vals.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
        return vals, bits
    raise ValueError(dtype)


def make_x(n, B, dtype, seed, k):
    """Activations [B, n] for layer k: (float64 values, raw dtype array)."""
    rng = np.random.default_rng([seed, k, B])
    return round_to_dtype(rng.standard_normal((B, n)), dtype)


def workload_layers(key):
    w = WORKLOADS[key]
    return [(k, s) for k, s in enumerate(w.layers)]


def random_layer(n, m, resid_bits, seed, n_pad=None, m_pad=None, extra_bits=()):
    """A layer of arbitrary shape (tests of ragged and tiny shapes)."""
    shape = LayerShape("t", n, m, n_pad or next_pow2(max(n, 8)), m_pad or next_pow2(max(m, 8)))
    return make_layer(shape, resid_bits, seed, 0, extra_bits=extra_bits)


def block_layer(n, m, resid_bits, seed, extra_bits=()):
    """An unpadded layer with block-diagonal transforms (n, m multiples of 8)."""
    return make_layer(LayerShape("t", n, m), resid_bits, seed, 0, extra_bits=extra_bits, block_diag=True)


def recipe_layer(n, m, bpw, seed, n_pad=None, m_pad=None):
    """A layer of a 2-8 bpw recipe of the "Bit widths" table."""
    resid_bits, extra_bits = RECIPES[bpw]
    return random_layer(n, m, resid_bits, seed, n_pad, m_pad, extra_bits)


# ---- E8-compressed paged KV cache (decode attention) ------------------------------
KV_RESID_SCALE = 0.25


@dataclass
class KVCache:
    """A synthetic paged K/V cache of E8 indices (host numpy arrays).

    k_idx0 / k_idx1 / v_idx0 / v_idx1: uint16 [pages, page_size, num_kv_heads, head_dim / 8]
    (idx1 None for one stage); k_scale / v_scale: float32 [pages, page_size, num_kv_heads];
    block_table: int32 [B, max_pages]; seq_lens: int32 [B].
    """
    num_kv_heads: int
    head_dim: int
    page_size: int
    stages: int
    k_idx0: np.ndarray
    k_idx1: object
    v_idx0: np.ndarray
    v_idx1: object
    k_scale: np.ndarray
    v_scale: np.ndarray
    block_table: np.ndarray
    seq_lens: np.ndarray
    resid_scale: float = KV_RESID_SCALE

    @property
    def pages(self):
        return self.k_idx0.shape[0]

    def kv_bytes(self):
        """Bytes the decode reads: each sequence's tokens of K and V (indices and scales)."""
        per_tok = self.num_kv_heads * (self.stages * self.head_dim // 8 * 2 + 4)
        return int(2 * per_tok * int(np.sum(self.seq_lens)))


def make_kv(seq_lens, num_kv_heads, head_dim, stages, page_size, seed, spare_pages=3):
    """Draw a paged cache: default_rng([seed, 7]) in this order: the physical page of
    every logical page (a permutation of all pages, so sequences are scattered),
    k_idx0, k_idx1 (two stages), v_idx0, v_idx1, k_scale, v_scale (uniform in
    [0.5, 2), float32).  Pages beyond the sequences' own (spare_pages) hold indices
    too and are never referenced."""
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    B = len(seq_lens)
    need = [(int(L) + page_size - 1) // page_size for L in seq_lens]
    max_pages = max(need)
    pages = sum(need) + spare_pages
    rng = np.random.default_rng([seed, 7])
    perm = rng.permutation(pages).astype(np.int32)
    table = np.zeros((B, max_pages), dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, :need[b]] = perm[off:off + need[b]]
        off += need[b]
    shape = (pages, page_size, num_kv_heads, head_dim // 8)
    draw = lambda: rng.integers(0, 65536, size=shape, dtype=np.uint16)
    k0 = draw()
    k1 = draw() if stages == 2 else None
    v0 = draw()
    v1 = draw() if stages == 2 else None
    ks = rng.uniform(0.5, 2.0, size=shape[:3]).astype(np.float32)
    vs = rng.uniform(0.5, 2.0, size=shape[:3]).astype(np.float32)
    return KVCache(num_kv_heads, head_dim, page_size, stages, k0, k1, v0, v1, ks, vs, table, seq_lens)


def make_q(B, num_q_heads, head_dim, dtype, seed):
    """Decode queries [B, num_q_heads, head_dim]: N(0, 1) from default_rng([seed, 8]),
    rounded once to dtype.  Returns (float64 values, raw array)."""
    rng = np.random.default_rng([seed, 8])
    v, raw = round_to_dtype(rng.standard_normal((B, num_q_heads * head_dim)), dtype)
    return v.reshape(B, num_q_heads, head_dim), raw.reshape(B, num_q_heads, head_dim)
