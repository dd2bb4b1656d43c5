"""E8 lattice codebook by enumeration (oracle; test infrastructure only).

glq 0.5.1 (PyPI project page), "How it works", item 1: the codebook is 2^16 points
of the 8-dimensional E8 lattice, the innermost ones (norm values 0 up to the
seventh), and each group of 8 weights is stored as a 16-bit index into it.  "Inference kernels" and "How it
works", item 4, put the codebook at 1 MB, i.e. 65,536 x 8 fp16 values.

E8 (Conway & Sloane, cited in the page's "Acknowledgments") is the union of
  D8          = { v in Z^8         : sum(v) even }
  D8 + 1/2    = { v in (Z + 1/2)^8 : sum(v) even }.
Its shells are the sets of equal squared norm 0, 2, 4, ..., and the k-th nonzero
shell has 240 * sigma_3(k) points.

Readings where the page is silent (each listed in the design notes):
  * the seven shells are norm^2 0, 2, ..., 12 with the origin included; shells
    0..10 are taken whole (56,881 points) and the last 8,655 entries come from
    the norm^2 = 12 shell;
  * order: ascending squared norm, ties broken lexicographically on the
    coordinate values, v0 most significant, ascending;
  * the 8-bit residual codebook is the first 256 entries of the same order and
    the 16-bit residual codebook is the primary codebook itself.

Work is done on doubled coordinates t = 2v, which are exact integers.
"""

import functools

import numpy as np

ENTRIES = 65536
RESID8_ENTRIES = 256


def e8_ball_doubled(max_norm2=12):
    """All E8 points v with |v|^2 <= max_norm2, returned as int64 rows t = 2v.

    Integer type: t even, |t_j| <= 2*floor(sqrt(max_norm2)), sum(t)/2 even.
    Half type:    t odd, sum(t)/2 even, i.e. sum(t) = 0 mod 4.
    Pinned by the shell-count and membership tests (theta series of E8).
    """
    bound = int(np.floor(np.sqrt(max_norm2)))
    lim = 4 * max_norm2  # |t|^2 = 4 |v|^2
    # integer-type points: v_j in [-bound, bound]
    r = np.arange(-bound, bound + 1, dtype=np.int64) * 2
    grid = np.stack(np.meshgrid(*([r] * 8), indexing="ij"), axis=-1).reshape(-1, 8)
    keep = ((grid * grid).sum(1) <= lim) & ((grid.sum(1) // 2) % 2 == 0)
    ints = grid[keep]
    # half-type points: v_j in {+-1/2, +-3/2, ...} with |v_j| <= sqrt(max_norm2)
    odd = np.arange(1, 2 * bound + 2, 2, dtype=np.int64)
    odd = odd[odd * odd <= lim]
    h = np.concatenate([-odd[::-1], odd])
    grid = np.stack(np.meshgrid(*([h] * 8), indexing="ij"), axis=-1).reshape(-1, 8)
    keep = ((grid * grid).sum(1) <= lim) & (grid.sum(1) % 4 == 0)
    halves = grid[keep]
    return np.concatenate([ints, halves], axis=0)


def sort_codebook_order(t):
    """Sort doubled points by (|v|^2, v0, v1, ..., v7) ascending."""
    norm2 = (t * t).sum(1)
    keys = [t[:, j] for j in range(7, -1, -1)] + [norm2]  # lexsort: last key primary
    return t[np.lexsort(keys)]


@functools.lru_cache(maxsize=1)
def _sorted_ball():
    t = sort_codebook_order(e8_ball_doubled(12))
    t.flags.writeable = False
    return t


def codebook_doubled(entries=ENTRIES):
    """The first `entries` E8 points in codebook order, as int64 t = 2v [entries, 8]."""
    t = _sorted_ball()
    if entries > len(t):
        raise ValueError("codebook larger than the enumerated ball")
    return t[:entries].copy()


def codebook(entries=ENTRIES):
    """Codebook values v as float64 [entries, 8] (exact: v in Z/2)."""
    return codebook_doubled(entries).astype(np.float64) / 2.0


def codebook_fp16_bits(entries=ENTRIES):
    """Codebook as fp16 bit patterns, uint16 [entries, 8].

    Every coordinate is a multiple of 1/2 with |v| <= 3, so fp16 holds it exactly
    (the "1 MB" codebook of the Inference kernels section).
    """
    v = codebook(entries)
    h = v.astype(np.float16)
    assert np.array_equal(h.astype(np.float64), v)
    return h.view(np.uint16)


def residual_codebook(bits):
    """Residual-stage codebook for an 8- or 16-bit residual index, float64 [2**bits, 8].

    "How it works", item 1: 8-bit (256-entry) or 16-bit (E8) residual codebooks.
    Reading: both are prefixes of the primary codebook order.
    """
    if bits == 8:
        return codebook(RESID8_ENTRIES)
    if bits == 16:
        return codebook(ENTRIES)
    raise ValueError("residual index width must be 8 or 16 bits")
