"""The codebook pack, built on the host by the library (glq_codebook_pack).

The decode kernel gathers codewords from the pack's LDS image: a 256-entry page
table and 4-byte slots of eight signed 4-bit values 2c, each negation-symmetric
shell stored once.  These tests resolve every index the way the kernel does
(m = -(desc & 1); byte address ((4 (i & 255)) ^ m) + desc mod 2^32, the word
complemented when m is all ones) and compare with the oracle's codebook; they also check the
integer identity the kernel's dot products rest on.  glq 0.5.1, "How it works", item 1;
"Inference kernels".
"""
import ctypes
import os

import numpy as np
import pytest

glq = pytest.importorskip("e8_lattice_codebook_amd")
from e8_lattice_codebook_amd import _lib  # noqa: E402
from oracle import e8  # noqa: E402

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="library not built")

LDS_BUDGET_DWORDS = 39680


def build(cb_bits):
    lib = _lib.load()
    n = cb_bits.shape[0]
    nbytes = lib.glq_codebook_pack_bytes(n)
    out = np.zeros(nbytes, dtype=np.uint8)
    st = lib.glq_codebook_pack(np.ascontiguousarray(cb_bits).ctypes.data_as(ctypes.c_void_p), n,
                               out.ctypes.data_as(ctypes.c_void_p), nbytes)
    return st, out


def image_of(pack, entries):
    hdr = pack[:256].view(np.uint32)
    off = (256 + entries * 8 + 255) // 256 * 256
    img = pack[off:].view(np.uint32)[:hdr[3]]
    return hdr, img


# coordinate e of a slot word sits in nibble (e >> 1) + 4 (e & 1): nibbles j and j + 4
# hold the adjacent coordinates 2j and 2j + 1
LANE_NIBBLE = np.array([(e >> 1) + 4 * (e & 1) for e in range(8)], dtype=np.uint32)


def nibbles_signed(words):
    w = np.asarray(words, dtype=np.uint32)[:, None]
    v = ((w >> (4 * LANE_NIBBLE)) & 15).astype(np.int64)
    return np.where(v >= 8, v - 16, v)


def resolve(img, idx):
    # the kernel's lookup: m = -(desc & 1), image byte offset ((4 (i & 255)) ^ m) + desc
    # in 32-bit arithmetic, the word complemented when m is all ones
    idx = np.asarray(idx, dtype=np.int64)
    desc = img[idx >> 8].astype(np.int64)
    m = np.where(desc & 1, -1, 0)
    ba = ((((idx & 0xFF) * 4) ^ (m & 0xFFFFFFFF)) + desc) & 0xFFFFFFFF
    assert (ba % 4 == 0).all() and (ba >= 1024).all()
    words = img[ba // 4]
    return words, m


def test_e8_pack_resolves_every_index():
    st, pack = build(e8.codebook_fp16_bits())
    assert st == 0
    hdr, img = image_of(pack, 65536)
    assert hdr[0] == 0x32514C47 and hdr[2] == 65536
    assert hdr[3] <= LDS_BUDGET_DWORDS            # fits the LDS budget of the decode kernel
    assert hdr[3] * 4 < 155 * 1024
    t = (2 * e8.codebook()).astype(np.int64)
    # int8 table
    assert np.array_equal(pack[256:256 + 65536 * 8].view(np.int8).reshape(-1, 8), t)
    words, m = resolve(img, np.arange(65536))
    vals = nibbles_signed(words)
    got = np.where(m[:, None] == -1, -vals, vals)
    assert np.array_equal(got, t)
    # the stored form of a complemented entry is ~n (lanes -2c - 1), as the kernel reads it
    mirrored = int((m == -1).sum())
    assert 27000 < mirrored < 28441        # lower halves of the symmetric shells


def test_resid8_pack_is_direct():
    st, pack = build(e8.codebook_fp16_bits(256))
    assert st == 0
    hdr, img = image_of(pack, 256)
    t = (2 * e8.codebook(256)).astype(np.int64)
    assert np.array_equal(nibbles_signed(img[256:512]), t)       # slot = index
    words, m = resolve(img, np.arange(256))
    assert (m == 0).all()


def test_pack_rejects_unrepresentable():
    cb = e8.codebook_fp16_bits(256).copy()
    cb[3, 2] = np.float16(0.25).view(np.uint16)     # not a multiple of 1/2
    assert build(cb)[0] == 8
    cb = e8.codebook_fp16_bits(256).copy()
    cb[7, 0] = np.float16(5.0).view(np.uint16)      # 2c = 10 does not fit 4 bits
    assert build(cb)[0] == 8
    cb = e8.codebook_fp16_bits(256).copy()
    cb[7, 0] = np.float16(np.inf).view(np.uint16)
    assert build(cb)[0] == 8
    # a random table has no shell symmetry: 65,536 direct slots do not fit in LDS
    rng = np.random.default_rng(0)
    cb = (rng.integers(-6, 7, size=(65536, 8)) / 2).astype(np.float16).view(np.uint16)
    assert build(cb)[0] == 8


def test_complement_identity_of_the_dot_products():
    # sum_j (~n)_j d_j = -sum_j n_j d_j - sum_j d_j for signed 4-bit lanes
    rng = np.random.default_rng(1)
    n = rng.integers(-6, 7, size=(1000, 8))
    d = rng.integers(-8, 8, size=(1000, 8))
    comp = -n - 1                                   # lanes of n ^ 0xF
    assert np.array_equal((comp * d).sum(1), -(n * d).sum(1) - d.sum(1))
    # four balanced base-16 digit planes reproduce |U| <= 30583
    U = rng.integers(-30583, 30584, size=5000)
    planes, r = [], U.copy()
    for _ in range(4):
        dd = ((r + 8) & 15) - 8
        planes.append(dd)
        r = (r - dd) >> 4
    assert (r == 0).all()
    assert np.array_equal(sum(p * 16 ** k for k, p in enumerate(planes)), U)
    assert all((p >= -8).all() and (p <= 7).all() for p in planes)


# ---- slot-code format -----------------------------------------------------------
# Header word 5: slot image dwords, word 6: delta.  After the 256-dword-aligned
# int8 table come the page image and the slot image (39,680 dwords each), then
# code_of [entries] uint16 (256-byte aligned) and index_of [65536] uint16.
IMAGE_MAX = 39680
SLOT_IMAGE_MAX = 37632  # a larger slot image gets no slot format


def slot_tables(pack, entries):
    hdr = pack[:256].view(np.uint32)
    img_off = (256 + entries * 8 + 255) // 256 * 256
    slot_off = img_off + IMAGE_MAX * 4
    code_off = slot_off + IMAGE_MAX * 4
    index_off = code_off + (entries * 2 + 255) // 256 * 256
    slots = pack[slot_off:slot_off + int(hdr[5]) * 4].view(np.uint32)
    code_of = pack[code_off:code_off + entries * 2].view(np.uint16)
    index_of = pack[index_off:index_off + 65536 * 2].view(np.uint16)
    return hdr, slots, code_of, index_of


def decode_codes(slots, delta, codes):
    # the kernels' lookup: c as int16, m = c >> 15, slot (c ^ m) + (m & delta),
    # the entry is the slot word's lanes, negated when m is all ones
    c = np.asarray(codes, dtype=np.uint16).view(np.int16).astype(np.int64)
    m = c >> 15
    P = (c ^ m) + (m & delta)
    assert (P >= 0).all() and (P < slots.size).all()
    vals = nibbles_signed(slots[P])
    return np.where(m[:, None] == -1, -vals, vals)


def test_e8_slot_codes_decode_every_index():
    st, pack = build(e8.codebook_fp16_bits())
    assert st == 0
    hdr, slots, code_of, index_of = slot_tables(pack, 65536)
    assert hdr[1] == 5                                # pack format
    # 28,440 negation pairs share slots: delta = 32768 - 28440; the 8,656 entries
    # without a partner (origin, the 8,655 of norm^2 12) fill both lone regions
    assert hdr[6] == 32768 - 28440 and hdr[5] == 32768 + 4328
    assert hdr[5] <= SLOT_IMAGE_MAX                   # fits beside the prefill kernel's codeword tiles
    assert np.array_equal(np.sort(code_of), np.arange(65536))   # a bijection
    assert np.array_equal(index_of[code_of], np.arange(65536))   # index_of inverts code_of
    t = (2 * e8.codebook()).astype(np.int64)
    assert np.array_equal(decode_codes(slots, int(hdr[6]), code_of), t)


def test_slot_codes_of_negation_pairs_share_a_slot():
    st, pack = build(e8.codebook_fp16_bits())
    hdr, slots, code_of, index_of = slot_tables(pack, 65536)
    cb = (2 * e8.codebook()).astype(np.int64)
    # idx 1 = (-1,-1,0,...) and idx 240 = (1,1,0,...) are negatives (hand pins)
    assert np.array_equal(cb[1], -cb[240])
    c1, c240 = int(code_of[1]), int(code_of[240])
    assert (c1 >= 32768) != (c240 >= 32768)           # one plain, one complemented
    s = lambda c: (np.int16(np.uint16(c)) ^ (np.int16(np.uint16(c)) >> 15)) + ((np.int16(np.uint16(c)) >> 15) & int(hdr[6]))
    assert s(c1) == s(c240)
    # the origin has no partner and is stored plain
    assert int(code_of[0]) < 32768
