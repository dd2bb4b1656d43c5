"""Host-side checks of the C ABI: the library loads, exports what include/glq.h
declares, builds the same codebook as the oracle, and rejects bad arguments
before launching anything.  No GPU is touched here.
"""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "glq.h")

glq = pytest.importorskip("e8_lattice_codebook_amd")
from e8_lattice_codebook_amd import _lib  # noqa: E402

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="library not built")

NO_GPU = not torch.cuda.is_available()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(glq_[a-z0-9_]+)\s*\(", text)))


def test_header_declarations_are_exported():
    lib = _lib.load()
    names = declared_functions()
    assert len(names) >= 14
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(_lib.SIGNATURES)


def test_abi_version_and_status_strings():
    lib = _lib.load()
    assert lib.glq_abi_version() == 5
    for s in range(9):
        assert lib.glq_status_string(s)
    assert lib.glq_status_string(0) == b"ok"


def test_library_codebook_equals_oracle_bit_for_bit():
    from oracle import e8
    got = glq.e8_codebook(65536)
    assert np.array_equal(got, e8.codebook_fp16_bits(65536))
    assert np.array_equal(glq.e8_codebook(256), e8.codebook_fp16_bits(256))


def test_codebook_builder_rejects_bad_sizes():
    lib = _lib.load()
    buf = np.zeros(16, dtype=np.uint16)
    assert lib.glq_e8_codebook(None, 1) == 1
    assert lib.glq_e8_codebook(buf.ctypes.data_as(ctypes.c_void_p), 0) == 2
    assert lib.glq_e8_codebook(buf.ctypes.data_as(ctypes.c_void_p), 65537) == 2


def test_workspace_queries():
    lib = _lib.load()
    assert lib.glq_codebook_pack_bytes(65536) >= 256 + 65536 * 8 + 151 * 1024
    assert lib.glq_codebook_pack_bytes(0) == 0
    # one workgroup per row up to 16384 points when there are at least 128 rows
    assert lib.glq_input_rht_workspace_bytes(128, 16384, 1) == 0
    assert lib.glq_input_rht_workspace_bytes(128, 32768, 1) == 128 * 32768 * 4
    assert lib.glq_input_rht_workspace_bytes(128, 32768, 0) == 0
    assert lib.glq_output_rht_workspace_bytes(130, 16384) == 0
    assert lib.glq_output_rht_workspace_bytes(130, 32768) == 130 * 32768 * 4
    # fewer rows: rows of at least 8192 points are split into segments of 4096 or
    # more (two passes through scratch) so that a launch has enough workgroups; fp32
    # u of one block is its own scratch
    assert lib.glq_input_rht_workspace_bytes(2, 16384, 1) == 2 * 16384 * 4
    assert lib.glq_input_rht_workspace_bytes(2, 16384, 0) == 0
    assert lib.glq_output_rht_workspace_bytes(3, 8192) == 3 * 8192 * 4
    assert lib.glq_output_rht_workspace_bytes(3, 4096) == 0
    # block-diagonal lengths: scratch when a block runs in two passes, also for fp32 u
    assert lib.glq_input_rht_workspace_bytes(128, 16384 + 64, 1) == 0
    assert lib.glq_input_rht_workspace_bytes(128, 32768 + 1024, 0) == 128 * (32768 + 1024) * 4
    assert lib.glq_output_rht_workspace_bytes(130, 32768 + 64) == 130 * (32768 + 64) * 4
    assert lib.glq_input_rht_workspace_bytes(2, 100, 0) == 0   # not a transform length
    L = fake_layer(n=5120, n_pad=8192, m=32768, m_pad=32768, resid_bits=16)
    one = lib.glq_e8rht_linear_workspace_bytes(ctypes.byref(L), 1)
    # B = 1 path: 2 split partials of m_pad fp32
    assert one >= 2 * 32768 * 4
    dec = lib.glq_e8rht_linear_workspace_bytes(ctypes.byref(L), 2)
    # staged decode: u fp32 + split partials + output-transform scratch
    assert dec >= 2 * 8192 * 4 + 2 * 32768 * 4 + 2 * 32768 * 4
    pre = lib.glq_e8rht_linear_workspace_bytes(ctypes.byref(L), 2048)
    assert pre >= 2048 * 8192 * 2 + 2 * 2048 * 32768 * 4
    # fragment-order u: whole 16-row blocks; k-steps in blocks of 4 (n_pad a multiple of
    # 128); then, at a 256-byte boundary, one int32 exponent per row of those blocks
    r256 = lambda v: (v + 255) // 256 * 256
    assert lib.glq_prefill_row_exp_offset(17, 2688) == r256(32 * 2688 * 2)
    assert lib.glq_prefill_u_bytes(17, 2688) == r256(32 * 2688 * 2) + r256(32 * 4)
    assert lib.glq_prefill_row_exp_offset(33, 2688) == r256(48 * 2688 * 2)
    assert lib.glq_prefill_u_bytes(33, 2688) == r256(48 * 2688 * 2) + r256(48 * 4)
    assert lib.glq_prefill_u_bytes(17, 320) == 0
    assert lib.glq_prefill_row_exp_offset(17, 320) == 0
    assert lib.glq_prefill_u_bytes(0, 1024) == 0


# ---- validation: fake, never-dereferenced device addresses --------------------
A = 1 << 20  # 256-byte aligned fake address


def fake_layer(n=256, n_pad=256, m=256, m_pad=256, resid_bits=0, **kw):
    L = _lib.GlqLayer(n, n_pad, m, m_pad, resid_bits, 0.02, 0.25, A, A, A, A if resid_bits else 0, A,
                      A if resid_bits else 0)
    for k, v in kw.items():
        setattr(L, k, v)
    return L


def linear_status(L, B=1, x=A, y=A, xdt=0, ydt=0, ws=A, ws_n=1 << 40):
    return _lib.load().glq_e8rht_linear(ctypes.byref(L), x, xdt, B, y, ydt, ws, ws_n, None)


def group_status(layers, count=None, x=A, y=A, B=1, ws=A, ws_n=1 << 40):
    arr = (_lib.GlqLayer * max(len(layers), 1))(*layers)
    n = len(layers) if count is None else count
    xs = (ctypes.c_void_p * max(n, 1))(*([x] * max(n, 1)))
    ys = (ctypes.c_void_p * max(n, 1))(*([y] * max(n, 1)))
    return _lib.load().glq_e8rht_linear_group(arr, n, xs, 0, B, ys, 0, ws, ws_n, None)


@pytest.mark.skipif(not NO_GPU, reason="fake-pointer validation runs only where no GPU exists")
class TestValidation:
    def test_group(self):
        lib = _lib.load()
        L = fake_layer()
        assert group_status([L], count=0) == 2
        assert group_status([L] * 5) == 2
        assert lib.glq_e8rht_linear_group(None, 1, None, 0, 1, None, 0, A, 1 << 40, None) == 1
        assert group_status([L, fake_layer(idx0=None)]) == 1      # any layer's validation fails: nothing runs
        assert group_status([L, fake_layer(resid_bits=4)]) == 4
        assert group_status([L, L], x=None) == 1
        assert group_status([L, L], B=0) == 2
        assert group_status([L, L], ws_n=16) == 6
        # one z-partial region per layer at B = 1 (one grouped launch), the largest
        # single-layer workspace otherwise
        arr = (_lib.GlqLayer * 2)(L, L)
        one = lib.glq_e8rht_linear_workspace_bytes(ctypes.byref(L), 1)
        assert lib.glq_e8rht_linear_group_workspace_bytes(arr, 2, 1) == 2 * one
        assert lib.glq_e8rht_linear_group_workspace_bytes(arr, 2, 5) == lib.glq_e8rht_linear_workspace_bytes(
            ctypes.byref(L), 5)
        assert lib.glq_e8rht_linear_group_workspace_bytes(arr, 0, 1) == 0
        assert group_status([L, L]) == 7                          # valid: no GPU to launch on

    def test_null_pointers(self):
        assert linear_status(fake_layer(idx0=None)) == 1
        assert linear_status(fake_layer(cb_pack=None)) == 1
        assert linear_status(fake_layer(sign_in=None)) == 1
        assert linear_status(fake_layer(), x=None) == 1
        assert linear_status(fake_layer(), y=None) == 1
        assert linear_status(fake_layer(resid_bits=8, idx1=None)) == 1
        assert linear_status(fake_layer(resid_bits=8, cb2_pack=None)) == 1

    def test_shapes(self):
        assert linear_status(fake_layer(n_pad=384, n=384)) == 7   # block-diagonal 256 + 128: valid, no GPU to launch on
        assert linear_status(fake_layer(n_pad=392, n=392)) == 2   # neither a power of two nor a multiple of 64
        assert linear_status(fake_layer(m_pad=11008, m=11008)) == 7
        assert linear_status(fake_layer(m_pad=(1 << 20) + 64)) == 2
        assert linear_status(fake_layer(n_pad=4, n=4)) == 2       # below 8
        assert linear_status(fake_layer(m_pad=1 << 21)) == 2      # above 2^20
        assert linear_status(fake_layer(n=257)) == 2              # n > n_pad
        assert linear_status(fake_layer(m=0)) == 2
        assert linear_status(fake_layer(), B=0) == 2

    def test_recipe_dtype_align_workspace(self):
        assert linear_status(fake_layer(resid_bits=4)) == 4
        assert linear_status(fake_layer(), xdt=7) == 3
        assert linear_status(fake_layer(), ydt=-1) == 3
        assert linear_status(fake_layer(idx0=A + 2)) == 5
        assert linear_status(fake_layer(cb_pack=A + 16)) == 5
        assert linear_status(fake_layer(), ws=None) == 6
        assert linear_status(fake_layer(), ws_n=16) == 6
        assert linear_status(fake_layer(), ws=A + 8) == 5

    def test_other_entry_points(self):
        lib = _lib.load()
        assert lib.glq_input_rht(A, 0, 1, 300, 256, A, A, 0, None, 0, None) == 2
        assert lib.glq_input_rht(A, 0, 1, 256, 256, None, A, 0, None, 0, None) == 1
        assert lib.glq_input_rht(A, 0, 1, 256, 256, A, A, 5, None, 0, None) == 3
        assert lib.glq_input_rht(A, 0, 1, 256, 32768, A, A, 1, None, 0, None) == 6
        assert lib.glq_output_rht(A, 0, 1, 256, 256, A, A, 0, None, 0, None) == 2
        assert lib.glq_output_rht(A, 1, 1, 256, 32768, A, A, 0, None, 0, None) == 6
        assert lib.glq_e8_dequant(ctypes.byref(fake_layer()), A + 4, 0, None) == 5
        assert lib.glq_e8_dequant(ctypes.byref(fake_layer(resid_bits=3)), A, 0, None) == 4
        assert lib.glq_e8_matmul(ctypes.byref(fake_layer()), A, 0, 17, A, A, 1 << 30, None) == 3
        assert lib.glq_e8_matmul(ctypes.byref(fake_layer()), A, 1, 16, A, A, 1 << 30, None) == 3
        assert lib.glq_e8_matmul(ctypes.byref(fake_layer()), A, 0, 0, A, A, 1 << 30, None) == 2
        assert lib.glq_e8_matmul(ctypes.byref(fake_layer()), A + 4, 0, 1, A, A, 1 << 30, None) == 5
        assert lib.glq_e8_matmul(ctypes.byref(fake_layer()), A, 0, 1, A, None, 0, None) == 6
        assert lib.glq_e8_matmul(ctypes.byref(fake_layer()), A, 0, 1, A, A, 8, None) == 6
        assert lib.glq_e8_matmul_splits(ctypes.byref(fake_layer(n_pad=32768)), 1) == 8
        assert lib.glq_e8_matmul_splits(ctypes.byref(fake_layer(n_pad=32768)), 17) == 1
        # fragment-order input transform: n_pad >= 256 and a multiple of 128
        assert lib.glq_input_rht_prefill(A, 0, 17, 300, 320, A, A, None, 0, None) == 2
        assert lib.glq_input_rht_prefill(A, 0, 17, 100, 128, A, A, None, 0, None) == 2
        assert lib.glq_input_rht_prefill(A, 0, 17, 300, 384, A, A + 8, None, 0, None) == 5


    def test_index_format(self):
        lib = _lib.load()
        assert linear_status(fake_layer(index_format=2)) == 4
        assert linear_status(fake_layer(index_format=-1)) == 4
        # slot codes of a 16-bit residual stage need the primary pack there too
        assert linear_status(fake_layer(resid_bits=16, index_format=1, cb2_pack=A + 256)) == 4
        assert lib.glq_slot_codes(None, A, 8, A, None) == 1
        assert lib.glq_slot_codes(A, None, 8, A, None) == 1
        assert lib.glq_slot_codes(A, A, -1, A, None) == 2
        assert lib.glq_slot_codes(A + 16, A, 8, A, None) == 5
        assert lib.glq_slot_codes(A, A + 1, 8, A, None) == 5
        assert lib.glq_slot_codes(A, None, 0, None, None) == 0  # nothing to do

    def test_further_stages(self):
        def multi(n_extra, bits, **kw):
            L = fake_layer(resid_bits=16, cb2_pack=A, n_extra=n_extra)
            for k, b in enumerate(bits):
                L.extra_bits[k] = b
                L.extra_scale[k] = 0.25 ** (k + 2)
                L.extra_idx[k] = A
            L.cb8_pack = A
            for k, v in kw.items():
                setattr(L, k, v)
            return L
        assert linear_status(multi(3, [16, 16])) == 4              # at most two further stages
        assert linear_status(multi(2, [8, 16])) == 4               # 16 bits for the first of two
        assert linear_status(multi(1, [4])) == 4
        assert linear_status(multi(1, [16], resid_bits=8)) == 4    # after a 16-bit residual stage only
        assert linear_status(multi(1, [16], cb2_pack=A + 256)) == 4
        assert linear_status(multi(1, [8], cb8_pack=None)) == 1
        assert linear_status(multi(1, [8], cb8_pack=A + 16)) == 5
        L = multi(1, [16])
        L.extra_idx[0] = None
        assert linear_status(L) == 1
        L = multi(1, [16])
        L.extra_idx[0] = A + 2
        assert linear_status(L) == 5
        L = multi(1, [16])
        L.extra_scale[0] = 0.0
        assert linear_status(L) == 4


def fake_kv(**kw):
    kv = _lib.GlqKvCache()
    kv.num_pages, kv.page_size, kv.num_kv_heads, kv.head_dim, kv.stages = 64, 16, 4, 128, 2
    kv.resid_scale, kv.index_format = 0.25, 0
    kv.k_idx[0] = kv.k_idx[1] = kv.v_idx[0] = kv.v_idx[1] = A
    kv.k_scale = kv.v_scale = kv.cb_pack = A
    for k, v in kw.items():
        setattr(kv, k, v)
    return kv


def kv_status(kv, B=2, hq=16, bt=A, lens=A, max_len=1000, q=A, out=A, qdt=2, odt=2, ws=A, ws_n=1 << 40):
    return _lib.load().glq_e8kv_attention_decode(ctypes.byref(kv), q, qdt, B, hq, bt, 64, lens, max_len, 0.088, out,
                                                 odt, ws, ws_n, None)


def test_kv_workspace_query():
    lib = _lib.load()
    kv = fake_kv()
    n = lib.glq_e8kv_attention_workspace_bytes(ctypes.byref(kv), 2, 16, 1000)
    # at least one chunk per (sequence, KV head): G * (D + 2) floats each
    assert n >= 2 * 4 * 4 * (128 + 2) * 4
    assert lib.glq_e8kv_attention_workspace_bytes(ctypes.byref(kv), 2, 12, 1000) == 0   # 12 / 4 = 3 heads per group
    assert lib.glq_e8kv_attention_workspace_bytes(ctypes.byref(kv), 2, 16, 0) == 0


@pytest.mark.skipif(not NO_GPU, reason="fake-pointer validation runs only where no GPU exists")
def test_kv_validation():
    assert kv_status(fake_kv()) == 7                         # valid: no GPU to launch on
    assert kv_status(fake_kv(cb_pack=None)) == 1
    assert kv_status(fake_kv(), q=None) == 1
    assert kv_status(fake_kv(), lens=None) == 1
    assert kv_status(fake_kv(stages=3)) == 4
    assert kv_status(fake_kv(index_format=2)) == 4
    assert kv_status(fake_kv(head_dim=96)) == 2
    assert kv_status(fake_kv(page_size=24)) == 2
    assert kv_status(fake_kv(page_size=2048)) == 2
    assert kv_status(fake_kv(), hq=12) == 2                   # 3 query heads per KV head
    assert kv_status(fake_kv(), hq=64) == 2                   # 16 per KV head
    assert kv_status(fake_kv(), max_len=0) == 2
    assert kv_status(fake_kv(), qdt=5) == 3
    assert kv_status(fake_kv(cb_pack=A + 16)) == 5
    assert kv_status(fake_kv(), bt=A + 2) == 5
    assert kv_status(fake_kv(), ws=None) == 6
    assert kv_status(fake_kv(), ws_n=16) == 6
    kv1 = fake_kv(stages=1)
    kv1.k_idx[1] = 0
    assert kv_status(kv1) == 7                               # one stage: the second arrays are unused
    kv2 = fake_kv()
    kv2.v_idx[1] = 0
    assert kv_status(kv2) == 1
