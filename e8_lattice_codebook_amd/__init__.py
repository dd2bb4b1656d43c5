"""E8RHTLinear (GLQ E8 lattice codebook layers) on AMD MI355X / gfx950.

A thin Python binding over the C ABI of libglq_mi355x.so (include/glq.h):
every step of the layer runs in the library's HIP kernels; torch supplies
device memory and the current HIP stream, and this module only marshals
arguments.  The entry points keep the C names without the glq_ prefix.
"""

import ctypes

import numpy as np
import torch

from . import _lib
from ._lib import GLQ_BF16, GLQ_F16, GLQ_F32, GLQError, GlqLayer  # noqa: F401

CODEBOOK_ENTRIES = 65536
RESID8_ENTRIES = 256
INDEX_CODEBOOK, INDEX_SLOT = 0, 1  # glq_index_format

_DT = {torch.float32: GLQ_F32, torch.float16: GLQ_F16, torch.bfloat16: GLQ_BF16}


def lib():
    return _lib.load()


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dt(dtype):
    if dtype not in _DT:
        raise TypeError("dtype must be float32, float16 or bfloat16")
    return _DT[dtype]


def _workspace(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ---- codebooks ------------------------------------------------------------------
def e8_codebook(entries=CODEBOOK_ENTRIES):
    """The E8 codebook as fp16 bit patterns, host numpy uint16 [entries, 8] (glq_e8_codebook)."""
    out = np.empty((entries, 8), dtype=np.uint16)
    _lib.check(lib().glq_e8_codebook(out.ctypes.data_as(ctypes.c_void_p), entries), "glq_e8_codebook")
    return out


def codebook_pack(cb_fp16_bits, device="cuda"):
    """Pack an fp16 codebook [entries, 8] (host uint16 bits) for the kernels (glq_codebook_pack).

    Built on the host by the library, then copied to `device`.
    """
    cb = np.ascontiguousarray(cb_fp16_bits, dtype=np.uint16)
    entries = cb.shape[0]
    nbytes = lib().glq_codebook_pack_bytes(entries)
    host = np.zeros(nbytes, dtype=np.uint8)
    _lib.check(lib().glq_codebook_pack(cb.ctypes.data_as(ctypes.c_void_p), entries,
                                       host.ctypes.data_as(ctypes.c_void_p), nbytes), "glq_codebook_pack")
    return torch.from_numpy(host).to(device)


class Codebooks:
    """The primary (65,536-entry) and 8-bit residual (256-entry) packs on one device."""

    def __init__(self, device="cuda"):
        self.device = torch.device(device)
        self.fp16 = e8_codebook(CODEBOOK_ENTRIES)
        self.primary = codebook_pack(self.fp16, self.device)
        self.resid8 = codebook_pack(self.fp16[:RESID8_ENTRIES], self.device)

    def residual(self, resid_bits):
        return {0: None, 8: self.resid8, 16: self.primary}[resid_bits]


# ---- layers ---------------------------------------------------------------------
class QuantizedLayer:
    """Device copy of one layer (signs, index arrays) plus its glq_layer descriptor."""

    def __init__(self, n, m, n_pad, m_pad, resid_bits, sign_in, sign_out, idx0, idx1, codebooks,
                 wscale=0.02, resid_scale=0.25, device=None, index_format=INDEX_CODEBOOK, extra=()):
        """extra: further residual stages of 5-8 bpw, (bits, index array, scale) each."""
        device = torch.device(device) if device is not None else codebooks.device
        self.n, self.m, self.n_pad, self.m_pad = int(n), int(m), int(n_pad), int(m_pad)
        self.resid_bits = int(resid_bits)
        self.wscale, self.resid_scale = float(wscale), float(resid_scale)
        self.sign_in = _to_dev(sign_in, torch.int8, device)
        self.sign_out = _to_dev(sign_out, torch.int8, device)
        self.idx0 = _to_dev(idx0, torch.int16, device)
        if idx1 is None:
            self.idx1 = None
        else:
            i1_8 = idx1.dtype == torch.uint8 if isinstance(idx1, torch.Tensor) else np.asarray(idx1).dtype == np.uint8
            self.idx1 = _to_dev(idx1, torch.uint8 if i1_8 else torch.int16, device)
        self.codebooks = codebooks
        self.device = device
        self.index_format = int(index_format)
        self.extra = tuple((int(b), _to_dev(i, torch.uint8 if int(b) == 8 else torch.int16, device), float(sc))
                           for b, i, sc in extra)
        self.desc = GlqLayer(self.n, self.n_pad, self.m, self.m_pad, self.resid_bits, self.wscale, self.resid_scale,
                             self.sign_in.data_ptr(), self.sign_out.data_ptr(), self.idx0.data_ptr(),
                             0 if self.idx1 is None else self.idx1.data_ptr(), codebooks.primary.data_ptr(),
                             0 if resid_bits == 0 else codebooks.residual(resid_bits).data_ptr(), self.index_format)
        self.desc.n_extra = len(self.extra)
        for k, (b, i, sc) in enumerate(self.extra):
            self.desc.extra_bits[k] = b
            self.desc.extra_scale[k] = sc
            self.desc.extra_idx[k] = i.data_ptr()
            if b == 8:
                self.desc.cb8_pack = codebooks.resid8.data_ptr()

    @classmethod
    def from_synth(cls, layer, codebooks, device=None):
        return cls(layer.n, layer.m, layer.n_pad, layer.m_pad, layer.resid_bits, layer.sign_in, layer.sign_out,
                   layer.idx0, layer.idx1, codebooks, layer.wscale, layer.resid_scale, device,
                   extra=getattr(layer, "extra", ()))

    def to_slot_codes(self):
        """The same layer with its 16-bit index arrays relabelled as slot codes
        (glq_slot_codes): idx0, idx1 when the residual stage is 16-bit, and the
        16-bit further stages."""
        if self.index_format == INDEX_SLOT:
            return self
        idx0 = slot_codes(self.idx0, self.codebooks)
        idx1 = self.idx1
        if self.resid_bits == 16:
            idx1 = slot_codes(self.idx1, self.codebooks)
        extra = tuple((b, slot_codes(i, self.codebooks) if b == 16 else i, sc) for b, i, sc in self.extra)
        return QuantizedLayer(self.n, self.m, self.n_pad, self.m_pad, self.resid_bits, self.sign_in, self.sign_out,
                              idx0, idx1, self.codebooks, self.wscale, self.resid_scale, self.device, INDEX_SLOT,
                              extra=extra)

    def index_bytes(self):
        return (self.idx0.numel() * 2 + (0 if self.idx1 is None else self.idx1.numel() * self.idx1.element_size())
                + sum(i.numel() * i.element_size() for _, i, _ in self.extra))


def _to_dev(a, dtype, device):
    if isinstance(a, torch.Tensor):
        return a.to(device).contiguous()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device=device, dtype=dtype).contiguous()


# ---- operations -----------------------------------------------------------------
def slot_codes(idx, codebooks, out=None):
    """codes[i] = the slot code of codebook index idx[i] (glq_slot_codes); int16/uint16 tensors."""
    idx = idx.contiguous()
    codes = out if out is not None else torch.empty_like(idx)
    _lib.check(lib().glq_slot_codes(codebooks.primary.data_ptr(), _ptr(idx), idx.numel(), _ptr(codes),
                                    _stream(idx.device)), "glq_slot_codes")
    return codes


def input_rht(x, n_pad, sign_in, u_dtype=torch.float32, out=None):
    """u = H (sign_in * [x, 0]) / sqrt(n_pad) per row of x [B, n] (glq_input_rht)."""
    B, n = x.shape
    x = x.contiguous()
    u = out if out is not None else torch.empty((B, n_pad), dtype=u_dtype, device=x.device)
    ws_n = lib().glq_input_rht_workspace_bytes(B, n_pad, _dt(u.dtype))
    ws = _workspace(ws_n, x.device) if ws_n else None
    _lib.check(lib().glq_input_rht(_ptr(x), _dt(x.dtype), B, n, n_pad, _ptr(sign_in), _ptr(u), _dt(u.dtype),
                                   _ptr(ws), ws_n, _stream(x.device)), "glq_input_rht")
    return u


def output_rht(z_parts, m, sign_out, y_dtype=torch.float32, out=None, workspace=None):
    """y = (sign_out * H (sum_s z_parts[s]) / sqrt(m_pad))[:, :m] (glq_output_rht)."""
    S, B, m_pad = z_parts.shape
    z_parts = z_parts.contiguous()
    y = out if out is not None else torch.empty((B, m), dtype=y_dtype, device=z_parts.device)
    y_dtype = y.dtype
    ws_n = lib().glq_output_rht_workspace_bytes(B, m_pad)
    ws = None
    if ws_n:
        ws = workspace if workspace is not None else _workspace(ws_n, z_parts.device)
        ws_n = ws.numel()
    _lib.check(lib().glq_output_rht(_ptr(z_parts), S, B, m, m_pad, _ptr(sign_out), _ptr(y), _dt(y_dtype), _ptr(ws),
                                    ws_n, _stream(y.device)), "glq_output_rht")
    return y


def e8_dequant(layer, dtype=torch.float32):
    """W~ [m_pad, n_pad] (glq_e8_dequant; tests and debugging only)."""
    w = torch.empty((layer.m_pad, layer.n_pad), dtype=dtype, device=layer.device)
    _lib.check(lib().glq_e8_dequant(ctypes.byref(layer.desc), _ptr(w), _dt(dtype), _stream(layer.device)),
               "glq_e8_dequant")
    return w


def e8_matmul_splits(layer, B):
    return int(lib().glq_e8_matmul_splits(ctypes.byref(layer.desc), B))


def e8_matmul(layer, u, out=None, workspace=None):
    """Split partial sums z_parts [S, B, m_pad] of z = u W~^T (glq_e8_matmul).

    u is fp32 [B, n_pad] for B <= 16 and fp16 for larger B.
    """
    B = u.shape[0]
    u = u.contiguous()
    S = e8_matmul_splits(layer, B)
    z = out if out is not None else torch.empty((S, B, layer.m_pad), dtype=torch.float32, device=u.device)
    ws_n = int(lib().glq_e8_matmul_workspace_bytes(ctypes.byref(layer.desc), B))
    ws = None
    if ws_n:
        ws = workspace if workspace is not None else _workspace(ws_n, u.device)
        ws_n = ws.numel()
    _lib.check(lib().glq_e8_matmul(ctypes.byref(layer.desc), _ptr(u), _dt(u.dtype), B, _ptr(z), _ptr(ws), ws_n,
                                   _stream(u.device)), "glq_e8_matmul")
    return z


def e8_matmul_prefill_supported(layer):
    return bool(lib().glq_e8_matmul_prefill_supported(ctypes.byref(layer.desc)))


def input_rht_prefill(x, n_pad, sign_in, out=None):
    """fp16 u = H (sign_in * [x, 0]) / sqrt(n_pad) in the prefill matmul's fragment
    order, as a flat uint8 tensor of prefill_u_bytes (glq_input_rht_prefill)."""
    B, n = x.shape
    x = x.contiguous()
    nbytes = int(lib().glq_prefill_u_bytes(B, n_pad))
    u = out if out is not None else torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    ws_n = lib().glq_input_rht_workspace_bytes(B, n_pad, GLQ_F16)
    ws = _workspace(ws_n, x.device) if ws_n else None
    _lib.check(lib().glq_input_rht_prefill(_ptr(x), _dt(x.dtype), B, n, n_pad, _ptr(sign_in), _ptr(u), _ptr(ws),
                                           ws_n, _stream(x.device)), "glq_input_rht_prefill")
    return u


def e8_matmul_prefill(layer, u_frag, B, out=None):
    """z [1, B, m_pad] fp32 = u W~^T from fragment-order fp16 u (glq_e8_matmul_prefill)."""
    z = out if out is not None else torch.empty((1, B, layer.m_pad), dtype=torch.float32, device=u_frag.device)
    _lib.check(lib().glq_e8_matmul_prefill(ctypes.byref(layer.desc), _ptr(u_frag), B, _ptr(z),
                                           _stream(u_frag.device)), "glq_e8_matmul_prefill")
    return z


def linear_workspace_bytes(layer, B):
    return int(lib().glq_e8rht_linear_workspace_bytes(ctypes.byref(layer.desc), B))


def linear_workspace(layer, B, device=None):
    """A workspace for e8rht_linear(layer, x[B]) (scratch; reusable by later calls on
    the same stream, whatever the layer or B, if large enough)."""
    device = device if device is not None else layer.device
    return torch.empty(max(linear_workspace_bytes(layer, B), 1), dtype=torch.uint8, device=device)


def e8rht_linear(layer, x, y_dtype=None, workspace=None, out=None):
    """The E8RHTLinear forward y [B, m] from x [B, n] (glq_e8rht_linear).

    workspace: from linear_workspace (or any device buffer of linear_workspace_bytes)."""
    B = x.shape[0]
    x = x.contiguous()
    y_dtype = y_dtype or x.dtype
    y = out if out is not None else torch.empty((B, layer.m), dtype=y_dtype, device=x.device)
    if workspace is None:
        workspace = linear_workspace(layer, B, x.device)
    _lib.check(lib().glq_e8rht_linear(ctypes.byref(layer.desc), _ptr(x), _dt(x.dtype), B, _ptr(y), _dt(y.dtype),
                                      _ptr(workspace), workspace.numel(), _stream(x.device)), "glq_e8rht_linear")
    return y


GROUP_MAX = 4  # GLQ_GROUP_MAX


def _layer_array(layers):
    arr = (GlqLayer * len(layers))()
    for k, ql in enumerate(layers):
        arr[k] = ql.desc
    return arr


def linear_group_workspace_bytes(layers, B):
    return int(lib().glq_e8rht_linear_group_workspace_bytes(_layer_array(layers), len(layers), B))


def e8rht_linear_group(layers, xs, y_dtype=None, workspace=None, outs=None):
    """The E8RHTLinear forwards y_k [B, m_k] of several layers (glq_e8rht_linear_group):
    one pair of launches at B = 1 when the layers allow it, else one call per layer.

    xs: one input per layer (the same tensor may be passed for several)."""
    if len(xs) != len(layers):
        raise ValueError("one input per layer")
    xs = [x.contiguous() for x in xs]
    B = xs[0].shape[0]
    y_dtype = y_dtype or xs[0].dtype
    ys = outs if outs is not None else [torch.empty((B, ql.m), dtype=y_dtype, device=xs[0].device) for ql in layers]
    arr = _layer_array(layers)
    if workspace is None:
        nb = int(lib().glq_e8rht_linear_group_workspace_bytes(arr, len(layers), B))
        workspace = torch.empty(max(nb, 1), dtype=torch.uint8, device=xs[0].device)
    xp = (ctypes.c_void_p * len(xs))(*[_ptr(x) for x in xs])
    yp = (ctypes.c_void_p * len(ys))(*[_ptr(y) for y in ys])
    _lib.check(lib().glq_e8rht_linear_group(arr, len(layers), xp, _dt(xs[0].dtype), B, yp, _dt(ys[0].dtype),
                                            _ptr(workspace), workspace.numel(), _stream(xs[0].device)),
               "glq_e8rht_linear_group")
    return ys


NOALLOC_SCRATCH_BYTES = 64 << 20  # GLQ_NOALLOC_SCRATCH_BYTES


def e8rht_linear_noalloc(layer, x, y_dtype=None, out=None):
    """The E8RHTLinear forward with the library's own device scratch as its workspace
    (glq_e8rht_linear_noalloc): nothing is allocated by the call when `out` is given.
    Calls that overlap on one device race on that scratch."""
    B = x.shape[0]
    x = x.contiguous()
    y_dtype = y_dtype or x.dtype
    y = out if out is not None else torch.empty((B, layer.m), dtype=y_dtype, device=x.device)
    _lib.check(lib().glq_e8rht_linear_noalloc(ctypes.byref(layer.desc), _ptr(x), _dt(x.dtype), B, _ptr(y),
                                              _dt(y.dtype), _stream(x.device)), "glq_e8rht_linear_noalloc")
    return y


class KVCache:
    """An E8-compressed paged K/V cache on the device (glq_kv_cache).

    k_idx / v_idx: one or two uint16 arrays [pages, page_size, num_kv_heads, head_dim/8]
    per stage; k_scale / v_scale: fp32 [pages, page_size, num_kv_heads].
    """

    def __init__(self, k_idx, v_idx, k_scale, v_scale, codebooks, resid_scale=0.25, device=None,
                 index_format=INDEX_CODEBOOK):
        device = device if device is not None else codebooks.device
        self.codebooks = codebooks
        self.device = torch.device(device)
        self.k_idx = [_to_dev(a, torch.int16, device) for a in k_idx]
        self.v_idx = [_to_dev(a, torch.int16, device) for a in v_idx]
        self.k_scale = _to_dev(k_scale, torch.float32, device)
        self.v_scale = _to_dev(v_scale, torch.float32, device)
        pages, page_size, heads, groups = self.k_idx[0].shape
        self.num_pages, self.page_size, self.num_kv_heads, self.head_dim = pages, page_size, heads, groups * 8
        self.stages = len(self.k_idx)
        self.resid_scale = float(resid_scale)
        self.index_format = int(index_format)
        d = _lib.GlqKvCache()
        d.num_pages, d.page_size, d.num_kv_heads, d.head_dim = pages, page_size, heads, groups * 8
        d.stages, d.resid_scale, d.index_format = self.stages, self.resid_scale, self.index_format
        for s in range(self.stages):
            d.k_idx[s] = self.k_idx[s].data_ptr()
            d.v_idx[s] = self.v_idx[s].data_ptr()
        d.k_scale, d.v_scale = self.k_scale.data_ptr(), self.v_scale.data_ptr()
        d.cb_pack = codebooks.primary.data_ptr()
        self.desc = d

    @classmethod
    def from_synth(cls, cache, codebooks, device=None):
        k = [cache.k_idx0] + ([] if cache.k_idx1 is None else [cache.k_idx1])
        v = [cache.v_idx0] + ([] if cache.v_idx1 is None else [cache.v_idx1])
        return cls(k, v, cache.k_scale, cache.v_scale, codebooks, cache.resid_scale, device)

    def to_slot_codes(self):
        """The same cache with every index relabelled as a slot code (glq_slot_codes)."""
        return KVCache([slot_codes(a, self.codebooks) for a in self.k_idx],
                       [slot_codes(a, self.codebooks) for a in self.v_idx], self.k_scale, self.v_scale,
                       self.codebooks, self.resid_scale, self.device, INDEX_SLOT)

    def nbytes(self):
        return sum(a.numel() * 2 for a in self.k_idx + self.v_idx) + 4 * (self.k_scale.numel() + self.v_scale.numel())


def e8kv_attention_workspace_bytes(cache, B, num_q_heads, max_seq_len):
    return int(lib().glq_e8kv_attention_workspace_bytes(ctypes.byref(cache.desc), B, num_q_heads, max_seq_len))


def e8kv_attention_decode(cache, q, block_table, seq_lens, max_seq_len, sm_scale=None, out_dtype=None,
                          workspace=None, out=None):
    """Decode attention out [B, Hq, D] over the compressed cache (glq_e8kv_attention_decode).

    q [B, Hq, D]; block_table int32 [B, max_pages]; seq_lens int32 [B] (device tensors)."""
    B, Hq, D = q.shape
    q = q.contiguous()
    sm_scale = float(D) ** -0.5 if sm_scale is None else float(sm_scale)
    out_dtype = out_dtype or q.dtype
    o = out if out is not None else torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    ws_n = e8kv_attention_workspace_bytes(cache, B, Hq, max_seq_len)
    ws = workspace if workspace is not None else _workspace(max(ws_n, 1), q.device)
    _lib.check(lib().glq_e8kv_attention_decode(ctypes.byref(cache.desc), _ptr(q), _dt(q.dtype), B, Hq,
                                               _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
                                               int(max_seq_len), sm_scale, _ptr(o), _dt(o.dtype), _ptr(ws),
                                               ws.numel(), _stream(q.device)), "glq_e8kv_attention_decode")
    return o
