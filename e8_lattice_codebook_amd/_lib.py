"""ctypes view of the C ABI in include/glq.h (libglq_mi355x.so, built in-tree).

Loading fails loudly when the library has not been built: there is no other
implementation of these operations in this package.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# GLQ_LIB_VARIANT=debug | asan selects a debug build of the same library (see build.py)
_VARIANT = os.environ.get("GLQ_LIB_VARIANT", "release")
LIB_NAME = {"release": "libglq_mi355x.so", "debug": "libglq_mi355x_debug.so",
            "asan": "libglq_mi355x_asan.so"}.get(_VARIANT, "libglq_mi355x.so")
LIB_PATH = os.path.join(_HERE, LIB_NAME)

GLQ_F32, GLQ_F16, GLQ_BF16 = 0, 1, 2
STATUS_NAMES = {
    0: "GLQ_OK", 1: "GLQ_ERR_NULL", 2: "GLQ_ERR_SHAPE", 3: "GLQ_ERR_DTYPE", 4: "GLQ_ERR_RECIPE",
    5: "GLQ_ERR_ALIGN", 6: "GLQ_ERR_WORKSPACE", 7: "GLQ_ERR_HIP", 8: "GLQ_ERR_CODEBOOK",
}

# every function the header declares, with (restype, argtypes)
c_i64, c_i32, c_f32, c_vp, c_sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class GlqLayer(ctypes.Structure):
    _fields_ = [
        ("n", c_i64), ("n_pad", c_i64), ("m", c_i64), ("m_pad", c_i64),
        ("resid_bits", c_i32), ("wscale", c_f32), ("resid_scale", c_f32),
        ("sign_in", c_vp), ("sign_out", c_vp), ("idx0", c_vp), ("idx1", c_vp),
        ("cb_pack", c_vp), ("cb2_pack", c_vp), ("index_format", c_i32),
        ("n_extra", c_i32), ("extra_bits", c_i32 * 2), ("extra_scale", c_f32 * 2), ("extra_idx", c_vp * 2),
        ("cb8_pack", c_vp),
    ]


_LP = ctypes.POINTER(GlqLayer)


class GlqKvCache(ctypes.Structure):
    _fields_ = [
        ("num_pages", c_i64), ("page_size", c_i32), ("num_kv_heads", c_i32), ("head_dim", c_i32),
        ("stages", c_i32), ("resid_scale", c_f32), ("index_format", c_i32),
        ("k_idx", c_vp * 2), ("v_idx", c_vp * 2), ("k_scale", c_vp), ("v_scale", c_vp), ("cb_pack", c_vp),
    ]


_KP = ctypes.POINTER(GlqKvCache)

SIGNATURES = {
    "glq_abi_version": (ctypes.c_int, []),
    "glq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "glq_debug_violations": (c_i64, []),
    "glq_e8_codebook": (ctypes.c_int, [c_vp, c_i64]),
    "glq_codebook_pack_bytes": (c_sz, [c_i64]),
    "glq_codebook_pack": (ctypes.c_int, [c_vp, c_i64, c_vp, c_sz]),
    "glq_input_rht_workspace_bytes": (c_sz, [c_i64, c_i64, ctypes.c_int]),
    "glq_input_rht": (ctypes.c_int, [c_vp, ctypes.c_int, c_i64, c_i64, c_i64, c_vp, c_vp, ctypes.c_int, c_vp, c_sz,
                                     c_vp]),
    "glq_output_rht_workspace_bytes": (c_sz, [c_i64, c_i64]),
    "glq_output_rht": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp, ctypes.c_int, c_vp, c_sz, c_vp]),
    "glq_e8_dequant": (ctypes.c_int, [_LP, c_vp, ctypes.c_int, c_vp]),
    "glq_slot_codes": (ctypes.c_int, [c_vp, c_vp, c_i64, c_vp, c_vp]),
    "glq_e8_matmul_splits": (c_i64, [_LP, c_i64]),
    "glq_e8_matmul_workspace_bytes": (c_sz, [_LP, c_i64]),
    "glq_e8_matmul": (ctypes.c_int, [_LP, c_vp, ctypes.c_int, c_i64, c_vp, c_vp, c_sz, c_vp]),
    "glq_prefill_u_bytes": (c_sz, [c_i64, c_i64]),
    "glq_prefill_row_exp_offset": (c_sz, [c_i64, c_i64]),
    "glq_e8_matmul_prefill_supported": (ctypes.c_int, [_LP]),
    "glq_input_rht_prefill": (ctypes.c_int, [c_vp, ctypes.c_int, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "glq_e8_matmul_prefill": (ctypes.c_int, [_LP, c_vp, c_i64, c_vp, c_vp]),
    "glq_e8rht_linear_workspace_bytes": (c_sz, [_LP, c_i64]),
    "glq_e8rht_linear": (ctypes.c_int, [_LP, c_vp, ctypes.c_int, c_i64, c_vp, ctypes.c_int, c_vp, c_sz, c_vp]),
    "glq_e8rht_linear_noalloc": (ctypes.c_int, [_LP, c_vp, ctypes.c_int, c_i64, c_vp, ctypes.c_int, c_vp]),
    "glq_e8rht_linear_group_workspace_bytes": (c_sz, [_LP, c_i32, c_i64]),
    "glq_e8rht_linear_group": (ctypes.c_int, [_LP, c_i32, ctypes.POINTER(c_vp), ctypes.c_int, c_i64,
                                              ctypes.POINTER(c_vp), ctypes.c_int, c_vp, c_sz, c_vp]),
    "glq_e8kv_attention_workspace_bytes": (c_sz, [_KP, c_i64, c_i32, c_i64]),
    "glq_e8kv_attention_decode": (ctypes.c_int, [_KP, c_vp, ctypes.c_int, c_i64, c_i32, c_vp, c_i64, c_vp, c_i64,
                                                 c_f32, c_vp, ctypes.c_int, c_vp, c_sz, c_vp]),
}

_lib = None


def load():
    """Load the library once; raise ImportError if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("%s is not built: run e8_lattice_codebook_amd/build.py "
                          "(or __graft_entry__.build()) first" % LIB_NAME)
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class GLQError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))
        msg = load().glq_status_string(status).decode()
        super().__init__("%s: %s (%s)" % (where, self.name, msg))


def check(status, where):
    if status != 0:
        raise GLQError(status, where)
