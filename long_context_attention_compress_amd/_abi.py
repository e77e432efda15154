"""ctypes mirror of include/v4attn.h and the loader of libv4attn.so.

The library is loaded from this package's directory only; if it is missing
the import of the binding fails loudly (there is no other implementation of
these operations on the product path).
"""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), 'libv4attn.so')

V4A_OK, V4A_EINVAL, V4A_ENULL, V4A_EALIGN, V4A_EFORMAT, V4A_EWORKSPACE, V4A_EHIP = 0, -1, -2, -3, -4, -5, -6
KV_F32, KV_E4M3_BF16 = 0, 1
NOALLOC_SCRATCH_BYTES = 32 << 20   # V4A_NOALLOC_SCRATCH_BYTES
IK_F32, IK_MXFP4 = 0, 1
ACT_F32, ACT_BF16 = 0, 1
POOL_BLOCK, POOL_OVERLAP, POOL_ROPE_AFTER, POOL_CHANNEL_GATE = 0, 1, 2, 3

c_i32, c_i64, c_p, c_f, c_d = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_double


class Plane(ctypes.Structure):
    _fields_ = [('ptr', c_p), ('row_stride', c_i64), ('batch_stride', c_i64)]


class KvStoreC(ctypes.Structure):
    _fields_ = [('fmt', c_i32), ('dim', c_i32), ('rows', c_i64), ('ring', c_i64),
                ('f32', Plane), ('nope', Plane), ('rope', Plane), ('scale', Plane)]


class IkStoreC(ctypes.Structure):
    _fields_ = [('fmt', c_i32), ('dim', c_i32), ('rows', c_i64),
                ('f32', Plane), ('e2m1', Plane), ('e8m0', Plane)]


class CompressArgs(ctypes.Structure):
    _fields_ = [('B', c_i32), ('t_new', c_i32), ('pos0', c_i64), ('m', c_i32), ('act_fmt', c_i32),
                ('rope_base', c_d), ('raw_k', c_p), ('raw_v', c_p), ('gate', c_p), ('pos_bias', c_p),
                ('raw_ik', c_p), ('k_out', ctypes.POINTER(KvStoreC)), ('v_out', ctypes.POINTER(KvStoreC)),
                ('ik_out', ctypes.POINTER(IkStoreC)), ('block_end', c_p), ('variant', c_i32)]


class IndexArgs(ctypes.Structure):
    _fields_ = [('B', c_i32), ('Tq', c_i32), ('H_I', c_i32), ('k', c_i32), ('m', c_i32),
                ('q_pos', c_p), ('iq', c_p), ('iq_scale', c_p), ('w', c_p),
                ('keys', ctypes.POINTER(IkStoreC)), ('out_idx', c_p), ('out_score', c_p)]


class AttnArgs(ctypes.Structure):
    _fields_ = [('B', c_i32), ('Tq', c_i32), ('H_q', c_i32), ('dim', c_i32), ('q_pos', c_p),
                ('q_fmt', c_i32), ('q', c_p),
                ('ent_k', ctypes.POINTER(KvStoreC)), ('ent_v', ctypes.POINTER(KvStoreC)), ('m', c_i32),
                ('win_k', ctypes.POINTER(KvStoreC)), ('win_v', ctypes.POINTER(KvStoreC)), ('W', c_i32),
                ('sm_scale', c_f), ('rope_base', c_d), ('o_fmt', c_i32), ('o', c_p), ('lse', c_p),
                ('append_k', c_p), ('append_v', c_p)]


EXPORTS = {
    'csa_compress': (c_i32, [ctypes.POINTER(CompressArgs), c_p]),
    'lightning_index_topk_workspace': (ctypes.c_size_t, [ctypes.POINTER(IndexArgs)]),
    'lightning_index_topk': (c_i32, [ctypes.POINTER(IndexArgs), c_p, ctypes.c_size_t, c_p]),
    'lightning_index_topk_noalloc': (c_i32, [ctypes.POINTER(IndexArgs), c_p]),
    'sparse_window_attn_workspace': (ctypes.c_size_t, [ctypes.POINTER(AttnArgs), c_i32]),
    'sparse_window_attn': (c_i32, [ctypes.POINTER(AttnArgs), c_p, c_i32, c_p, ctypes.c_size_t, c_p]),
    'hca_attn_workspace': (ctypes.c_size_t, [ctypes.POINTER(AttnArgs), c_i64]),
    'hca_attn': (c_i32, [ctypes.POINTER(AttnArgs), c_i64, c_p, ctypes.c_size_t, c_p]),
    'v4a_workspace_init': (c_i32, [c_p, ctypes.c_size_t, c_p]),
    'v4a_strerror': (ctypes.c_char_p, [c_i32]),
    'v4a_last_error': (ctypes.c_char_p, []),
    'v4a_version': (ctypes.c_char_p, []),
}

_lib = None


def load():
    """Load libv4attn.so from the package directory (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f'{LIB_PATH} is missing: build it with '
                              'python -m long_context_attention_compress_amd.build')
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib
