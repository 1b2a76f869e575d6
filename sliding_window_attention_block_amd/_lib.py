"""ctypes declarations of the C ABI in include/bsattn.h.

The shared library is the in-tree ``libbsattn.so`` built by ``build.py``.  There
is no fallback: if the library is missing, loading raises.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# BSATTN_LIBRARY names another build of the same library (the host-sanitizer
# build the CPU tests load); there is no other implementation to fall back to
LIB_PATH = os.environ.get("BSATTN_LIBRARY") or os.path.join(_HERE, "libbsattn.so")

BSATTN_OK = 0
BSATTN_ERR_INVALID = 1
BSATTN_ERR_UNSUPPORTED = 2
BSATTN_ERR_HIP = 3
BSATTN_ERR_WORKSPACE = 4
BSATTN_F32 = 0
BSATTN_BF16 = 1
BSATTN_FP4_E2M1 = 2
BSATTN_NOALLOC_SCRATCH_BYTES = 16 << 20  # include/bsattn.h: the allocation-free step's scratch

EXPORTS = (
    "bsattn_build_summaries",
    "bsattn_append_kv",
    "bsattn_select_prefill",
    "bsattn_select_exact",
    "bsattn_sparse_prefill",
    "bsattn_select_topk",
    "bsattn_decode_workspace_bytes",
    "bsattn_decode",
    "bsattn_decode_step",
    "bsattn_decode_step_noalloc",
    "bsattn_prefill",
    "bsattn_prefill_workspace_bytes",
    "bsattn_prefill_dilated",
    "bsattn_probe_gather",
    "bsattn_status_string",
    "bsattn_last_error",
    "bsattn_version",
)


class Shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("n_ctx", ctypes.c_int32),
        ("kv_capacity", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
    ]


_lib = None

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_st = ctypes.c_int
_pshape = ctypes.POINTER(Shape)


class PagedKV(ctypes.Structure):
    """bsattn_paged_kv: block table (device int32 [B, max_pages]) of a paged K/V cache."""
    _fields_ = [("block_table", ctypes.c_void_p), ("page_tokens", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("n_pages", ctypes.c_int32)]


_ppaged = ctypes.POINTER(PagedKV)
_pi32 = ctypes.POINTER(ctypes.c_int32)


def load():
    """Load libbsattn.so (once).  Raises OSError when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise OSError(f"{LIB_PATH} is missing: build it with "
                      "`python -m sliding_window_attention_block_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.bsattn_build_summaries.argtypes = [_pshape, _vp, _i32, _i32, _i32, _i32, _vp, _i32, _vp, _i32,
                                           _vp, _vp, _i32, _ppaged, _vp]
    lib.bsattn_build_summaries.restype = _st
    lib.bsattn_append_kv.argtypes = [_pshape, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _i32, _vp, _i32, _vp,
                                     _vp, _i32, _ppaged, _vp]
    lib.bsattn_append_kv.restype = _st
    lib.bsattn_select_prefill.argtypes = [_pshape, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp]
    lib.bsattn_select_prefill.restype = _st
    lib.bsattn_select_exact.argtypes = [_pshape, _vp, _vp, _i32, _i32, _i32, _i32, _pi32, _i32, _vp, _vp, _vp]
    lib.bsattn_select_exact.restype = _st
    lib.bsattn_sparse_prefill.argtypes = [_pshape, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp]
    lib.bsattn_sparse_prefill.restype = _st
    lib.bsattn_select_topk.argtypes = [_pshape, _vp, _vp, _i32, _vp, _i32, _vp, _vp, _i32, _i32, _i32,
                                       _i32, _i32, _i32, _pi32, _i32, _vp, _vp, _vp]
    lib.bsattn_select_topk.restype = _st
    lib.bsattn_decode_workspace_bytes.argtypes = [_pshape, _i32, _i32, _i32, _i32]
    lib.bsattn_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.bsattn_decode.argtypes = [_pshape, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _pi32, _i32,
                                  _vp, _vp, _vp, ctypes.c_size_t, _ppaged, _vp]
    lib.bsattn_decode.restype = _st
    lib.bsattn_decode_step.argtypes = [_pshape, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _vp, _vp, _i32,
                                       _i32, _i32, _i32, _i32, _i32, _pi32, _i32, _vp, _vp, _vp, _vp,
                                       _vp, ctypes.c_size_t, _ppaged, _vp]
    lib.bsattn_decode_step.restype = _st
    lib.bsattn_decode_step_noalloc.argtypes = [_pshape, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _vp, _vp, _i32,
                                               _i32, _i32, _i32, _i32, _i32, _pi32, _i32, _vp, _vp, _vp, _vp,
                                               _ppaged, _vp]
    lib.bsattn_decode_step_noalloc.restype = _st
    lib.bsattn_prefill.argtypes = [_pshape, _vp, _vp, _vp, _i32, _i32, _i32, _pi32, _i32,
                                   _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.bsattn_prefill.restype = _st
    lib.bsattn_prefill_dilated.argtypes = [_pshape, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp]
    lib.bsattn_prefill_dilated.restype = _st
    lib.bsattn_prefill_workspace_bytes.argtypes = [_pshape, _i32]
    lib.bsattn_prefill_workspace_bytes.restype = ctypes.c_size_t
    lib.bsattn_probe_gather.argtypes = [_pshape, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp]
    lib.bsattn_probe_gather.restype = _st
    lib.bsattn_status_string.argtypes = [_st]
    lib.bsattn_status_string.restype = ctypes.c_char_p
    lib.bsattn_last_error.argtypes = []
    lib.bsattn_last_error.restype = ctypes.c_char_p
    lib.bsattn_version.argtypes = []
    lib.bsattn_version.restype = ctypes.c_char_p
    _lib = lib
    return lib
