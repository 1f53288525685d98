"""ctypes declarations of the C ABI in include/kvq.h (libkvq.so, built for gfx950).

Loading fails loudly when the library is missing: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq.so")


def use_phase_timer_build(path=None) -> None:
    """Load the profiling variant libkvq_phases.so (same sources, decode phase timers; or the
    build at `path`) instead of libkvq.so; only the phase profiler calls this, before anything
    loads the library."""
    global _LIB_PATH
    if _lib is not None:
        raise RuntimeError("the library is already loaded")
    _LIB_PATH = path or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq_phases.so")

KVQ_OK, KVQ_ERR_INVALID_ARG, KVQ_ERR_UNSUPPORTED, KVQ_ERR_ALIGNMENT, KVQ_ERR_WORKSPACE, KVQ_ERR_HIP = range(6)
KVQ_BF16, KVQ_F32 = 0, 1
KVQ_LAYER_INT, KVQ_LAYER_FP8, KVQ_LAYER_BF16 = 0, 1, 2

EXPORTED = ("kvq_status_str", "kvq_format_version", "kvq_head_page_bytes", "kvq_page_bytes",
            "kvq_equiv_bits", "kvq_validate_model", "kvq_pack", "kvq_append", "kvq_dequant",
            "kvq_decode_workspace_bytes", "kvq_workspace_init", "kvq_decode_attn", "kvq_append_decode_attn",
            "kvq_append_decode_attn_noalloc", "kvq_noalloc_scratch_bytes")


class KvqModel(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("k_bits", ctypes.POINTER(ctypes.c_uint8)), ("v_bits", ctypes.POINTER(ctypes.c_uint8)),
                ("k_mode", ctypes.POINTER(ctypes.c_uint8)), ("layer_format", ctypes.POINTER(ctypes.c_uint8))]


class KvqLayerCache(ctypes.Structure):
    _fields_ = [("pages", ctypes.c_void_p), ("n_pages", ctypes.c_int64),
                ("resid_k", ctypes.c_void_p), ("resid_v", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("batch", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("fp8_scales", ctypes.c_void_p)]


class KvqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what} failed: {status_str(status)}")


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(hipcc, gfx950); there is no CPU fallback")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        mp, cp = ctypes.POINTER(KvqModel), ctypes.POINTER(KvqLayerCache)
        L.kvq_status_str.argtypes = [ctypes.c_int]
        L.kvq_status_str.restype = ctypes.c_char_p
        L.kvq_format_version.argtypes = []
        L.kvq_format_version.restype = i32
        L.kvq_head_page_bytes.argtypes = [i32, i32]
        L.kvq_head_page_bytes.restype = sz
        L.kvq_page_bytes.argtypes = [mp, i32]
        L.kvq_page_bytes.restype = sz
        L.kvq_equiv_bits.argtypes = [mp]
        L.kvq_equiv_bits.restype = ctypes.c_double
        L.kvq_validate_model.argtypes = [mp]
        L.kvq_validate_model.restype = ctypes.c_int
        L.kvq_pack.argtypes = [mp, i32, cp, ctypes.c_int, vp, vp, i32, vp, vp]
        L.kvq_pack.restype = ctypes.c_int
        L.kvq_append.argtypes = [mp, i32, cp, vp, vp, vp, vp]
        L.kvq_append.restype = ctypes.c_int
        L.kvq_dequant.argtypes = [mp, i32, cp, i32, vp, vp, vp, vp]
        L.kvq_dequant.restype = ctypes.c_int
        L.kvq_decode_workspace_bytes.argtypes = [mp, i32, i32, i32]
        L.kvq_decode_workspace_bytes.restype = sz
        L.kvq_workspace_init.argtypes = [vp, sz, vp]
        L.kvq_workspace_init.restype = ctypes.c_int
        L.kvq_decode_attn.argtypes = [mp, i32, cp, ctypes.c_int, vp, vp, i32, i32, vp, vp, vp, sz, vp]
        L.kvq_decode_attn.restype = ctypes.c_int
        L.kvq_append_decode_attn.argtypes = [mp, i32, cp, vp, vp, vp, ctypes.c_int, vp, i32, i32, vp, vp, vp, sz, vp]
        L.kvq_append_decode_attn.restype = ctypes.c_int
        if hasattr(L, "kvq_append_decode_attn_noalloc"):
            L.kvq_append_decode_attn_noalloc.argtypes = [mp, i32, cp, vp, vp, vp, ctypes.c_int, vp, i32, i32, vp, vp, vp]
            L.kvq_append_decode_attn_noalloc.restype = ctypes.c_int
            L.kvq_noalloc_scratch_bytes.argtypes = [mp, i32, i32, i32]
            L.kvq_noalloc_scratch_bytes.restype = sz
        if hasattr(L, "kvq_profile_set_phase_buffer"):
            L.kvq_profile_set_phase_buffer.argtypes = [vp, sz]
            L.kvq_profile_set_phase_buffer.restype = None
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().kvq_status_str(int(status)).decode()


def check(status: int, what: str) -> None:
    if status != KVQ_OK:
        raise KvqError(status, what)
