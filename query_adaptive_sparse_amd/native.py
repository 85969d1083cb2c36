"""ctypes binding of libsparse_decode.so (include/sparse_decode.h, include/sparse_prefill.h), same names.

Argument marshalling only: structs mirror the C ABI, functions forward to the
library and raise on a non-OK status. The library must be built
(``python -m query_adaptive_sparse_amd.build``); loading fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libsparse_decode.so")

SD_OK, SD_EINVAL, SD_EUNSUPPORTED, SD_EWORKSPACE, SD_EHIP = range(5)
SD_F32, SD_BF16 = 0, 1
SD_TOPK, SD_TOPP, SD_HIER_TOPK, SD_COVERAGE = 0, 1, 2, 3
SD_ROUTE_SUMMARY, SD_ROUTE_PROXY = 0, 1

STATUS_NAMES = {0: "SD_OK", 1: "SD_EINVAL", 2: "SD_EUNSUPPORTED", 3: "SD_EWORKSPACE", 4: "SD_EHIP"}

EXPORTS = ("sparse_decode_init", "sparse_decode_num_levels", "sparse_decode_attend_blocks",
           "sparse_decode_score_chunks", "sparse_decode_select",
           "sparse_decode_attend", "sparse_decode_combine", "sparse_decode_step", "sparse_decode_step_static",
           "sparse_decode_selection_view",
           "sparse_decode_last_error", "sparse_decode_destroy",
           "sparse_prefill_init", "sparse_prefill_select", "sparse_prefill_attend", "sparse_prefill_view",
           "sparse_prefill_destroy",
           "sparse_gist_prefill_init", "sparse_gist_prefill_attend", "sparse_gist_prefill_destroy")


class sd_config(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_queries", ctypes.c_int32), ("kv_batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("n_ctx", ctypes.c_int64), ("chunk_size", ctypes.c_int32), ("seg_size", ctypes.c_int32),
        ("route", ctypes.c_int32), ("route_dim", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
        ("mode", ctypes.c_int32), ("top_k", ctypes.c_int32), ("top_k_seg", ctypes.c_int32),
        ("top_p", ctypes.c_double), ("select_scale", ctypes.c_double), ("tau", ctypes.c_double),
        ("softmax_scale", ctypes.c_float),
        ("keep_first", ctypes.c_int32), ("keep_last", ctypes.c_int32),
        ("sink", ctypes.c_int32), ("window", ctypes.c_int32),
        ("attend_summary", ctypes.c_int32), ("attend_blocks", ctypes.c_int32), ("head_masks", ctypes.c_int32),
        ("head_mode", ctypes.POINTER(ctypes.c_int8)),
    ]


class sd_tensors(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("q_sb", ctypes.c_int64), ("q_sh", ctypes.c_int64), ("q_st", ctypes.c_int64),
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("kv_sb", ctypes.c_int64), ("kv_sh", ctypes.c_int64), ("kv_st", ctypes.c_int64),
        ("kg", ctypes.c_void_p), ("vg", ctypes.c_void_p),
        ("g_sb", ctypes.c_int64), ("g_sh", ctypes.c_int64), ("g_st", ctypes.c_int64),
        ("kmg", ctypes.c_void_p), ("mg_sb", ctypes.c_int64), ("mg_sh", ctypes.c_int64), ("mg_st", ctypes.c_int64),
        ("kp", ctypes.c_void_p), ("kp_sb", ctypes.c_int64), ("kp_sh", ctypes.c_int64), ("kp_st", ctypes.c_int64),
        ("proj", ctypes.c_void_p), ("ctx_len", ctypes.c_void_p),
    ]


class sd_selection_view(ctypes.Structure):
    _fields_ = [
        ("scores0", ctypes.c_void_p), ("len0", ctypes.c_int64),
        ("scores1", ctypes.c_void_p), ("len1", ctypes.c_int64),
        ("cand1", ctypes.c_void_p),
        ("head_bits", ctypes.c_void_p), ("words", ctypes.c_int64),
        ("list", ctypes.c_void_p), ("n_entries", ctypes.c_int64),
        ("count", ctypes.c_void_p),
        ("status", ctypes.c_void_p),
    ]


class sp_config(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("seq_len", ctypes.c_int64), ("window", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32), ("tau", ctypes.c_double), ("softmax_scale", ctypes.c_double),
    ]


class sp_tensors(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("q_sb", ctypes.c_int64), ("q_sh", ctypes.c_int64), ("q_st", ctypes.c_int64),
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("kv_sb", ctypes.c_int64), ("kv_sh", ctypes.c_int64), ("kv_st", ctypes.c_int64),
        ("head_mode", ctypes.c_void_p),
    ]


class sp_view(ctypes.Structure):
    _fields_ = [
        ("importance", ctypes.c_void_p), ("budget", ctypes.c_void_p),
        ("head_bits", ctypes.c_void_p), ("words", ctypes.c_int64),
        ("list", ctypes.c_void_p), ("status", ctypes.c_void_p),
    ]


class gp_config(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("n_tokens", ctypes.c_int64), ("chunk_size", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_double),
    ]


class gp_tensors(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("q_sb", ctypes.c_int64), ("q_sh", ctypes.c_int64), ("q_st", ctypes.c_int64),
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("kv_sb", ctypes.c_int64), ("kv_sh", ctypes.c_int64), ("kv_st", ctypes.c_int64),
        ("qg", ctypes.c_void_p), ("qg_sb", ctypes.c_int64), ("qg_sh", ctypes.c_int64), ("qg_st", ctypes.c_int64),
        ("kg", ctypes.c_void_p), ("vg", ctypes.c_void_p),
        ("kvg_sb", ctypes.c_int64), ("kvg_sh", ctypes.c_int64), ("kvg_st", ctypes.c_int64),
    ]


class SparseDecodeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m query_adaptive_sparse_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int
        L.sparse_decode_init.argtypes = [ctypes.POINTER(sd_config), ctypes.POINTER(vp), ctypes.POINTER(ctypes.c_size_t)]
        L.sparse_decode_init.restype = st
        L.sparse_decode_num_levels.argtypes = [vp]
        L.sparse_decode_num_levels.restype = i32
        L.sparse_decode_attend_blocks.argtypes = [vp]
        L.sparse_decode_attend_blocks.restype = i32
        L.sparse_decode_score_chunks.argtypes = [vp, ctypes.POINTER(sd_tensors), ctypes.c_int, vp, vp]
        L.sparse_decode_score_chunks.restype = st
        L.sparse_decode_select.argtypes = [vp, ctypes.c_int, vp, vp]
        L.sparse_decode_select.restype = st
        L.sparse_decode_attend.argtypes = [vp, ctypes.POINTER(sd_tensors), vp, vp]
        L.sparse_decode_attend.restype = st
        L.sparse_decode_combine.argtypes = [vp, vp, vp, vp, vp]
        L.sparse_decode_combine.restype = st
        L.sparse_decode_step.argtypes = [vp, ctypes.POINTER(sd_tensors), vp, vp, vp, vp]
        L.sparse_decode_step.restype = st
        L.sparse_decode_step_static.argtypes = [vp, ctypes.POINTER(sd_tensors), vp, vp, vp]
        L.sparse_decode_step_static.restype = st
        L.sparse_decode_selection_view.argtypes = [vp, vp, ctypes.POINTER(sd_selection_view)]
        L.sparse_decode_selection_view.restype = st
        L.sparse_decode_last_error.argtypes = []
        L.sparse_decode_last_error.restype = ctypes.c_char_p
        L.sparse_decode_destroy.argtypes = [vp]
        L.sparse_decode_destroy.restype = None
        L.sparse_prefill_init.argtypes = [ctypes.POINTER(sp_config), ctypes.POINTER(vp), ctypes.POINTER(ctypes.c_size_t)]
        L.sparse_prefill_init.restype = st
        L.sparse_prefill_select.argtypes = [vp, ctypes.POINTER(sp_tensors), vp, vp]
        L.sparse_prefill_select.restype = st
        L.sparse_prefill_attend.argtypes = [vp, ctypes.POINTER(sp_tensors), vp, vp, vp]
        L.sparse_prefill_attend.restype = st
        L.sparse_prefill_view.argtypes = [vp, vp, ctypes.POINTER(sp_view)]
        L.sparse_prefill_view.restype = st
        L.sparse_prefill_destroy.argtypes = [vp]
        L.sparse_prefill_destroy.restype = None
        L.sparse_gist_prefill_init.argtypes = [ctypes.POINTER(gp_config), ctypes.POINTER(vp),
                                               ctypes.POINTER(ctypes.c_size_t)]
        L.sparse_gist_prefill_init.restype = st
        L.sparse_gist_prefill_attend.argtypes = [vp, ctypes.POINTER(gp_tensors), vp, vp, vp, vp]
        L.sparse_gist_prefill_attend.restype = st
        L.sparse_gist_prefill_destroy.argtypes = [vp]
        L.sparse_gist_prefill_destroy.restype = None
        _lib = L
    return _lib


def _check(status: int):
    if status != SD_OK:
        raise SparseDecodeError(status, lib().sparse_decode_last_error().decode())


def sparse_decode_init(cfg: sd_config):
    """Returns (handle, workspace_bytes)."""
    h = ctypes.c_void_p()
    n = ctypes.c_size_t()
    _check(lib().sparse_decode_init(ctypes.byref(cfg), ctypes.byref(h), ctypes.byref(n)))
    return h, n.value


def sparse_decode_num_levels(handle) -> int:
    return lib().sparse_decode_num_levels(handle)


def sparse_decode_attend_blocks(handle) -> int:
    return lib().sparse_decode_attend_blocks(handle)


def sparse_decode_score_chunks(handle, tensors: sd_tensors, level: int, ws: int, stream: int):
    _check(lib().sparse_decode_score_chunks(handle, ctypes.byref(tensors), level, ws, stream))


def sparse_decode_select(handle, level: int, ws: int, stream: int):
    _check(lib().sparse_decode_select(handle, level, ws, stream))


def sparse_decode_attend(handle, tensors: sd_tensors, ws: int, stream: int):
    _check(lib().sparse_decode_attend(handle, ctypes.byref(tensors), ws, stream))


def sparse_decode_combine(handle, ws: int, out: int, lse_out: int, stream: int):
    _check(lib().sparse_decode_combine(handle, ws, out, lse_out, stream))


def sparse_decode_step(handle, tensors: sd_tensors, ws: int, out: int, lse_out: int, stream: int):
    _check(lib().sparse_decode_step(handle, ctypes.byref(tensors), ws, out, lse_out, stream))


def sparse_decode_step_static(handle, tensors: sd_tensors, out: int, lse_out: int, stream: int):
    _check(lib().sparse_decode_step_static(handle, ctypes.byref(tensors), out, lse_out, stream))


def sparse_decode_selection_view(handle, ws: int) -> sd_selection_view:
    v = sd_selection_view()
    _check(lib().sparse_decode_selection_view(handle, ws, ctypes.byref(v)))
    return v


def sparse_decode_last_error() -> str:
    return lib().sparse_decode_last_error().decode()


def sparse_decode_destroy(handle):
    lib().sparse_decode_destroy(handle)


def sparse_prefill_init(cfg: sp_config):
    """Returns (handle, workspace_bytes)."""
    h = ctypes.c_void_p()
    n = ctypes.c_size_t()
    _check(lib().sparse_prefill_init(ctypes.byref(cfg), ctypes.byref(h), ctypes.byref(n)))
    return h, n.value


def sparse_prefill_select(handle, tensors: sp_tensors, ws: int, stream: int):
    _check(lib().sparse_prefill_select(handle, ctypes.byref(tensors), ws, stream))


def sparse_prefill_attend(handle, tensors: sp_tensors, ws: int, out: int, stream: int):
    _check(lib().sparse_prefill_attend(handle, ctypes.byref(tensors), ws, out, stream))


def sparse_prefill_view(handle, ws: int) -> sp_view:
    v = sp_view()
    _check(lib().sparse_prefill_view(handle, ws, ctypes.byref(v)))
    return v


def sparse_prefill_destroy(handle):
    lib().sparse_prefill_destroy(handle)


def sparse_gist_prefill_init(cfg: gp_config):
    """Returns (handle, workspace bytes)."""
    h = ctypes.c_void_p()
    n = ctypes.c_size_t(0)
    _check(lib().sparse_gist_prefill_init(ctypes.byref(cfg), ctypes.byref(h), ctypes.byref(n)))
    return h, n.value


def sparse_gist_prefill_attend(handle, tensors: gp_tensors, ws: int, out: int, out_gist: int, stream: int):
    _check(lib().sparse_gist_prefill_attend(handle, ctypes.byref(tensors), ws, out, out_gist, stream))


def sparse_gist_prefill_destroy(handle):
    lib().sparse_gist_prefill_destroy(handle)
