"""ctypes declarations of libpaged_decode.so (include/paged_decode.h).

Loading order matters: torch is imported first so that its HIP runtime is the
one the library binds to (both carry the soname libamdhip64.so.7).  There is
no fallback: if the library is missing this module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime the library will share)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpaged_decode.so")

PD_OK, PD_E_INVALID, PD_E_UNSUPPORTED, PD_E_CAPACITY, PD_E_HIP, PD_E_SCRATCH = range(6)
PD_BIND_FULL, PD_BIND_STEADY = 0, 1
PD_PLAN_WAVES, PD_PLAN_TEAM_MAX = 2048, 4  # the split plan's launch constants (header #defines)
PD_ERR_NEG_SEQ_LEN = 1 << 0
PD_ERR_SEQ_OVER_TABLE = 1 << 1
PD_ERR_TOTAL_OVER_CAP = 1 << 2
PD_ERR_BAD_PAGE = 1 << 3
PD_ERR_EXTEND_OVER_LEN = 1 << 4

EXPORTS = (
    "paged_decode_workspace_bytes",
    "paged_decode_init_workspace",
    "paged_decode_layout",
    "paged_decode_num_splits",
    "paged_decode_bind",
    "paged_decode_bind_contiguous",
    "paged_decode_attn",
    "paged_decode_append_kv",
    "paged_decode_append_attn",
    "paged_decode_merge",
    "paged_decode_attn_merge_noalloc",
    "paged_decode_bind_extend",
    "paged_decode_prefill_attn",
    "paged_decode_graph_pool_create",
    "paged_decode_graph_pool_warmup",
    "paged_decode_graph_pool_step",
    "paged_decode_graph_pool_num_keys",
    "paged_decode_graph_pool_key",
    "paged_decode_graph_pool_destroy",
    "paged_decode_read_error",
    "paged_decode_destroy",
    "paged_decode_strerror",
)


class PdConfig(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_batch", ctypes.c_int32),
        ("max_splits", ctypes.c_int32),
        ("max_pages_per_req", ctypes.c_int32),
        ("num_slots", ctypes.c_int64),
        ("max_total_tokens", ctypes.c_int64),
    ]


class PdLayout(ctypes.Structure):
    _fields_ = [(name, ctypes.c_size_t) for name in (
        "arena_bytes", "kv_indptr", "kv_indices", "page_indptr", "o_part", "ml_part", "qo_indptr", "item_indptr",
        "req_order", "meta", "error_word")]


class PdStepBuffers(ctypes.Structure):
    _fields_ = [
        ("seq_lens", ctypes.c_void_p),
        ("position_ids", ctypes.c_void_p),
        ("req_to_page", ctypes.c_void_p),
        ("req_base", ctypes.c_void_p),
        ("q", ctypes.c_void_p),
        ("k_store", ctypes.c_void_p),
        ("v_store", ctypes.c_void_p),
        ("k_new", ctypes.c_void_p),
        ("v_new", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("scale", ctypes.c_float),
    ]


PD_POOL_EAGER = 1


class PagedDecodeError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: status {status} ({msg})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (loads it on first use; raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m paged_kv_decode_10_amd.build` "
            "(hipcc, gfx950). There is no fallback implementation.")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    sig = {
        "paged_decode_workspace_bytes": [ctypes.POINTER(PdConfig), ctypes.POINTER(SZ)],
        "paged_decode_init_workspace": [ctypes.POINTER(PdConfig), P, SZ, ctypes.POINTER(P)],
        "paged_decode_layout": [P, ctypes.POINTER(PdLayout)],
        "paged_decode_num_splits": [P, I32, I32, ctypes.POINTER(I32)],
        "paged_decode_bind": [P, I32, I32, P, P, P, P],
        "paged_decode_bind_contiguous": [P, I32, I32, P, P, P, P],
        "paged_decode_attn": [P, I32, I32, I32, P, P, P, F, P],
        "paged_decode_append_kv": [P, I32, I32, P, P, P, P, P],
        "paged_decode_append_attn": [P, I32, I32, I32, P, P, P, P, P, F, P],
        "paged_decode_merge": [P, I32, I32, P, P],
        "paged_decode_attn_merge_noalloc": [P, I32, I32, I32, P, P, P, F, P, P],
        "paged_decode_bind_extend": [P, I32, P, P, P, P, P],
        "paged_decode_prefill_attn": [P, I32, I32, P, I32, P, P, F, P, P],
        "paged_decode_graph_pool_create": [P, ctypes.POINTER(PdStepBuffers), ctypes.c_uint32, ctypes.POINTER(P)],
        "paged_decode_graph_pool_warmup": [P],
        "paged_decode_graph_pool_step": [P, I32, P],
        "paged_decode_graph_pool_num_keys": [P, ctypes.POINTER(I32)],
        "paged_decode_graph_pool_key": [P, I32, ctypes.POINTER(I32), ctypes.POINTER(I32), ctypes.POINTER(I32)],
        "paged_decode_graph_pool_destroy": [P],
        "paged_decode_read_error": [P, ctypes.POINTER(ctypes.c_uint32), P],
        "paged_decode_destroy": [P],
    }
    for name, argtypes in sig.items():
        fn = getattr(L, name)
        fn.argtypes = argtypes
        fn.restype = ctypes.c_int
    L.paged_decode_strerror.argtypes = [ctypes.c_int]
    L.paged_decode_strerror.restype = ctypes.c_char_p
    _ = I64
    _lib = L
    return L


def check(fn: str, status: int) -> None:
    if status != PD_OK:
        raise PagedDecodeError(fn, status, lib().paged_decode_strerror(status).decode())
