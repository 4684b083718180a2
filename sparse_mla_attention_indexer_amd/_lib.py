"""ctypes loader for ``libsmla.so`` (the C ABI of ``include/smla.h``).

Argument marshalling only: every step of the path runs in the library's HIP kernels. There is
no fallback: if the library is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# SMLA_LIB names another build of the same sources (the sanitizer test uses it)
LIB_PATH = os.environ.get("SMLA_LIB") or os.path.join(_HERE, "libsmla.so")

SMLA_OK = 0
SMLA_E_INVALID = -1
SMLA_E_UNSUPPORTED = -2
SMLA_E_WORKSPACE = -3
SMLA_E_HIP = -4

KV_BF16 = 0
KV_FP8_656 = 1

# Every symbol include/smla.h declares.
EXPORTS = (
    "smla_batch_table_bytes",
    "smla_batch_build",
    "smla_batch_build_pos",
    "smla_indexer_scores",
    "smla_indexer_topk_workspace_bytes",
    "smla_indexer_scores_topk",
    "smla_indexer_scores_fp8",
    "smla_indexer_scores_topk_fp8",
    "smla_topk_merge",
    "smla_dcp_local_indices",
    "smla_lse_merge",
    "smla_hot_resolve",
    "smla_sparse_mla_workspace_bytes",
    "smla_sparse_mla_prefill",
    "smla_sparse_mla_decode",
    "smla_sparse_mla_decode_noalloc",
    "smla_kv_append",
    "smla_set_stage_events",
    "smla_status_str",
    "smla_last_error",
    "smla_version",
)


class Batch(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("total_q", ctypes.c_int32),
        ("max_q", ctypes.c_int32),
        ("n_items", ctypes.c_int32),
        ("max_kv", ctypes.c_int64),
        ("total_rows", ctypes.c_int64),
        ("total_cand", ctypes.c_int64),
        ("min_cand", ctypes.c_int64),
        ("table", ctypes.c_void_p),
        ("table_bytes", ctypes.c_size_t),
    ]


class SmlaError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: {status_str(status)} ({status}): {msg}")
        self.status = status


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built: run __graft_entry__.build() (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        BP = ctypes.POINTER(Batch)
        L.smla_batch_table_bytes.argtypes = [i32, i32, i64]
        L.smla_batch_table_bytes.restype = sz
        L.smla_batch_build.argtypes = [i32, P, P, P, sz, P, BP]
        L.smla_batch_build_pos.argtypes = [i32, P, P, P, P, P, sz, P, BP]
        L.smla_indexer_scores.argtypes = [BP, P, P, P, i32, i32, P, P]
        L.smla_indexer_topk_workspace_bytes.argtypes = [BP, i32, i32, i32]
        L.smla_indexer_topk_workspace_bytes.restype = sz
        L.smla_indexer_scores_topk.argtypes = [BP, P, P, P, i32, i32, i32, P, P, P, sz, P]
        L.smla_indexer_scores_fp8.argtypes = [BP, P, P, P, P, i32, i32, P, P]
        L.smla_indexer_scores_topk_fp8.argtypes = [BP, P, P, P, P, i32, i32, i32, P, P, P, sz, P]
        L.smla_topk_merge.argtypes = [i32, i32, i32, P, P, i64, i32, i32, P, P, P, P]
        L.smla_dcp_local_indices.argtypes = [i32, i32, P, i32, P, P]
        L.smla_lse_merge.argtypes = [i32, i32, i32, i32, P, P, P, P, P]
        L.smla_hot_resolve.argtypes = [BP, P, i32, P, P, i32, P, P, i32, P, i64, P, i32, P, P, P, P]
        L.smla_sparse_mla_workspace_bytes.argtypes = [BP, i32, i32, i32, i32]
        L.smla_sparse_mla_workspace_bytes.restype = sz
        for fn in ("smla_sparse_mla_prefill", "smla_sparse_mla_decode"):
            getattr(L, fn).argtypes = [BP, P, P, i32, i32, i32, i32, P, i32, ctypes.c_float, P, P,
                                       P, sz, P]
        L.smla_sparse_mla_decode_noalloc.argtypes = [BP, P, P, i32, i32, i32, i32, P, i32,
                                                      ctypes.c_float, P, P, P]
        L.smla_kv_append.argtypes = [i64, P, P, i32, P, P, P, P]
        L.smla_set_stage_events.argtypes = [P, P, i32]
        L.smla_status_str.argtypes = [ctypes.c_int]
        L.smla_status_str.restype = ctypes.c_char_p
        L.smla_last_error.restype = ctypes.c_char_p
        L.smla_version.restype = i32
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().smla_status_str(status).decode()


def last_error() -> str:
    return lib().smla_last_error().decode()


def check(fn: str, status: int):
    if status != SMLA_OK:
        raise SmlaError(fn, status, last_error())
