"""CPU oracle for the indexer -> top-k -> sparse-MLA path (ctypes over plain C).

TEST INFRASTRUCTURE ONLY: tests, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg
may use it; the product library never does. It shares no code with the GPU path. The definitions
it implements, and the passages they follow, are stated in ``smla_oracle.h``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# SMLA_ORACLE_LIB names another build of the same sources (the sanitizer test uses it)
LIB_PATH = os.environ.get("SMLA_ORACLE_LIB") or os.path.join(_HERE, "libsmla_oracle.so")
SRC = os.path.join(_HERE, "smla_oracle.c")


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc into ``oracle/libsmla_oracle.so``."""
    cmd = ["gcc", "-O3", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared", "-pthread",
           "-Wall", "-Wextra", "-o", LIB_PATH + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    global _lib
    _lib = None
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run oracle.build()")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        L.smla_oracle_e4m3.argtypes = [ctypes.c_uint8]
        L.smla_oracle_e4m3.restype = ctypes.c_double
        L.smla_oracle_bf16.argtypes = [ctypes.c_uint16]
        L.smla_oracle_bf16.restype = ctypes.c_double
        L.smla_oracle_dequant_row.argtypes = [P, i32, i32, P]
        L.smla_oracle_e4m3_encode.argtypes = [ctypes.c_double]
        L.smla_oracle_e4m3_encode.restype = ctypes.c_uint8
        L.smla_oracle_fp8_row_encode.argtypes = [P, P]
        L.smla_oracle_indexer_scores.argtypes = [P, P, P, i32, i32, i64, P]
        L.smla_oracle_indexer_scores_fp8.argtypes = [P, P, P, P, i32, i32, i64, P, P]
        L.smla_oracle_topk.argtypes = [P, i64, i32, P, P]
        L.smla_oracle_topk_merge.argtypes = [P, P, i32, i32, i32, P, P]
        L.smla_oracle_lse_merge.argtypes = [i32, i32, i32, P, P, P, P]
        L.smla_oracle_hot_resolve.argtypes = [i32, i32, P, i64, i64, i32, P, P, i32, i64, P, P, P]
        L.smla_oracle_attend.argtypes = [P, P, i32, i32, i32, i32, i32, P, i32, ctypes.c_double,
                                         P, P]
        L.smla_oracle_indexer_topk_batch.argtypes = [i32, P, P, P, P, P, i32, i32, i32, P, i64, P,
                                                     P, i32]
        L.smla_oracle_sparse_mla_batch.argtypes = [i32, P, P, P, P, i32, i32, i32, i32, i32, P,
                                                   i32, ctypes.c_double, P, i64, P, P, i32]
        L.smla_oracle_default_threads.restype = i32
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def default_threads() -> int:
    return int(lib().smla_oracle_default_threads())


def e4m3(code: int) -> float:
    return lib().smla_oracle_e4m3(code)


def bf16(bits: int) -> float:
    return lib().smla_oracle_bf16(bits)


def e4m3_encode(v: float) -> int:
    """OCP E4M3 code of v, round to nearest-even, saturating at 448."""
    return int(lib().smla_oracle_e4m3_encode(float(v)))


def fp8_row_encode(latent: np.ndarray) -> np.ndarray:
    """One token's 576 bf16 bit patterns (uint16) -> its 656-byte FP8 row (uint8)."""
    lat = np.ascontiguousarray(latent, dtype=np.uint16)
    assert lat.shape == (576,)
    row = np.zeros(656, np.uint8)
    lib().smla_oracle_fp8_row_encode(_p(lat), _p(row))
    return row


def dequant_row(row: np.ndarray, fmt: int, D_qk: int) -> np.ndarray:
    row = _c(row, np.uint8)
    out = np.empty(D_qk, np.float64)
    if lib().smla_oracle_dequant_row(_p(row), fmt, D_qk, _p(out)) != 0:
        raise ValueError("dequant_row: bad format")
    return out


def indexer_scores(q_tok, keys, w) -> np.ndarray:
    """Scores of one query token q_tok [H_I, D_I] against keys [n, D_I] (int64)."""
    q_tok = _c(q_tok, np.int8)
    keys = _c(keys, np.int8)
    w = _c(w, np.int32)
    H_I, D_I = q_tok.shape
    n = keys.shape[0]
    out = np.empty(n, np.int64)
    rc = lib().smla_oracle_indexer_scores(_p(q_tok), _p(keys), _p(w), H_I, D_I, n, _p(out))
    if rc != 0:
        raise OverflowError("indexer score outside [0, 2^31)")
    return out


def indexer_scores_fp8(q_tok, keys, k_scale, w):
    """FP8-key scores of one query token: q_tok [H_I, D_I] and keys [n, D_I] E4M3 codes (uint8),
    k_scale [n] and w [H_I] float32. Returns (score, magnitude), both float64 [n]."""
    q_tok = _c(q_tok, np.uint8)
    keys = _c(keys, np.uint8)
    k_scale = _c(k_scale, np.float32)
    w = _c(w, np.float32)
    H_I, D_I = q_tok.shape
    n = keys.shape[0]
    assert keys.shape == (n, D_I) and k_scale.shape == (n,) and w.shape == (H_I,)
    out = np.empty(n, np.float64)
    mag = np.empty(n, np.float64)
    rc = lib().smla_oracle_indexer_scores_fp8(_p(q_tok), _p(keys), _p(k_scale), _p(w), H_I, D_I,
                                              n, _p(out), _p(mag))
    if rc != 0:
        raise ValueError("indexer_scores_fp8: NaN code, or a negative or non-finite weight or scale")
    return out, mag


def topk(scores, top_k: int):
    """Exact top-k of one score row by (score desc, index asc); -1 padding."""
    scores = _c(scores, np.int64)
    idx = np.empty(top_k, np.int32)
    sc = np.empty(top_k, np.int32)
    if lib().smla_oracle_topk(_p(scores), scores.size, top_k, _p(idx), _p(sc)) != 0:
        raise ValueError("topk failed")
    return idx, sc


def topk_merge(idx_lists, score_lists, top_k: int):
    """DCP top-k merge of one query token: per-shard lists [n_lists, k_in] (local indices, shard
    l holds tokens l, l + n_lists, ...) -> the top_k of their union by (score desc, global index
    asc), -1 padding."""
    idx_lists = _c(idx_lists, np.int32)
    score_lists = _c(score_lists, np.int32)
    n_lists, k_in = idx_lists.shape
    idx = np.empty(top_k, np.int32)
    sc = np.empty(top_k, np.int32)
    if lib().smla_oracle_topk_merge(_p(idx_lists), _p(score_lists), n_lists, k_in, top_k, _p(idx),
                                    _p(sc)) != 0:
        raise ValueError("topk_merge failed")
    return idx, sc


def lse_merge(outs, lses):
    """LSE merge of partial attention results over disjoint row sets: outs [n, H, D_v],
    lses [n, H] -> (out [H, D_v], lse [H])."""
    outs = _c(outs, np.float64)
    lses = _c(lses, np.float64)
    n, H, D_v = outs.shape
    out = np.empty((H, D_v), np.float64)
    lse = np.empty(H, np.float64)
    if lib().smla_oracle_lse_merge(n, H, D_v, _p(outs), _p(lses), _p(out), _p(lse)) != 0:
        raise ValueError("lse_merge failed")
    return out, lse


class HotResolveOverflow(ValueError):
    """The request's distinct offloaded selections outnumber the hot buffer's slots."""


class HotResolveBounds(ValueError):
    """resident_from / hot_base out of the request's bounds."""


def hot_resolve(idx, resident_from: int, hot_tok, hot_age, step: int, hot_base: int,
                kv_len: int = -1):
    """Hot-buffer resolve of one request: idx [n_q, top_k]; hot_tok / hot_age [H] int32 are
    updated in place. kv_len >= 0 also checks the request's bounds (HotResolveBounds).
    Returns (idx_out [n_q, top_k], copies [(token, slot), ...])."""
    idx = _c(idx, np.int32)
    assert hot_tok.dtype == np.int32 and hot_age.dtype == np.int32
    assert hot_tok.flags.c_contiguous and hot_age.flags.c_contiguous
    n_q, top_k = idx.shape
    H = hot_tok.size
    out = np.empty_like(idx)
    copies = np.empty((n_q * top_k + 1, 2), np.int32)
    nc = ctypes.c_int32(0)
    rc = lib().smla_oracle_hot_resolve(n_q, top_k, _p(idx), kv_len, resident_from, H, _p(hot_tok),
                                       _p(hot_age), step, hot_base, _p(out), _p(copies),
                                       ctypes.byref(nc))
    if rc == -2:
        raise HotResolveOverflow("hot_resolve: more distinct offloaded rows than slots")
    if rc == -3:
        raise HotResolveBounds("hot_resolve: resident_from / hot_base out of the request's bounds")
    if rc != 0:
        raise ValueError("hot_resolve failed")
    return out, [tuple(int(v) for v in copies[i]) for i in range(nc.value)]


def attend(q_tok, rows, fmt, D_v, idx, sm_scale):
    """One token: q_tok [H, D_qk] bf16 bits (uint16), rows [n, row_bytes] uint8, idx [k]."""
    q_tok = _c(q_tok, np.uint16)
    rows = _c(rows, np.uint8)
    idx = _c(idx, np.int32)
    H, D_qk = q_tok.shape
    out = np.empty((H, D_v), np.float64)
    lse = np.empty(H, np.float64)
    rc = lib().smla_oracle_attend(_p(q_tok), _p(rows), fmt, rows.shape[1], H, D_qk, D_v, _p(idx),
                                  idx.size, sm_scale, _p(out), _p(lse))
    if rc != 0:
        raise ValueError("attend failed (no valid row or bad format)")
    return out, lse


def indexer_topk_batch(n_q, kv_len, q_idx, k_idx, w, top_k, tokens, nthreads=0,
                       with_scores=True):
    n_q = _c(n_q, np.int32)
    kv_len = _c(kv_len, np.int64)
    q_idx = _c(q_idx, np.int8)
    k_idx = _c(k_idx, np.int8)
    w = _c(w, np.int32)
    tokens = _c(tokens, np.int64)
    H_I, D_I = q_idx.shape[-2], q_idx.shape[-1]
    idx = np.empty((tokens.size, top_k), np.int32)
    sc = np.empty((tokens.size, top_k), np.int32) if with_scores else None
    rc = lib().smla_oracle_indexer_topk_batch(n_q.size, _p(n_q), _p(kv_len), _p(q_idx), _p(k_idx),
                                              _p(w), H_I, D_I, top_k, _p(tokens), tokens.size,
                                              _p(idx), _p(sc), nthreads)
    if rc != 0:
        raise ValueError("indexer_topk_batch failed")
    return idx, sc


def sparse_mla_batch(n_q, kv_len, q, kv, fmt, D_v, idx, sm_scale, tokens, nthreads=0):
    n_q = _c(n_q, np.int32)
    kv_len = _c(kv_len, np.int64)
    q = _c(q, np.uint16)
    kv = _c(kv, np.uint8)
    idx = _c(idx, np.int32)
    tokens = _c(tokens, np.int64)
    H, D_qk = q.shape[-2], q.shape[-1]
    top_k = idx.shape[-1]
    out = np.empty((tokens.size, H, D_v), np.float64)
    lse = np.empty((tokens.size, H), np.float64)
    rc = lib().smla_oracle_sparse_mla_batch(n_q.size, _p(n_q), _p(kv_len), _p(q), _p(kv), fmt,
                                            kv.shape[-1], H, D_qk, D_v, _p(idx), top_k, sm_scale,
                                            _p(tokens), tokens.size, _p(out), _p(lse), nthreads)
    if rc != 0:
        raise ValueError("sparse_mla_batch failed")
    return out, lse
