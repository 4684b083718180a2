"""Seeded synthetic inputs for the indexer -> top-k -> sparse-MLA path (host C library, ctypes).

This module draws inputs and compares results; it holds none of the method's arithmetic. The
CPU oracle's tests and the GPU path read the same bytes from it. The shapes are those of the
pages' problem statement (BF16 queries, 656-byte FP8 latent rows shared by 64 heads, top-k 2048;
"Serving GLM-5.3 ... PCP, DCP, Hybrid HiSparse", section "Why the numbers work").
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# SMLA_WORKLOAD_LIB names another build of the same sources (the sanitizer test uses it)
LIB_PATH = os.environ.get("SMLA_WORKLOAD_LIB") or os.path.join(_HERE, "libsmla_workload.so")

KV_BF16 = 0
KV_FP8_656 = 1

CONFIG_NAMES = {0: "tiny", 1: "decode", 2: "chunked", 3: "prefill32k", 4: "million"}


class Dims(ctypes.Structure):
    _fields_ = [
        ("config_id", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("n_q", ctypes.c_int32),
        ("kv_format", ctypes.c_int32),
        ("cached", ctypes.c_int64),
        ("H", ctypes.c_int32),
        ("D_qk", ctypes.c_int32),
        ("D_v", ctypes.c_int32),
        ("H_I", ctypes.c_int32),
        ("D_I", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("row_bytes", ctypes.c_int32),
        ("_pad", ctypes.c_int32),
        ("total_q", ctypes.c_int64),
        ("total_rows", ctypes.c_int64),
        ("max_kv", ctypes.c_int64),
        ("sm_scale", ctypes.c_double),
        ("seed", ctypes.c_uint64),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_ if name != "_pad"}


class TopkReport(ctypes.Structure):
    _fields_ = [("rows_checked", ctypes.c_int64), ("rows_bad", ctypes.c_int64),
                ("first_bad", ctypes.c_int64), ("bad_entries", ctypes.c_int64)]


class AttnReport(ctypes.Structure):
    _fields_ = [("max_abs", ctypes.c_double), ("rel_l2", ctypes.c_double),
                ("argmax", ctypes.c_int64), ("n_nonfinite", ctypes.c_int64)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        L.smla_workload_dims_get.argtypes = [ctypes.c_int32, ctypes.POINTER(Dims)]
        L.smla_workload_dims_finish.argtypes = [ctypes.POINTER(Dims)]
        L.smla_workload_gen.argtypes = [ctypes.POINTER(Dims), ctypes.c_uint64, ctypes.c_int32,
                                        P, P, P, P, P]
        L.smla_workload_latent_f64.argtypes = [ctypes.POINTER(Dims), ctypes.c_uint64,
                                               ctypes.c_int64, ctypes.c_int64, P]
        L.smla_workload_default_threads.restype = ctypes.c_int32
        L.smla_check_topk.argtypes = [P, P, P, P, ctypes.c_int64, ctypes.c_int32,
                                      ctypes.POINTER(TopkReport)]
        L.smla_check_attn.argtypes = [P, P, ctypes.c_int64, ctypes.c_double, ctypes.c_double,
                                      ctypes.POINTER(AttnReport)]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def config_dims(config_id: int) -> Dims:
    d = Dims()
    rc = lib().smla_workload_dims_get(config_id, ctypes.byref(d))
    if rc != 0:
        raise ValueError(f"unknown workload config {config_id}")
    return d


def custom_dims(*, batch, n_q, cached, H, D_qk, D_v, H_I, D_I, top_k, kv_format,
                seed=0x5EED1000) -> Dims:
    d = Dims()
    d.config_id = -1
    d.batch, d.n_q, d.cached = batch, n_q, cached
    d.H, d.D_qk, d.D_v, d.H_I, d.D_I, d.top_k = H, D_qk, D_v, H_I, D_I, top_k
    d.kv_format = kv_format
    d.seed = seed
    if lib().smla_workload_dims_finish(ctypes.byref(d)) != 0:
        raise ValueError("invalid custom workload dims")
    return d


def small_big_dims(*, batch=1, n_q, cached, top_k=2048, seed=0x5EED1000) -> Dims:
    """A workload with the big head/row shapes (64 heads, 576/512 dims, FP8 rows, 64x128 indexer)
    but short contexts, for parity at sizes the oracle finishes in seconds."""
    return custom_dims(batch=batch, n_q=n_q, cached=cached, H=64, D_qk=576, D_v=512, H_I=64,
                       D_I=128, top_k=top_k, kv_format=KV_FP8_656, seed=seed)


@dataclass
class Inputs:
    dims: Dims
    seed: int
    q: np.ndarray      # uint16 bf16 bits [total_q, H, D_qk]
    kv: np.ndarray     # uint8 [total_rows, row_bytes]
    q_idx: np.ndarray  # int8 [total_q, H_I, D_I]
    k_idx: np.ndarray  # int8 [total_rows, D_I]
    w: np.ndarray      # int32 [H_I]
    n_q: np.ndarray    # int32 [batch] per-request query tokens
    kv_len: np.ndarray  # int64 [batch] per-request rows (cached + n_q)


def generate(d: Dims, seed: int | None = None, nthreads: int = 0, *, parts=("q", "kv", "q_idx",
             "k_idx", "w")) -> Inputs:
    seed = int(d.seed if seed is None else seed)
    q = np.empty((d.total_q, d.H, d.D_qk), np.uint16) if "q" in parts else None
    kv = np.empty((d.total_rows, d.row_bytes), np.uint8) if "kv" in parts else None
    q_idx = np.empty((d.total_q, d.H_I, d.D_I), np.int8) if "q_idx" in parts else None
    k_idx = np.empty((d.total_rows, d.D_I), np.int8) if "k_idx" in parts else None
    w = np.empty((d.H_I,), np.int32) if "w" in parts else None
    rc = lib().smla_workload_gen(ctypes.byref(d), seed, nthreads, _ptr(q), _ptr(kv), _ptr(q_idx),
                                 _ptr(k_idx), _ptr(w))
    if rc != 0:
        raise RuntimeError(f"smla_workload_gen failed ({rc})")
    n_q = np.full((d.batch,), d.n_q, np.int32)
    kv_len = np.full((d.batch,), d.max_kv, np.int64)
    return Inputs(d, seed, q, kv, q_idx, k_idx, w, n_q, kv_len)


@dataclass
class Fp8IndexerInputs:
    q: np.ndarray        # uint8 E4M3 codes [total_q, H_I, D_I]
    k: np.ndarray        # uint8 E4M3 codes [total_rows, D_I]
    k_scale: np.ndarray  # float32 [total_rows]
    w: np.ndarray        # float32 [total_q, H_I]


def _e4m3_codes(rng, shape, e_lo=5, e_hi=10):
    """Random E4M3 bit patterns from two random bytes per code: sign and the 3 mantissa bits from
    the first, the 4-bit exponent field (on [e_lo, e_hi], near uniform) from the second, whose top
    4 of 256 values make the code zero (1 in 64). Never a NaN code."""
    n = int(np.prod(shape))
    r = np.frombuffer(rng.bytes(2 * n), np.uint8).reshape(2, n)
    a, b = r[0], r[1]
    codes = (a & np.uint8(0x87)) | ((np.uint8(e_lo) + b % np.uint8(e_hi - e_lo + 1)) << np.uint8(3))
    codes[b >= 252] = 0
    return codes.reshape(shape)


def fp8_indexer_inputs(d: Dims, seed: int | None = None) -> Fp8IndexerInputs:
    """Inputs for the FP8-key indexer at the shapes of `d` (H_I x D_I per query token): E4M3 codes
    with exponent fields 5..10 (magnitudes 1/4 .. 7.5, one code in 64 zero), key scales uniform
    on [1/64, 1/8), per-token head weights uniform on [1/4, 1)."""
    seed = int(d.seed if seed is None else seed) ^ 0xF8F8F8F8
    rng = np.random.default_rng(seed)
    q = _e4m3_codes(rng, (d.total_q, d.H_I, d.D_I))
    k = _e4m3_codes(rng, (d.total_rows, d.D_I))
    k_scale = rng.uniform(1 / 64, 1 / 8, d.total_rows).astype(np.float32)
    w = rng.uniform(0.25, 1.0, (d.total_q, d.H_I)).astype(np.float32)
    return Fp8IndexerInputs(q, k, k_scale, w)


def latent_f64(d: Dims, seed: int, row0: int, nrows: int) -> np.ndarray:
    out = np.empty((nrows, d.D_qk), np.float64)
    rc = lib().smla_workload_latent_f64(ctypes.byref(d), seed, row0, nrows, _ptr(out))
    if rc != 0:
        raise ValueError("row range out of bounds")
    return out


def default_threads() -> int:
    return int(lib().smla_workload_default_threads())


def check_topk(got_idx, got_score, ref_idx, ref_score, top_k):
    got_idx = np.ascontiguousarray(got_idx, np.int32)
    ref_idx = np.ascontiguousarray(ref_idx, np.int32)
    gs = None if got_score is None else np.ascontiguousarray(got_score, np.int32)
    rs = None if ref_score is None else np.ascontiguousarray(ref_score, np.int32)
    rows = got_idx.size // top_k
    assert ref_idx.size == got_idx.size
    rep = TopkReport()
    rc = lib().smla_check_topk(_ptr(got_idx), _ptr(gs), _ptr(ref_idx), _ptr(rs), rows, top_k,
                               ctypes.byref(rep))
    return rc == 0, rep


def check_attn(got_bf16, ref, atol=2e-2, rel_l2=1e-2):
    got = np.ascontiguousarray(got_bf16).view(np.uint16).reshape(-1)
    ref = np.ascontiguousarray(ref, np.float64).reshape(-1)
    assert got.size == ref.size
    rep = AttnReport()
    rc = lib().smla_check_attn(_ptr(got), _ptr(ref), got.size, atol, rel_l2, ctypes.byref(rep))
    return rc == 0, rep
