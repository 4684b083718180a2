"""Torch-facing wrappers over the C ABI (argument marshalling and host-side shape checks only).

torch provides device memory and the current HIP stream; every step of the path runs in the
library's gfx950 kernels. Shapes are checked here against the batch plan before any launch, so a
kernel never sees buffers smaller than its grid assumes.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from ._lib import KV_BF16, KV_FP8_656, Batch, check, lib

__all__ = ["BatchPlan", "indexer_scores", "indexer_topk", "sparse_mla", "KV_BF16", "KV_FP8_656"]


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _req(t: torch.Tensor, name: str, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


class BatchPlan:
    """Device batch table for requests with `n_q[b]` query tokens and `kv_len[b]` cached rows
    (queries are the last n_q rows of their request, unless `positions` [total_q] gives every
    token's position). Built once, reused by every call."""

    def __init__(self, n_q, kv_len, device="cuda:0", positions=None):
        self.device = torch.device(device)
        self.n_q = np.ascontiguousarray(n_q, np.int32).reshape(-1)
        self.kv_len = np.ascontiguousarray(kv_len, np.int64).reshape(-1)
        if self.n_q.size != self.kv_len.size or self.n_q.size < 1:
            raise ValueError("n_q and kv_len must be non-empty and of equal length")
        B = int(self.n_q.size)
        total_q = int(self.n_q.sum())
        max_kv = int(self.kv_len.max())
        pos = None
        if positions is not None:
            pos = np.ascontiguousarray(positions, np.int64).reshape(-1)
            if pos.size != total_q:
                raise ValueError("positions must hold one entry per query token")
        nbytes = int(lib().smla_batch_table_bytes(B, total_q, max_kv))
        if nbytes == 0:
            raise ValueError("invalid batch sizes")
        self.table = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.desc = Batch()
        with torch.cuda.device(self.device):
            check("smla_batch_build_pos",
                  lib().smla_batch_build_pos(B, self.n_q.ctypes.data, self.kv_len.ctypes.data,
                                             None if pos is None else pos.ctypes.data, None,
                                             self.table.data_ptr(), nbytes, _stream(self.device),
                                             ctypes.byref(self.desc)))
        self.batch = B
        self.total_q = total_q
        self.total_rows = int(self.kv_len.sum())
        self.max_kv = max_kv
        self.positions = pos if pos is not None else np.concatenate(
            [np.arange(k - n, k) for n, k in zip(self.n_q, self.kv_len)]).astype(np.int64)

    @property
    def ref(self):
        return ctypes.byref(self.desc)


def _check_indexer(plan: BatchPlan, q_idx, k_idx, w):
    d = plan.device
    if q_idx.dim() != 3:
        raise ValueError("q_idx must be [total_q, H_I, D_I]")
    H_I, D_I = int(q_idx.shape[1]), int(q_idx.shape[2])
    _req(q_idx, "q_idx", torch.int8, (plan.total_q, H_I, D_I), d)
    if k_idx.dim() != 2 or k_idx.shape[0] < plan.total_rows:
        raise ValueError(f"k_idx must be [>= {plan.total_rows}, D_I]")
    _req(k_idx, "k_idx", torch.int8, (k_idx.shape[0], D_I), d)
    _req(w, "w", torch.int32, (H_I,), d)
    return H_I, D_I


def indexer_scores(plan: BatchPlan, q_idx, k_idx, w, out=None):
    """Full score matrix [total_q, max_kv] int32 (-1 where s > p)."""
    H_I, D_I = _check_indexer(plan, q_idx, k_idx, w)
    if out is None:
        out = torch.empty((plan.total_q, plan.max_kv), dtype=torch.int32, device=plan.device)
    _req(out, "out", torch.int32, (plan.total_q, plan.max_kv), plan.device)
    with torch.cuda.device(plan.device):
        check("smla_indexer_scores",
              lib().smla_indexer_scores(plan.ref, q_idx.data_ptr(), k_idx.data_ptr(), w.data_ptr(),
                                        H_I, D_I, out.data_ptr(), _stream(plan.device)))
    return out


def topk_workspace(plan: BatchPlan, H_I: int, D_I: int, top_k: int) -> torch.Tensor:
    # zero-filled once: the library returns its histogram and counters to zero after each call
    n = int(lib().smla_indexer_topk_workspace_bytes(plan.ref, H_I, D_I, top_k))
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=plan.device)


def indexer_topk(plan: BatchPlan, q_idx, k_idx, w, top_k: int, with_scores=True, idx=None,
                 score=None, workspace=None):
    """Exact top-k per query token: idx [total_q, top_k] ascending, -1 padded; optional scores."""
    H_I, D_I = _check_indexer(plan, q_idx, k_idx, w)
    shape = (plan.total_q, top_k)
    if idx is None:
        idx = torch.empty(shape, dtype=torch.int32, device=plan.device)
    _req(idx, "idx", torch.int32, shape, plan.device)
    if with_scores and score is None:
        score = torch.empty(shape, dtype=torch.int32, device=plan.device)
    if score is not None:
        _req(score, "score", torch.int32, shape, plan.device)
    if workspace is None:
        workspace = topk_workspace(plan, H_I, D_I, top_k)
    with torch.cuda.device(plan.device):
        check("smla_indexer_scores_topk",
              lib().smla_indexer_scores_topk(plan.ref, q_idx.data_ptr(), k_idx.data_ptr(),
                                             w.data_ptr(), H_I, D_I, top_k, idx.data_ptr(),
                                             score.data_ptr() if score is not None else None,
                                             workspace.data_ptr(), workspace.numel(),
                                             _stream(plan.device)))
    return idx, score


def _check_indexer_fp8(plan: BatchPlan, q, k, k_scale, w):
    d = plan.device
    if q.dim() != 3:
        raise ValueError("q must be [total_q, H_I, D_I] E4M3 codes (uint8)")
    H_I, D_I = int(q.shape[1]), int(q.shape[2])
    _req(q, "q", torch.uint8, (plan.total_q, H_I, D_I), d)
    if k.dim() != 2 or k.shape[0] < plan.total_rows:
        raise ValueError(f"k must be [>= {plan.total_rows}, D_I] E4M3 codes (uint8)")
    _req(k, "k", torch.uint8, (k.shape[0], D_I), d)
    _req(k_scale, "k_scale", torch.float32, (k.shape[0],), d)
    _req(w, "w", torch.float32, (plan.total_q, H_I), d)
    return H_I, D_I


def indexer_scores_fp8(plan: BatchPlan, q, k, k_scale, w, out=None):
    """FP8 keys: full score matrix [total_q, max_kv] fp32 (-1.0 where s > p)."""
    H_I, D_I = _check_indexer_fp8(plan, q, k, k_scale, w)
    if out is None:
        out = torch.empty((plan.total_q, plan.max_kv), dtype=torch.float32, device=plan.device)
    _req(out, "out", torch.float32, (plan.total_q, plan.max_kv), plan.device)
    with torch.cuda.device(plan.device):
        check("smla_indexer_scores_fp8",
              lib().smla_indexer_scores_fp8(plan.ref, q.data_ptr(), k.data_ptr(), k_scale.data_ptr(),
                                            w.data_ptr(), H_I, D_I, out.data_ptr(),
                                            _stream(plan.device)))
    return out


def indexer_topk_fp8(plan: BatchPlan, q, k, k_scale, w, top_k: int, with_scores=True, idx=None,
                     score=None, workspace=None):
    """FP8 keys: exact top-k per query token of the fp32 scores; idx [total_q, top_k] ascending,
    -1 padded; optional scores fp32 (-1.0 on padding)."""
    H_I, D_I = _check_indexer_fp8(plan, q, k, k_scale, w)
    shape = (plan.total_q, top_k)
    if idx is None:
        idx = torch.empty(shape, dtype=torch.int32, device=plan.device)
    _req(idx, "idx", torch.int32, shape, plan.device)
    if with_scores and score is None:
        score = torch.empty(shape, dtype=torch.float32, device=plan.device)
    if score is not None:
        _req(score, "score", torch.float32, shape, plan.device)
    if workspace is None:
        workspace = topk_workspace(plan, H_I, D_I, top_k)
    with torch.cuda.device(plan.device):
        check("smla_indexer_scores_topk_fp8",
              lib().smla_indexer_scores_topk_fp8(plan.ref, q.data_ptr(), k.data_ptr(),
                                                 k_scale.data_ptr(), w.data_ptr(), H_I, D_I, top_k,
                                                 idx.data_ptr(),
                                                 score.data_ptr() if score is not None else None,
                                                 workspace.data_ptr(), workspace.numel(),
                                                 _stream(plan.device)))
    return idx, score


def topk_merge(idx_lists, score_lists, top_k: int, idx=None, score=None, float_scores=False,
               local=None):
    """DCP top-k merge: idx_lists / score_lists [n_lists, total_q, k_in] int32 (shard l holds the
    tokens l, l + n_lists, ...; local indices, -1 padding; scores as int32, or fp32 bit patterns
    with float_scores) -> the exact global top_k per token, idx [total_q, top_k] ascending (-1
    padded) and its scores (int32 bit patterns). local [n_lists, total_q, top_k] (optional): also
    every shard's part of the selection, as dcp_local_indices gives it."""
    if idx_lists.dim() != 3 or score_lists.shape != idx_lists.shape:
        raise ValueError("idx_lists and score_lists must both be [n_lists, total_q, k_in]")
    n_lists, total_q, k_in = (int(v) for v in idx_lists.shape)
    d = idx_lists.device
    _req(idx_lists, "idx_lists", torch.int32, (n_lists, total_q, k_in), d)
    _req(score_lists, "score_lists", torch.int32, (n_lists, total_q, k_in), d)
    if idx is None:
        idx = torch.empty((total_q, top_k), dtype=torch.int32, device=d)
    if score is None:
        score = torch.empty((total_q, top_k), dtype=torch.int32, device=d)
    _req(idx, "idx", torch.int32, (total_q, top_k), d)
    _req(score, "score", torch.int32, (total_q, top_k), d)
    if local is not None:
        _req(local, "local", torch.int32, (n_lists, total_q, top_k), d)
    with torch.cuda.device(d):
        check("smla_topk_merge",
              lib().smla_topk_merge(total_q, n_lists, k_in, idx_lists.data_ptr(), score_lists.data_ptr(),
                                    total_q * k_in, int(bool(float_scores)), top_k, idx.data_ptr(),
                                    score.data_ptr(), None if local is None else local.data_ptr(),
                                    _stream(d)))
    return idx, score


def dcp_shard_positions(n_q, kv_len, n_shards: int, shard: int):
    """Round-robin KV sharding ("Serving GLM-5.3 ... PCP, DCP, Hybrid HiSparse", section "DCP"):
    shard `shard` of n_shards holds rows shard, shard + n, ... of every request. Returns its rows
    per request and its query tokens' local positions, for
    BatchPlan(n_q, rows, positions=local): the token at global position P = kv_len - n_q + j sees
    the local rows j' with j' n + shard <= P, so its local position is floor((P - shard) / n)."""
    n_q = np.ascontiguousarray(n_q, np.int64).reshape(-1)
    kv_len = np.ascontiguousarray(kv_len, np.int64).reshape(-1)
    if n_shards < 1 or not 0 <= shard < n_shards:
        raise ValueError("need 0 <= shard < n_shards")
    rows = (kv_len - shard + n_shards - 1) // n_shards
    P = np.concatenate([np.arange(k - n, k) for n, k in zip(n_q, kv_len)])
    if (P < shard).any():
        raise ValueError("a query token sees no row of this shard (position below the shard id)")
    return rows, (P - shard) // n_shards


def dcp_local_indices(idx, n_shards: int, out=None):
    """Every shard's part of a global selection idx [total_q, top_k] (global indices): out
    [n_shards, total_q, top_k], for shard s the entries g with g % n_shards == s as
    g // n_shards, in order, then -1."""
    if idx.dim() != 2:
        raise ValueError("idx must be [total_q, top_k]")
    total_q, top_k = (int(v) for v in idx.shape)
    _req(idx, "idx", torch.int32, (total_q, top_k), idx.device)
    if out is None:
        out = torch.empty((n_shards, total_q, top_k), dtype=torch.int32, device=idx.device)
    _req(out, "out", torch.int32, (n_shards, total_q, top_k), idx.device)
    with torch.cuda.device(idx.device):
        check("smla_dcp_local_indices",
              lib().smla_dcp_local_indices(total_q, top_k, idx.data_ptr(), n_shards, out.data_ptr(),
                                           _stream(idx.device)))
    return out


def lse_merge(outs, lses, out=None, lse=None):
    """Partial attention results over disjoint row sets merged by log-sum-exp: outs
    [n_parts, total_q, H, D_v] bf16, lses [n_parts, total_q, H] fp32 -> out [total_q, H, D_v]
    bf16, lse [total_q, H] fp32."""
    if outs.dim() != 4:
        raise ValueError("outs must be [n_parts, total_q, H, D_v]")
    n, total_q, H, D_v = (int(v) for v in outs.shape)
    d = outs.device
    _req(outs, "outs", torch.bfloat16, (n, total_q, H, D_v), d)
    _req(lses, "lses", torch.float32, (n, total_q, H), d)
    if out is None:
        out = torch.empty((total_q, H, D_v), dtype=torch.bfloat16, device=d)
    if lse is None:
        lse = torch.empty((total_q, H), dtype=torch.float32, device=d)
    _req(out, "out", torch.bfloat16, (total_q, H, D_v), d)
    _req(lse, "lse", torch.float32, (total_q, H), d)
    with torch.cuda.device(d):
        check("smla_lse_merge",
              lib().smla_lse_merge(total_q, H, D_v, n, outs.data_ptr(), lses.data_ptr(),
                                   out.data_ptr(), lse.data_ptr(), _stream(d)))
    return out, lse


def hot_resolve(plan: BatchPlan, idx, resident_from, hot_base, hot_tok, hot_age, step: int,
                host_rows, host_row0, kv, idx_out=None, n_copied=None):
    """Resolve a step's selections idx [total_q, top_k] against each request's hot buffer:
    offloaded rows (local row < resident_from[b]) are served from hot slots (hot_tok / hot_age
    [batch, n_slots] int32, updated in place), misses copied from host_rows (a pinned CPU tensor
    [n, row_bytes] uint8, request b's local row u at host row host_row0[b] + u) into kv rows
    R_b + hot_base[b] + slot. Returns (idx_out [total_q, top_k], n_copied [batch]); a negative
    n_copied[b] means request b was rejected (see the C header)."""
    d = plan.device
    if idx.dim() != 2:
        raise ValueError("idx must be [total_q, top_k]")
    top_k = int(idx.shape[1])
    _req(idx, "idx", torch.int32, (plan.total_q, top_k), d)
    for name, t in (("resident_from", resident_from), ("hot_base", hot_base)):
        _req(t, name, torch.int32, (plan.batch,), d)
    _req(host_row0, "host_row0", torch.int64, (plan.batch,), d)
    if hot_tok.dim() != 2:
        raise ValueError("hot_tok must be [batch, n_slots]")
    n_slots = int(hot_tok.shape[1])
    _req(hot_tok, "hot_tok", torch.int32, (plan.batch, n_slots), d)
    _req(hot_age, "hot_age", torch.int32, (plan.batch, n_slots), d)
    if host_rows.device.type != "cpu" or not host_rows.is_pinned() or host_rows.dim() != 2:
        raise ValueError("host_rows must be a pinned 2-D CPU tensor")
    if host_rows.dtype != torch.uint8 or not host_rows.is_contiguous():
        raise ValueError("host_rows must be contiguous uint8")
    row_bytes = int(host_rows.shape[1])
    if kv.dim() != 2 or kv.device != d or not kv.is_contiguous() or kv.shape[0] < plan.total_rows:
        raise ValueError(f"kv must be a contiguous [>= {plan.total_rows}, row] tensor on {d}")
    if int(kv.shape[1]) * kv.element_size() != row_bytes:
        raise ValueError("kv rows and host rows differ in size")
    if idx_out is None:
        idx_out = torch.empty_like(idx)
    if n_copied is None:
        n_copied = torch.empty(plan.batch, dtype=torch.int32, device=d)
    _req(idx_out, "idx_out", torch.int32, (plan.total_q, top_k), d)
    _req(n_copied, "n_copied", torch.int32, (plan.batch,), d)
    with torch.cuda.device(d):
        check("smla_hot_resolve",
              lib().smla_hot_resolve(plan.ref, idx.data_ptr(), top_k, resident_from.data_ptr(),
                                     hot_base.data_ptr(), n_slots, hot_tok.data_ptr(),
                                     hot_age.data_ptr(), int(step), host_rows.data_ptr(),
                                     int(host_rows.shape[0]), host_row0.data_ptr(), row_bytes,
                                     kv.data_ptr(), idx_out.data_ptr(), n_copied.data_ptr(),
                                     _stream(d)))
    return idx_out, n_copied


def mla_workspace(plan: BatchPlan, H: int, D_v: int, top_k: int, decode: bool) -> torch.Tensor:
    n = int(lib().smla_sparse_mla_workspace_bytes(plan.ref, H, D_v, top_k, int(decode)))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=plan.device)


def sparse_mla(plan: BatchPlan, q, kv, kv_format: int, D_v: int, idx, sm_scale: float,
               decode=False, with_lse=True, out=None, lse=None, workspace=None, noalloc=False):
    """Sparse MLA over the selected rows: out [total_q, H, D_v] bf16 (+ lse [total_q, H] fp32).

    noalloc (decode only): smla_sparse_mla_decode_noalloc, whose split partials live in the
    library's built-in scratch; the caller passes out (and lse) to allocate nothing at all.

    q is [total_q, H, D_qk] bf16; kv is [>= total_rows, row_bytes] uint8 (656-byte FP8 rows) or
    [>= total_rows, D_qk] bf16; idx is [total_q, top_k] int32."""
    d = plan.device
    if q.dim() != 3:
        raise ValueError("q must be [total_q, H, D_qk]")
    H, D_qk = int(q.shape[1]), int(q.shape[2])
    _req(q, "q", torch.bfloat16, (plan.total_q, H, D_qk), d)
    if kv_format == KV_FP8_656:
        if kv.dim() != 2 or kv.shape[0] < plan.total_rows:
            raise ValueError(f"kv must be [>= {plan.total_rows}, 656] uint8")
        _req(kv, "kv", torch.uint8, (kv.shape[0], 656), d)
    elif kv_format == KV_BF16:
        if kv.dim() != 2 or kv.shape[0] < plan.total_rows:
            raise ValueError(f"kv must be [>= {plan.total_rows}, {D_qk}] bf16")
        _req(kv, "kv", torch.bfloat16, (kv.shape[0], D_qk), d)
    else:
        raise ValueError(f"unknown kv_format {kv_format}")
    if idx.dim() != 2:
        raise ValueError("idx must be [total_q, top_k]")
    top_k = int(idx.shape[1])
    _req(idx, "idx", torch.int32, (plan.total_q, top_k), d)
    if out is None:
        out = torch.empty((plan.total_q, H, D_v), dtype=torch.bfloat16, device=d)
    _req(out, "out", torch.bfloat16, (plan.total_q, H, D_v), d)
    if with_lse and lse is None:
        lse = torch.empty((plan.total_q, H), dtype=torch.float32, device=d)
    if lse is not None:
        _req(lse, "lse", torch.float32, (plan.total_q, H), d)
    if noalloc:
        if not decode:
            raise ValueError("noalloc is the decode entry point")
        with torch.cuda.device(d):
            check("smla_sparse_mla_decode_noalloc",
                  lib().smla_sparse_mla_decode_noalloc(
                      plan.ref, q.data_ptr(), kv.data_ptr(), kv_format, H, D_qk, D_v, idx.data_ptr(),
                      top_k, float(sm_scale), out.data_ptr(),
                      lse.data_ptr() if lse is not None else None, _stream(d)))
        return out, lse
    if workspace is None:
        workspace = mla_workspace(plan, H, D_v, top_k, decode)
    fn = "smla_sparse_mla_decode" if decode else "smla_sparse_mla_prefill"
    with torch.cuda.device(d):
        check(fn, getattr(lib(), fn)(plan.ref, q.data_ptr(), kv.data_ptr(), kv_format, H, D_qk, D_v,
                                     idx.data_ptr(), top_k, float(sm_scale), out.data_ptr(),
                                     lse.data_ptr() if lse is not None else None,
                                     workspace.data_ptr(), workspace.numel(), _stream(d)))
    return out, lse


def kv_append(latent, rows, kv, k_new=None, k_idx=None):
    """New tokens into the caches: latent [n, 576] bf16 -> FP8 rows kv[rows] ([R, 656] uint8),
    and (optionally) indexer keys k_new [n, D_I] int8 -> k_idx[rows]. See smla_kv_append."""
    d = kv.device
    n = latent.shape[0] if latent.dim() == 2 else -1
    _req(latent, "latent", torch.bfloat16, (n, 576), d)
    _req(rows, "rows", torch.int64, (n,), d)
    if kv.dtype != torch.uint8 or kv.dim() != 2 or kv.shape[1] != 656 or not kv.is_contiguous():
        raise ValueError("kv must be a contiguous uint8 [R, 656] tensor")
    D_I = 0
    if k_new is not None:
        if k_idx is None:
            raise ValueError("k_idx is required with k_new")
        D_I = k_new.shape[1] if k_new.dim() == 2 else -1
        _req(k_new, "k_new", torch.int8, (n, D_I), d)
        if k_idx.dtype != torch.int8 or k_idx.dim() != 2 or k_idx.shape[1] != D_I or not k_idx.is_contiguous():
            raise ValueError("k_idx must be a contiguous int8 [R, D_I] tensor")
    check("smla_kv_append",
          lib().smla_kv_append(n, latent.data_ptr(), k_new.data_ptr() if k_new is not None else None,
                               D_I, rows.data_ptr(), kv.data_ptr(),
                               k_idx.data_ptr() if k_idx is not None else None, _stream(d)))
