"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path through the C ABI,
and compute the oracle's answers for chosen query tokens (inputs from the shared generator
only; expected values from the oracle only)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from sparse_mla_attention_indexer_amd import ops
from sparse_mla_attention_indexer_amd import workload as W

ATOL = 2e-2     # max |out - ref|
REL_L2 = 1e-2   # ||out - ref|| / ||ref||
LSE_ATOL = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class Dev:
    def __init__(self, x: W.Inputs, device="cuda:0", n_q=None, kv_len=None, positions=None):
        self.x = x
        d = x.dims
        self.device = torch.device(device)
        self.n_q = x.n_q if n_q is None else np.asarray(n_q, np.int32)
        self.kv_len = x.kv_len if kv_len is None else np.asarray(kv_len, np.int64)
        self.plan = ops.BatchPlan(self.n_q, self.kv_len, self.device, positions=positions)
        self.q = torch.from_numpy(x.q.view(np.int16)).view(torch.bfloat16).to(self.device)
        if d.kv_format == W.KV_FP8_656:
            self.kv = torch.from_numpy(x.kv).to(self.device)
        else:
            self.kv = torch.from_numpy(x.kv.view(np.int16).reshape(d.total_rows, d.D_qk)).view(
                torch.bfloat16).to(self.device)
        self.q_idx = torch.from_numpy(x.q_idx).to(self.device)
        self.k_idx = torch.from_numpy(x.k_idx).to(self.device)
        self.w = torch.from_numpy(x.w).to(self.device)

    def topk(self, top_k=None, with_scores=True):
        top_k = self.x.dims.top_k if top_k is None else top_k
        # one workspace per top_k, reused across calls: each call must leave it ready for the next
        ws = self._ws.get(top_k) if hasattr(self, "_ws") else None
        if ws is None:
            d = self.x.dims
            ws = ops.topk_workspace(self.plan, d.H_I, d.D_I, top_k)
            self._ws = getattr(self, "_ws", {})
            self._ws[top_k] = ws
        idx, sc = ops.indexer_topk(self.plan, self.q_idx, self.k_idx, self.w, top_k, with_scores,
                                   workspace=ws)
        torch.cuda.synchronize()
        return idx.cpu().numpy(), (sc.cpu().numpy() if sc is not None else None)

    def scores(self):
        s = ops.indexer_scores(self.plan, self.q_idx, self.k_idx, self.w)
        torch.cuda.synchronize()
        return s.cpu().numpy()

    def mla(self, idx_np, decode=False):
        d = self.x.dims
        idx = torch.from_numpy(np.ascontiguousarray(idx_np, np.int32)).to(self.device)
        out, lse = ops.sparse_mla(self.plan, self.q, self.kv, d.kv_format, d.D_v, idx, d.sm_scale,
                                  decode=decode)
        torch.cuda.synchronize()
        return out.view(torch.int16).cpu().numpy().view(np.uint16), lse.cpu().numpy()


def oracle_topk(x: W.Inputs, tokens, top_k=None, n_q=None, kv_len=None):
    top_k = x.dims.top_k if top_k is None else top_k
    n_q = x.n_q if n_q is None else n_q
    kv_len = x.kv_len if kv_len is None else kv_len
    return oracle.indexer_topk_batch(n_q, kv_len, x.q_idx, x.k_idx, x.w, top_k, tokens)


def sort_by_index(idx, sc):
    """Order each row by index ascending with -1 padding last (the library's output order)."""
    key = np.where(idx < 0, np.iinfo(np.int64).max, idx.astype(np.int64))
    o = np.argsort(key, axis=1, kind="stable")
    return np.take_along_axis(idx, o, 1), np.take_along_axis(sc, o, 1)


def oracle_mla(x: W.Inputs, idx_rows, tokens, n_q=None, kv_len=None):
    """Oracle attention for `tokens` whose selected rows are idx_rows [len(tokens), top_k]."""
    d = x.dims
    n_q = x.n_q if n_q is None else n_q
    kv_len = x.kv_len if kv_len is None else kv_len
    total_q = int(np.sum(n_q))
    full = np.full((total_q, idx_rows.shape[1]), -1, np.int32)
    full[np.asarray(tokens)] = idx_rows
    return oracle.sparse_mla_batch(n_q, kv_len, x.q, x.kv, d.kv_format, d.D_v, full, d.sm_scale,
                                   tokens)


def assert_topk_equal(got_idx, got_sc, ref_idx, ref_sc, label=""):
    ri, rs = sort_by_index(ref_idx, ref_sc)
    bad = np.nonzero((got_idx != ri).any(1) | ((got_sc != rs) & (ri >= 0)).any(1))[0]
    assert bad.size == 0, (f"{label}: {bad.size} rows differ, first row {bad[0]}: got "
                           f"{got_idx[bad[0]][:8]}.. ref {ri[bad[0]][:8]}..")


def assert_attn_close(got_bf16, ref, got_lse=None, ref_lse=None, label=""):
    ok, rep = W.check_attn(got_bf16, ref, ATOL, REL_L2)
    say(f"  {label}: max_abs={rep.max_abs:.3e} rel_l2={rep.rel_l2:.3e} nonfinite={rep.n_nonfinite}")
    assert ok, f"{label}: max_abs {rep.max_abs:.3e} rel_l2 {rep.rel_l2:.3e} at {rep.argmax}"
    if got_lse is not None:
        err = np.abs(got_lse - ref_lse)
        err = np.where(np.isinf(ref_lse) & (got_lse == ref_lse), 0.0, err)
        assert err.max() <= LSE_ATOL, f"{label}: lse error {err.max():.3e}"
