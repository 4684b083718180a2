"""GPU parity for batches whose query tokens carry explicit positions (smla_batch_build_pos):
positions that repeat or jump, as a DCP shard's local positions do, on short rows (p + 1 below
k), rows of the register-resident top-k and rows past its 32,768-candidate limit.

Expected values come from the oracle one token at a time: a token at position p of request b
is the lone query of a request made of that request's rows 0..p, which is the batch layout the
oracle takes.
"""
import numpy as np
import pytest

import oracle
from sparse_mla_attention_indexer_amd import workload as W

pytestmark = pytest.mark.gpu

from gpu_harness import Dev, assert_attn_close, say  # noqa: E402

N_Q = np.array([6, 5], np.int32)
KV_LEN = np.array([3000, 40000], np.int64)
POS = np.array([100, 100, 1500, 1501, 1501, 2999, 20000, 33000, 33000, 33001, 39999], np.int64)


def _one_token(x, t, b, p):
    """(q_idx, k_idx, q, kv) of token t at position p of request b, as a request of its own."""
    r0 = int(np.concatenate([[0], np.cumsum(KV_LEN)])[b])
    return (x.q_idx[t:t + 1], x.k_idx[r0:r0 + p + 1], x.q[t], x.kv[r0:r0 + p + 1])


def test_explicit_positions_topk_and_attention():
    # one request of 11 tokens over 43,000 rows, re-cut into two requests with explicit positions
    x = W.generate(W.small_big_dims(batch=1, n_q=int(N_Q.sum()), cached=int(KV_LEN.sum() - N_Q.sum())))
    d = x.dims
    say(f"[case] explicit positions n_q={N_Q.tolist()} kv_len={KV_LEN.tolist()} pos={POS.tolist()}")
    dev = Dev(x, n_q=N_Q, kv_len=KV_LEN, positions=POS)
    idx, sc = dev.topk()
    req = np.repeat(np.arange(N_Q.size), N_Q)
    for t in range(int(N_Q.sum())):
        b, p = int(req[t]), int(POS[t])
        qi, ki, _, _ = _one_token(x, t, b, p)
        oi, os_ = oracle.indexer_topk_batch(np.ones(1, np.int32), np.array([p + 1], np.int64), qi, ki,
                                            x.w, d.top_k, np.zeros(1, np.int64))
        o = np.argsort(np.where(oi[0] < 0, np.iinfo(np.int64).max, oi[0].astype(np.int64)), kind="stable")
        assert np.array_equal(idx[t], oi[0][o]) and np.array_equal(sc[t], os_[0][o]), (t, p)
        assert idx[t].max() <= p
    for decode in (False, True):
        out, lse = dev.mla(idx, decode=decode)
        for t in range(int(N_Q.sum())):
            b, p = int(req[t]), int(POS[t])
            _, _, q_tok, rows = _one_token(x, t, b, p)
            ro, rl = oracle.attend(q_tok, rows, d.kv_format, d.D_v, idx[t], d.sm_scale)
            assert_attn_close(out[t][None], ro[None], lse[t][None], rl[None],
                              f"token {t} p={p} decode={decode}")


def test_batch_table_built_without_waiting():
    # a table assembled in pinned staging memory and copied on the stream without a wait gives
    # the same selection as the blocking build
    import ctypes
    import torch
    from sparse_mla_attention_indexer_amd import _lib, ops

    x = W.generate(W.small_big_dims(batch=2, n_q=5, cached=3000))
    d = x.dims
    say("[case] batch table through pinned staging, no wait")
    dev = Dev(x)
    ref_idx, ref_sc = dev.topk()
    nbytes = dev.plan.table.numel()
    staging = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    table = torch.empty(nbytes, dtype=torch.uint8, device=dev.device)
    desc = _lib.Batch()
    n_q = np.ascontiguousarray(x.n_q, np.int32)
    kv_len = np.ascontiguousarray(x.kv_len, np.int64)
    stream = torch.cuda.current_stream(dev.device).cuda_stream
    _lib.check("smla_batch_build_pos",
               _lib.lib().smla_batch_build_pos(d.batch, n_q.ctypes.data, kv_len.ctypes.data, None,
                                               staging.data_ptr(), table.data_ptr(), nbytes, stream,
                                               ctypes.byref(desc)))
    plan = ops.BatchPlan.__new__(ops.BatchPlan)
    plan.__dict__.update(dev.plan.__dict__)
    plan.table, plan.desc = table, desc
    idx, sc = ops.indexer_topk(plan, dev.q_idx, dev.k_idx, dev.w, d.top_k,
                               workspace=ops.topk_workspace(plan, d.H_I, d.D_I, d.top_k))
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), ref_idx) and np.array_equal(sc.cpu().numpy(), ref_sc)
