"""C-ABI checks that need no GPU: the library loads, exports every function include/smla.h
declares, and rejects bad arguments on the host before touching the device. Also checks that the
product never reaches the oracle."""
import ctypes
import os
import re

import numpy as np
import pytest

from sparse_mla_attention_indexer_amd import _build, _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions(name):
    text = open(os.path.join(ROOT, "include", name)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(smla_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        _build.build_hip()
    return _lib.lib()


def test_exports_every_declared_symbol(L):
    declared = _header_functions("smla.h")
    assert set(declared) == set(_lib.EXPORTS)
    for fn in declared:
        assert hasattr(L, fn), fn


def test_workload_library_exports_declared_symbols():
    from sparse_mla_attention_indexer_amd import workload as W

    L = W.lib()
    for fn in _header_functions("smla_workload.h"):
        assert hasattr(L, fn), fn


def _fake_batch(**kw):
    b = _lib.Batch()
    b.batch, b.total_q, b.max_q, b.n_items = 1, 4, 4, 1
    b.max_kv, b.total_rows, b.total_cand, b.min_cand = 100, 100, 394, 97
    b.table, b.table_bytes = 0x10000, 4096
    for k, v in kw.items():
        setattr(b, k, v)
    return b


FAKE = 0x20000  # aligned, never dereferenced: validation fails before any launch


def test_batch_build_rejects_bad_lengths(L):
    out = _lib.Batch()
    n_q = np.array([2, 5], np.int32)
    kv = np.array([10, 4], np.int64)  # n_q > kv_len in request 1
    rc = L.smla_batch_build(2, n_q.ctypes.data, kv.ctypes.data, FAKE, 1 << 20, None, ctypes.byref(out))
    assert rc == _lib.SMLA_E_INVALID and "request 1" in _lib.last_error()
    rc = L.smla_batch_build(0, n_q.ctypes.data, kv.ctypes.data, FAKE, 1 << 20, None, ctypes.byref(out))
    assert rc == _lib.SMLA_E_INVALID
    rc = L.smla_batch_build(1, n_q.ctypes.data, kv.ctypes.data, FAKE + 8, 1 << 20, None, ctypes.byref(out))
    assert rc == _lib.SMLA_E_INVALID and "aligned" in _lib.last_error()
    kv_ok = np.array([10, 9], np.int64)
    rc = L.smla_batch_build(2, n_q.ctypes.data, kv_ok.ctypes.data, FAKE, 64, None, ctypes.byref(out))
    assert rc == _lib.SMLA_E_WORKSPACE


def test_batch_build_pos_validation(L):
    # explicit positions: inside [0, kv_len), non-decreasing within a request (repeats allowed)
    out = _lib.Batch()
    n_q = np.array([3, 2], np.int32)
    kv = np.array([10, 6], np.int64)

    def build(pos):
        p = None if pos is None else np.asarray(pos, np.int64)
        return L.smla_batch_build_pos(2, n_q.ctypes.data, kv.ctypes.data,
                                      None if p is None else p.ctypes.data, None, FAKE, 64, None,
                                      ctypes.byref(out))

    # every check passes and only the (deliberately small) table is refused
    assert build([4, 4, 9, 0, 5]) == _lib.SMLA_E_WORKSPACE
    assert build([0, 0, 0, 5, 5]) == _lib.SMLA_E_WORKSPACE
    assert build(None) == _lib.SMLA_E_WORKSPACE
    assert build([4, 3, 9, 0, 5]) == _lib.SMLA_E_INVALID and "request 0 token 1" in _lib.last_error()
    assert build([4, 4, 10, 0, 5]) == _lib.SMLA_E_INVALID  # position == kv_len
    assert build([4, 4, 9, -1, 5]) == _lib.SMLA_E_INVALID
    assert build([4, 4, 9, 5, 6]) == _lib.SMLA_E_INVALID and "request 1 token 1" in _lib.last_error()


def test_dcp_shard_positions():
    # a shard's rows and its tokens' local positions, against counting the shard's rows that
    # each token sees one by one
    from sparse_mla_attention_indexer_amd import ops
    rng = np.random.default_rng(11)
    for _ in range(50):
        B = int(rng.integers(1, 4))
        n = int(rng.integers(1, 9))
        n_q = rng.integers(1, 6, size=B)
        kv_len = n_q + rng.integers(n, 60, size=B)
        for s in range(n):
            rows, pos = ops.dcp_shard_positions(n_q, kv_len, n, s)
            t = 0
            for b in range(B):
                owned = [g for g in range(int(kv_len[b])) if g % n == s]
                assert rows[b] == len(owned)
                for j in range(int(n_q[b])):
                    P = int(kv_len[b] - n_q[b] + j)
                    assert pos[t] == sum(1 for g in owned if g <= P) - 1
                    t += 1
    with pytest.raises(ValueError):
        ops.dcp_shard_positions([2], [3], 8, 5)  # position 1 sees no row of shard 5


def test_table_bytes_bounds(L):
    assert L.smla_batch_table_bytes(0, 1, 1) == 0
    assert L.smla_batch_table_bytes(1, 32768, 32768) > 0


def test_indexer_validation(L):
    b = _fake_batch()
    rc = L.smla_indexer_scores(None, FAKE, FAKE, FAKE, 64, 128, FAKE, None)
    assert rc == _lib.SMLA_E_INVALID
    rc = L.smla_indexer_scores(ctypes.byref(b), FAKE, FAKE, FAKE, 48, 128, FAKE, None)
    assert rc == _lib.SMLA_E_UNSUPPORTED
    rc = L.smla_indexer_scores(ctypes.byref(b), FAKE + 4, FAKE, FAKE, 64, 128, FAKE, None)
    assert rc == _lib.SMLA_E_INVALID
    rc = L.smla_indexer_scores(ctypes.byref(b), FAKE, FAKE, FAKE, 64, 128, None, None)
    assert rc == _lib.SMLA_E_INVALID
    uninit = _lib.Batch()
    rc = L.smla_indexer_scores(ctypes.byref(uninit), FAKE, FAKE, FAKE, 64, 128, FAKE, None)
    assert rc == _lib.SMLA_E_INVALID and "smla_batch_build" in _lib.last_error()


def test_topk_validation(L):
    b = _fake_batch()
    for k in (0, 2049):
        rc = L.smla_indexer_scores_topk(ctypes.byref(b), FAKE, FAKE, FAKE, 64, 128, k, FAKE, None,
                                        FAKE, 1 << 30, None)
        assert rc == _lib.SMLA_E_UNSUPPORTED
    need = L.smla_indexer_topk_workspace_bytes(ctypes.byref(b), 64, 128, 2048)
    assert need >= 394 * 4
    rc = L.smla_indexer_scores_topk(ctypes.byref(b), FAKE, FAKE, FAKE, 64, 128, 2048, FAKE, None,
                                    FAKE, need - 1, None)
    assert rc == _lib.SMLA_E_WORKSPACE
    rc = L.smla_indexer_scores_topk(ctypes.byref(b), FAKE, FAKE, FAKE, 64, 128, 2048, None, None,
                                    FAKE, need, None)
    assert rc == _lib.SMLA_E_INVALID


def test_fp8_indexer_validation(L):
    b = _fake_batch()
    rc = L.smla_indexer_scores_fp8(None, FAKE, FAKE, FAKE, FAKE, 64, 128, FAKE, None)
    assert rc == _lib.SMLA_E_INVALID
    rc = L.smla_indexer_scores_fp8(ctypes.byref(b), FAKE, FAKE, FAKE, FAKE, 16, 32, FAKE, None)
    assert rc == _lib.SMLA_E_UNSUPPORTED  # no generic FP8 kernel
    rc = L.smla_indexer_scores_fp8(ctypes.byref(b), FAKE, FAKE, None, FAKE, 64, 128, FAKE, None)
    assert rc == _lib.SMLA_E_INVALID      # the key scales are required
    rc = L.smla_indexer_scores_fp8(ctypes.byref(b), FAKE, FAKE + 8, FAKE, FAKE, 64, 128, FAKE, None)
    assert rc == _lib.SMLA_E_INVALID
    rc = L.smla_indexer_scores_fp8(ctypes.byref(b), FAKE, FAKE, FAKE + 2, FAKE, 64, 128, FAKE, None)
    assert rc == _lib.SMLA_E_INVALID
    need = L.smla_indexer_topk_workspace_bytes(ctypes.byref(b), 64, 128, 2048)
    for k in (0, 2049):
        rc = L.smla_indexer_scores_topk_fp8(ctypes.byref(b), FAKE, FAKE, FAKE, FAKE, 64, 128, k,
                                            FAKE, None, FAKE, need, None)
        assert rc == _lib.SMLA_E_UNSUPPORTED
    rc = L.smla_indexer_scores_topk_fp8(ctypes.byref(b), FAKE, FAKE, FAKE, FAKE, 64, 128, 2048,
                                        FAKE, None, FAKE, need - 1, None)
    assert rc == _lib.SMLA_E_WORKSPACE
    rc = L.smla_indexer_scores_topk_fp8(ctypes.byref(b), FAKE, FAKE, FAKE, FAKE, 64, 128, 2048,
                                        None, None, FAKE, need, None)
    assert rc == _lib.SMLA_E_INVALID


def test_dcp_merge_validation(L):
    # top-k merge: sizes, union cap, list stride, flag, pointers
    ok = dict(total_q=4, n_lists=8, k_in=2048, stride=4 * 2048, flt=0, top_k=2048)

    def merge(**kw):
        a = {**ok, **kw}
        return L.smla_topk_merge(a["total_q"], a["n_lists"], a["k_in"], FAKE, FAKE, a["stride"],
                                 a["flt"], a["top_k"], FAKE, None, a.get("local"), None)

    assert merge(n_lists=0) == _lib.SMLA_E_INVALID
    assert merge(n_lists=9) == _lib.SMLA_E_UNSUPPORTED   # 9 x 2048 candidates > 16,384
    assert merge(top_k=2049) == _lib.SMLA_E_UNSUPPORTED
    assert merge(stride=100) == _lib.SMLA_E_INVALID
    assert merge(flt=2) == _lib.SMLA_E_INVALID
    assert L.smla_topk_merge(4, 8, 2048, None, FAKE, 4 * 2048, 0, 2048, FAKE, None, None,
                             None) == _lib.SMLA_E_INVALID
    # the per-shard local lists: aligned, and at most 64 lists
    assert merge(local=FAKE + 2) == _lib.SMLA_E_INVALID
    assert merge(n_lists=65, k_in=16, stride=4 * 16, local=FAKE) == _lib.SMLA_E_UNSUPPORTED
    assert L.smla_dcp_local_indices(4, 2049, FAKE, 8, FAKE, None) == _lib.SMLA_E_INVALID
    assert L.smla_dcp_local_indices(4, 2048, FAKE, 0, FAKE, None) == _lib.SMLA_E_INVALID
    assert L.smla_dcp_local_indices(4, 2048, None, 8, FAKE, None) == _lib.SMLA_E_INVALID
    assert L.smla_lse_merge(4, 64, 512, 0, FAKE, FAKE, FAKE, None, None) == _lib.SMLA_E_INVALID
    assert L.smla_lse_merge(4, 64, 5000, 8, FAKE, FAKE, FAKE, None, None) == _lib.SMLA_E_INVALID
    assert L.smla_lse_merge(4, 64, 512, 8, FAKE, FAKE + 2, FAKE, None, None) == _lib.SMLA_E_INVALID


def test_hot_resolve_validation(L):
    # sizes, step, row size, pointers and aliasing are refused on the host; a host pointer
    # that is not pinned HIP memory is refused too (here: no runtime at all), never launched
    b = _fake_batch()
    ok = dict(top_k=2048, n_slots=4096, step=0, row_bytes=656, host=FAKE, idx=FAKE, out=FAKE + 256)

    def call(**kw):
        a = {**ok, **kw}
        return L.smla_hot_resolve(ctypes.byref(b), a["idx"], a["top_k"], FAKE, FAKE, a["n_slots"],
                                  FAKE, FAKE, a["step"], a["host"], 1 << 20, FAKE, a["row_bytes"],
                                  FAKE, a["out"], FAKE, None)

    assert call(top_k=0) == _lib.SMLA_E_UNSUPPORTED
    assert call(top_k=8193) == _lib.SMLA_E_UNSUPPORTED      # n_q * top_k above 8192
    assert call(n_slots=0) == _lib.SMLA_E_UNSUPPORTED
    assert call(n_slots=4097) == _lib.SMLA_E_UNSUPPORTED
    assert call(step=-1) == _lib.SMLA_E_INVALID
    assert call(row_bytes=650) == _lib.SMLA_E_INVALID
    assert call(host=None) == _lib.SMLA_E_INVALID
    assert call(host=FAKE + 8) == _lib.SMLA_E_INVALID        # 16-byte alignment
    assert call(out=FAKE) == _lib.SMLA_E_INVALID             # idx_out aliases idx
    assert call() == _lib.SMLA_E_INVALID                     # not pinned host memory


def test_mla_validation(L):
    b = _fake_batch()
    args = dict(H=64, D_qk=576, D_v=512)

    def call(fn="smla_sparse_mla_prefill", fmt=1, H=64, D_qk=576, D_v=512, k=2048, scale=0.04,
             q=FAKE, ws=FAKE, ws_bytes=1 << 30):
        return getattr(L, fn)(ctypes.byref(b), q, FAKE, fmt, H, D_qk, D_v, FAKE, k, scale, FAKE,
                              None, ws, ws_bytes, None)

    assert call(H=32) == _lib.SMLA_E_UNSUPPORTED
    assert call(D_qk=512) == _lib.SMLA_E_UNSUPPORTED
    assert call(fmt=7) == _lib.SMLA_E_INVALID
    assert call(fmt=0, H=64) == _lib.SMLA_E_UNSUPPORTED  # bf16 rows only on the small-head kernel
    assert call(k=0) == _lib.SMLA_E_UNSUPPORTED
    assert call(scale=0.0) == _lib.SMLA_E_INVALID
    assert call(q=FAKE + 2) == _lib.SMLA_E_INVALID
    need = L.smla_sparse_mla_workspace_bytes(ctypes.byref(b), 64, 512, 2048, 1)
    assert need > 0  # 4 tokens split across workgroups
    assert call("smla_sparse_mla_decode", ws_bytes=need - 1) == _lib.SMLA_E_WORKSPACE
    assert L.smla_sparse_mla_workspace_bytes(ctypes.byref(b), 64, 512, 2048, 0) == 0
    del args


def test_kv_append_validation(L):
    assert L.smla_kv_append(0, None, None, 0, None, None, None, None) == _lib.SMLA_OK  # no-op
    assert L.smla_kv_append(-1, FAKE, None, 0, FAKE, FAKE, None, None) == _lib.SMLA_E_INVALID
    assert L.smla_kv_append(4, None, None, 0, FAKE, FAKE, None, None) == _lib.SMLA_E_INVALID
    assert L.smla_kv_append(4, FAKE + 8, None, 0, FAKE, FAKE, None, None) == _lib.SMLA_E_INVALID
    assert "aligned" in _lib.last_error()
    assert L.smla_kv_append(4, FAKE, FAKE, 128, FAKE, FAKE, None, None) == _lib.SMLA_E_INVALID
    assert "k_idx" in _lib.last_error()
    for bad in (8, 24, 2048):
        rc = L.smla_kv_append(4, FAKE, FAKE, bad, FAKE, FAKE, FAKE, None)
        assert rc == _lib.SMLA_E_UNSUPPORTED, bad


def test_status_strings(L):
    assert _lib.status_str(0) == "SMLA_OK"
    assert _lib.status_str(-3) == "SMLA_E_WORKSPACE"
    assert L.smla_version() >= 100


def test_product_never_reaches_the_oracle():
    pkg = os.path.join(ROOT, "sparse_mla_attention_indexer_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h", ".c")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "smla_oracle" not in text, f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith((".c", ".h")):
            text = open(os.path.join(ROOT, "oracle", f)).read()
            assert "smla_internal" not in text and "hip" not in text.lower().replace("ship", ""), f
