"""GPU parity of the hot-buffer resolve (hybrid offload: a request's older rows in pinned host
memory, the selected ones served from a GPU hot buffer managed least-recently-used).

Over several steps with drifting selections (hits and misses), the library's rewritten
selections, the slot table (token and last use), the copy counts and the hot rows themselves
must equal the oracle's bit for bit; attention over the rewritten selections, with every
offloaded device row overwritten, must match the oracle's attention over the original
selections and the whole cache.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_mla_attention_indexer_amd import ops
from sparse_mla_attention_indexer_amd import workload as W

pytestmark = pytest.mark.gpu

from gpu_harness import Dev, assert_attn_close, oracle_mla, say  # noqa: E402

POISON = 0xEE


class Offload:
    """A batch whose rows below resident_from[b] are only in pinned host memory (the device
    copies are overwritten with POISON), with a hot buffer of n_slots rows at hot_base[b]."""

    def __init__(self, n_q, kv_len, rows, resident_from, hot_base, n_slots, device="cuda:0",
                 poison=POISON):
        self.dv = torch.device(device)
        self.plan = ops.BatchPlan(n_q, kv_len, self.dv)
        self.n_q, self.kv_len = np.asarray(n_q), np.asarray(kv_len, np.int64)
        self.row0 = np.concatenate([[0], np.cumsum(self.kv_len)[:-1]]).astype(np.int64)
        self.rows = rows
        self.host = torch.from_numpy(rows).pin_memory()
        dev_rows = rows.copy()
        for b, rf in enumerate(resident_from):
            dev_rows[self.row0[b]: self.row0[b] + rf] = poison
        self.kv = torch.from_numpy(dev_rows).to(self.dv)
        self.rf = np.asarray(resident_from, np.int32)
        self.hb = np.asarray(hot_base, np.int32)
        B = len(n_q)
        self.t_rf = torch.from_numpy(self.rf).to(self.dv)
        self.t_hb = torch.from_numpy(self.hb).to(self.dv)
        self.t_h0 = torch.from_numpy(self.row0).to(self.dv)
        self.tok = torch.full((B, n_slots), -1, dtype=torch.int32, device=self.dv)
        self.age = torch.full((B, n_slots), -1, dtype=torch.int32, device=self.dv)
        self.o_tok = np.full((B, n_slots), -1, np.int32)
        self.o_age = np.full((B, n_slots), -1, np.int32)

    def step(self, idx_np, step):
        idx = torch.from_numpy(np.ascontiguousarray(idx_np, np.int32)).to(self.dv)
        out, nc = ops.hot_resolve(self.plan, idx, self.t_rf, self.t_hb, self.tok, self.age, step,
                                  self.host, self.t_h0, self.kv)
        torch.cuda.synchronize()
        return out.cpu().numpy(), nc.cpu().numpy()

    def check_against_oracle(self, idx_np, step, label):
        got, nc = self.step(idx_np, step)
        q0 = 0
        for b, nq in enumerate(self.n_q):
            sel = idx_np[q0: q0 + nq]
            try:
                ref, cp = oracle.hot_resolve(sel, int(self.rf[b]), self.o_tok[b], self.o_age[b], step,
                                             int(self.hb[b]), kv_len=int(self.kv_len[b]))
                want_nc = len(cp)
            except oracle.HotResolveOverflow:
                ref, want_nc = np.full_like(sel, -1), -1
            except oracle.HotResolveBounds:
                ref, want_nc = np.full_like(sel, -1), -2
            assert np.array_equal(got[q0: q0 + nq], ref), f"{label}: request {b} selections differ"
            assert nc[b] == want_nc, f"{label}: request {b} copied {nc[b]}, oracle {want_nc}"
            q0 += nq
        assert np.array_equal(self.tok.cpu().numpy(), self.o_tok), f"{label}: slot tokens differ"
        assert np.array_equal(self.age.cpu().numpy(), self.o_age), f"{label}: slot ages differ"
        kv = self.kv.cpu().numpy()
        for b in range(len(self.n_q)):
            for s in np.nonzero(self.o_tok[b] >= 0)[0]:
                r = self.row0[b] + self.hb[b] + s
                assert np.array_equal(kv[r], self.rows[self.row0[b] + self.o_tok[b, s]]), (label, b, s)
        return nc


def _drifting_selection(rng, n_q, kv_len, rf, top_k, centre, spread):
    """Per token: top_k distinct rows, most of them near `centre` in the offloaded range, some
    resident, ascending, the tail padded with -1."""
    out = []
    for nq, kl, r in zip(n_q, kv_len, rf):
        for _ in range(nq):
            n_valid = int(rng.integers(top_k // 2, top_k + 1))
            lo = max(0, centre - spread)
            pool = np.arange(lo, min(kl, max(r, 1) if r > 0 else kl, centre + spread))
            n_off = min(pool.size, int(n_valid * 0.8)) if r > 0 else 0
            a = rng.choice(pool, size=n_off, replace=False) if n_off else np.zeros(0, np.int64)
            res = rng.choice(np.arange(r, kl), size=min(n_valid - n_off, kl - r), replace=False)
            v = np.sort(np.concatenate([a, res]))
            row = np.full(top_k, -1, np.int32)
            row[: v.size] = v
            out.append(row)
    return np.stack(out)


def test_hot_resolve_steps_against_oracle():
    rng = np.random.default_rng(0x407)
    n_q = np.array([1, 3, 2, 1], np.int32)
    kv_len = np.array([6000, 9000, 5000, 3000], np.int64)
    rf = [4000, 6000, 0, 3000]     # request 2 fully resident; request 3 fully offloaded
    hb = [0, 100, 0, 2000]
    n_slots, top_k = 512, 256
    rows = rng.integers(0, 256, size=(int(kv_len.sum()), 656), dtype=np.uint8)
    off = Offload(n_q, kv_len, rows, rf, hb, n_slots)
    say("[case] hot resolve: 4 requests, 8 steps, 512 slots, top_k 256")
    total = 0
    for step in range(8):
        centre = 600 + 180 * step
        idx = _drifting_selection(rng, n_q, kv_len, rf, top_k, centre, 260)
        if step == 5:  # a decode token's list out of order: the sorting path
            rng.shuffle(idx[0])
        last = off.check_against_oracle(idx, step, f"step {step}")
        total += int(last[last > 0].sum())
    assert total > 0
    # the same selection again: all hits, nothing copied
    nc = off.check_against_oracle(idx, 8, "repeat")
    assert (nc[(np.array(rf) > 0) & (last >= 0)] == 0).all()


def test_hot_resolve_rejections():
    rng = np.random.default_rng(0x408)
    n_q = np.array([1, 1, 1, 1], np.int32)
    kv_len = np.array([3000, 3000, 3000, 3000], np.int64)
    rows = rng.integers(0, 256, size=(12000, 656), dtype=np.uint8)
    # request 1: hot buffer overlaps resident rows; request 2: host rows outside the pool
    off = Offload(n_q, kv_len, rows, [2000, 2000, 2000, 2000], [0, 1800, 0, 0], 256)
    off.t_h0[2] = 11000
    idx = np.full((4, 300), -1, np.int32)
    idx[0, :200] = np.arange(200) * 3               # fits
    idx[1, :10] = np.arange(10)
    idx[2, :10] = np.arange(10)
    idx[3, :300] = np.arange(300)                   # 300 distinct offloaded rows > 256 slots
    got, nc = off.step(idx, 0)
    assert nc.tolist() == [200, -2, -3, -1]
    assert (got[1:] == -1).all()
    t = off.tok.cpu().numpy()
    assert (t[1:] == -1).all() and (off.age.cpu().numpy()[1:] == -1).all()
    ref, _ = oracle.hot_resolve(idx[:1], 2000, off.o_tok[0], off.o_age[0], 0, 0)
    assert np.array_equal(got[:1], ref)
    # pageable host memory is refused before anything runs
    with pytest.raises(ValueError):
        ops.hot_resolve(off.plan, torch.from_numpy(idx).to(off.dv), off.t_rf, off.t_hb, off.tok,
                        off.age, 1, torch.from_numpy(rows), off.t_h0, off.kv)


def test_hot_resolve_request_bound_two_tokens():
    # two query tokens per request (positions kv_len - 2 and kv_len - 1): the offloaded prefix
    # may end at the first token's own row (resident_from = kv_len - 1) but not past it
    rng = np.random.default_rng(0x40B)
    n_q = np.array([2, 2], np.int32)
    kv_len = np.array([3000, 3000], np.int64)
    rows = rng.integers(0, 256, size=(6000, 656), dtype=np.uint8)
    off = Offload(n_q, kv_len, rows, [2999, 3000], [100, 100], 256)
    idx = np.full((4, 128), -1, np.int32)
    for t, p in enumerate((2998, 2999, 2998, 2999)):
        idx[t, :100] = np.arange(100) * 7
        idx[t, 100] = p
    say("[case] hot resolve: resident_from at kv_len - n_q + 1 and one past it")
    nc = off.check_against_oracle(idx, 0, "request bound")
    assert nc.tolist() == [101, -2]


def _nan_row():
    """A 656-byte row of NaN codes, non-finite block scales and NaN rope dims."""
    r = np.full(656, 0x7F, np.uint8)
    r[512:528] = np.array([np.nan, np.inf, -np.inf, np.nan], np.float32).view(np.uint8)
    r[528:656] = np.full(64, 0x7FC0, np.uint16).view(np.uint8)
    return r


@pytest.mark.parametrize("decode", [False, True])
def test_hot_resolve_hot_base_padded_lists_attention(decode):
    # hot buffers at hot_base > 0 inside offloaded prefixes whose device rows (row 0 included)
    # hold NaN rows; selections with -1 holes in the middle, lists cut short, and a request whose
    # kv_len is below top_k (its lists are padded by the selection itself); the attention over
    # the resolved selections must match the oracle's over the original ones and the clean cache
    x = W.generate(W.small_big_dims(batch=3, n_q=2, cached=5000, seed=0x5EED4200))
    d = x.dims
    n_q = np.array([2, 2, 2], np.int32)
    kv_len = np.array([5002, 1500, 5002], np.int64)
    dev = Dev(x, n_q=n_q, kv_len=kv_len)
    idx, _ = dev.topk(with_scores=False)
    assert (idx[2:4] < 0).any(axis=1).all(), "request 1 should have padded lists"
    rng = np.random.default_rng(0x40C)
    sel = idx.copy()
    sel[rng.random(sel.shape) < 0.12] = -1
    sel[0, 1300:] = -1
    sel[5, 900:] = -1
    rf = [4600, 0, 4700]
    hb = [300, 0, 500]
    say(f"[case] hot resolve at hot_base {hb} over NaN rows, padded lists, decode={decode}")
    off = Offload(n_q, kv_len, x.kv, rf, hb, 4096, poison=_nan_row())
    nc = off.check_against_oracle(sel, 0, "hot_base > 0, step 0")
    assert nc[0] > 0 and nc[2] > 0 and nc[1] == 0
    got_idx, nc = off.step(sel, 1)
    assert (nc == 0).all()
    idx_t = torch.from_numpy(got_idx).to(off.dv)
    out, lse = ops.sparse_mla(off.plan, dev.q, off.kv, d.kv_format, d.D_v, idx_t, d.sm_scale,
                              decode=decode)
    torch.cuda.synchronize()
    tokens = np.arange(int(n_q.sum()))
    ref_o, ref_l = oracle_mla(x, sel, tokens, n_q=n_q, kv_len=kv_len)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert_attn_close(got, ref_o, lse.cpu().numpy(), ref_l, f"hot_base > 0 decode={decode}")


def test_hot_resolve_then_attention_decode():
    # a decode batch whose older rows are offloaded: top-k, resolve into a hot buffer of twice
    # top-k rows, attention over the resolved rows with every offloaded device row overwritten
    x = W.generate(W.small_big_dims(batch=4, n_q=1, cached=20000))
    d = x.dims
    dev = Dev(x)
    say(f"[case] hot resolve + attention: B={d.batch} kv_len={int(x.kv_len[0])}")
    ref_idx, _ = dev.topk()
    rf = (x.kv_len - 4096).astype(np.int32)
    n_slots = 2 * d.top_k
    off = Offload(x.n_q, x.kv_len, x.kv, rf, np.zeros(d.batch, np.int32), n_slots)
    nc = off.check_against_oracle(ref_idx, 0, "decode cold step")
    assert (nc > 0).all()
    got_idx, nc = off.step(ref_idx, 1)  # the same selection again: all hits
    assert (nc == 0).all()
    idx_t = torch.from_numpy(got_idx).to(off.dv)
    out, lse = ops.sparse_mla(off.plan, dev.q, off.kv, d.kv_format, d.D_v, idx_t, d.sm_scale,
                              decode=True)
    torch.cuda.synchronize()
    sample = np.arange(d.batch)
    ref_o, ref_l = oracle_mla(x, ref_idx[sample], sample)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)[sample]
    assert_attn_close(got, ref_o, lse.cpu().numpy()[sample], ref_l, "hot-resolved attention")


def test_hot_resolve_maximum_sizes():
    # the limits: 4 tokens x top-k 2,048 = 8,192 selections per request (the sorting path at its
    # largest) and 4,096 slots; later steps move the selection window so the buffer fills and
    # least-recently-used slots are evicted
    rng = np.random.default_rng(0x409)
    n_q = np.array([4, 4], np.int32)
    kv_len = np.array([200000, 120000], np.int64)
    rf = [150000, 100000]
    rows = rng.integers(0, 256, size=(int(kv_len.sum()), 656), dtype=np.uint8)
    off = Offload(n_q, kv_len, rows, rf, [0, 5000], 4096)
    say("[case] hot resolve maximum sizes: 2 x 4 tokens x 2048, 4096 slots")
    for step, lo in enumerate((0, 2000, 4000, 4000)):
        idx = np.full((8, 2048), -1, np.int32)
        for t in range(8):
            b = t // 4
            o = np.sort(rng.choice(np.arange(lo, lo + 3000) + (0 if b == 0 else 6000), 1500, replace=False))
            r = np.sort(rng.choice(np.arange(rf[b], int(kv_len[b])), 548, replace=False))
            idx[t] = np.concatenate([o, r])
        nc = off.check_against_oracle(idx, step, f"max step {step}")
        assert (nc >= 0).all()
        say(f"  step {step}: rows copied {nc.tolist()}")


def test_hot_resolve_long_rows_and_prefill_attention():
    # two tokens per request sharing the buffer: the prefill entry point attends over the
    # resolved rows; the same selections over 1,152-byte rows (a bf16 576-dim row: 72 x 16 bytes,
    # so a lane copies more than one piece of a row) match the oracle too
    x = W.generate(W.small_big_dims(batch=3, n_q=2, cached=6000, top_k=512, seed=0x5EED4100))
    d = x.dims
    dev = Dev(x)
    say(f"[case] hot resolve + prefill attention: B={d.batch} n_q=2 kv_len={int(x.kv_len[0])}")
    ref_idx, _ = dev.topk()
    rf = (x.kv_len - 1500).astype(np.int32)
    off = Offload(x.n_q, x.kv_len, x.kv, rf, np.zeros(d.batch, np.int32), 2 * d.top_k)
    nc = off.check_against_oracle(ref_idx, 0, "two tokens, step 0")
    assert (nc > 0).all()
    got_idx, nc = off.step(ref_idx, 1)
    assert (nc == 0).all()
    idx_t = torch.from_numpy(got_idx).to(off.dv)
    out, lse = ops.sparse_mla(off.plan, dev.q, off.kv, d.kv_format, d.D_v, idx_t, d.sm_scale,
                              decode=False)
    torch.cuda.synchronize()
    sample = np.arange(d.total_q)
    ref_o, ref_l = oracle_mla(x, ref_idx[sample], sample)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)[sample]
    assert_attn_close(got, ref_o, lse.cpu().numpy()[sample], ref_l, "hot-resolved prefill")
    rng = np.random.default_rng(0x40A)
    long_rows = rng.integers(0, 256, size=(d.total_rows, 1152), dtype=np.uint8)
    off2 = Offload(x.n_q, x.kv_len, long_rows, rf, np.full(d.batch, 7, np.int32), 2 * d.top_k)
    off2.check_against_oracle(ref_idx, 0, "1152-byte rows, step 0")
    shifted = np.where(ref_idx >= 0, np.maximum(ref_idx - 900, 0), -1).astype(np.int32)
    for t in range(shifted.shape[0]):  # keep each token's list distinct and ascending
        v = np.unique(shifted[t][shifted[t] >= 0])
        shifted[t] = -1
        shifted[t, : v.size] = v
    off2.check_against_oracle(shifted, 1, "1152-byte rows, step 1")
