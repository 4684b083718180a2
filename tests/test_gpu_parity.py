"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, element by element.

Index sets and scores must be bit-exact; attention outputs within max-abs 2e-2 and relative L2
1e-2 of the fp64 oracle on the same dequantised inputs. Small cases compare every token; the
full-size workloads compare sampled tokens the oracle computes one by one, in the launch
configuration the benchmark times.
"""
import numpy as np
import pytest

from sparse_mla_attention_indexer_amd import workload as W

pytestmark = pytest.mark.gpu

try:  # imported lazily so CPU-only collection never touches the GPU
    from gpu_harness import (Dev, assert_attn_close, assert_topk_equal, oracle_mla,
                             oracle_topk, say)
except Exception:  # pragma: no cover
    raise


def _full_case(x, label, decode_too=True, top_k=None):
    d = x.dims
    top_k = d.top_k if top_k is None else top_k
    say(f"[case] {label}: B={d.batch} n_q={d.n_q} cached={d.cached} k={top_k}")
    dev = Dev(x)
    tokens = np.arange(d.total_q)
    idx, sc = dev.topk(top_k)
    ref_idx, ref_sc = oracle_topk(x, tokens, top_k)
    assert_topk_equal(idx, sc, ref_idx, ref_sc, label)
    out, lse = dev.mla(idx)
    ref, ref_lse = oracle_mla(x, ref_idx, tokens)
    assert_attn_close(out, ref, lse.reshape(ref_lse.shape), ref_lse, label + " prefill")
    if decode_too:
        out, lse = dev.mla(idx, decode=True)
        assert_attn_close(out, ref, lse.reshape(ref_lse.shape), ref_lse, label + " decode")
    return dev, idx


def test_tiny_config_scores_topk_attention():
    x = W.generate(W.config_dims(0))
    dev, _ = _full_case(x, "tiny")
    # full score matrix against the oracle, -1 above the diagonal
    import oracle

    s = dev.scores()
    d = x.dims
    for t in range(0, d.total_q, 37):
        ref = oracle.indexer_scores(x.q_idx[t], x.k_idx[: t + 1], x.w)
        assert np.array_equal(s[t, : t + 1], ref)
        assert (s[t, t + 1:] == -1).all()


def test_big_shape_scores_full_matrix_mfma():
    import oracle

    x = W.generate(W.small_big_dims(batch=2, n_q=37, cached=300))
    say("[case] mfma scores 2x37 after 300")
    dev = Dev(x)
    s = dev.scores()
    d = x.dims
    for t in range(d.total_q):
        b, j = divmod(t, d.n_q)
        p = d.cached + j
        keys = x.k_idx[b * d.max_kv: b * d.max_kv + p + 1]
        assert np.array_equal(s[t, : p + 1], oracle.indexer_scores(x.q_idx[t], keys, x.w)), t
        assert (s[t, p + 1:] == -1).all()


def _fold_edge_queries(x):
    """Per token, queries on both sides of the weight fold's limit (every w_h q[d] inside int8):
    t % 3 == 0 one value one past it (that token is scored without folding), t % 3 == 1 the
    extreme values that still fold, t % 3 == 2 unchanged."""
    w = x.w.astype(np.int64)
    for t in range(x.q_idx.shape[0]):
        if t % 3 == 0:
            h = (7 * t) % 64
            x.q_idx[t, h, 3] = min(127, 127 // w[h] + 1)
        elif t % 3 == 1:
            x.q_idx[t, :, 0] = (127 // w).astype(np.int8)
            x.q_idx[t, :, 1] = (-(128 // w)).astype(np.int8)


@pytest.mark.parametrize("n_q,batch,cached", [(37, 2, 300), (1, 6, 5000)])
def test_indexer_weight_fold_limits(n_q, batch, cached):
    # tokens whose w q fits int8 are scored with the weights folded into the queries, the others
    # with the weights applied after the ReLU; both must match the oracle exactly, in the
    # multi-token kernel (n_q = 37) and the single-token one (decode)
    import oracle

    x = W.generate(W.small_big_dims(batch=batch, n_q=n_q, cached=cached))
    _fold_edge_queries(x)
    say(f"[case] weight fold limits B={batch} n_q={n_q} cached={cached}")
    dev = Dev(x)
    s = dev.scores()
    d = x.dims
    for t in range(d.total_q):
        b, j = divmod(t, d.n_q)
        p = d.cached + j
        keys = x.k_idx[b * d.max_kv: b * d.max_kv + p + 1]
        assert np.array_equal(s[t, : p + 1], oracle.indexer_scores(x.q_idx[t], keys, x.w)), t
    tokens = np.arange(d.total_q)
    idx, sc = dev.topk()
    ref_idx, ref_sc = oracle_topk(x, tokens)
    assert_topk_equal(idx, sc, ref_idx, ref_sc, "fold limits")


def test_big_shape_prefill_boundary_positions():
    # positions 2000..2299 cross p + 1 = k - 1, k, k + 1
    _full_case(W.generate(W.small_big_dims(n_q=300, cached=2000)), "prefill 300 after 2000")


@pytest.mark.parametrize("top_k", [1, 100, 777])
def test_big_shape_other_k(top_k):
    x = W.generate(W.small_big_dims(n_q=24, cached=1500, top_k=top_k, seed=0x5EED2000 + top_k))
    _full_case(x, f"k={top_k}", decode_too=False, top_k=top_k)


def test_ragged_batch_both_topk_paths_and_decode():
    # one request per shape family: short (p+1 < k), around k, and > 32768 candidates (the
    # histogram / filter / resolve path)
    n_q = np.array([1, 4, 2, 3, 1], np.int32)
    kv_len = np.array([3000, 50, 2049, 40000, 2048], np.int64)
    d = W.small_big_dims(batch=1, n_q=int(n_q.sum()), cached=int(kv_len.sum() - n_q.sum()))
    x = W.generate(d)
    x.n_q, x.kv_len = n_q, kv_len
    say("[case] ragged batch", n_q.tolist(), kv_len.tolist())
    dev = Dev(x)
    tokens = np.arange(int(n_q.sum()))
    idx, sc = dev.topk()
    ref_idx, ref_sc = oracle_topk(x, tokens)
    assert_topk_equal(idx, sc, ref_idx, ref_sc, "ragged")
    idx2, sc2 = dev.topk()
    assert np.array_equal(idx, idx2) and np.array_equal(sc, sc2), "top-k not deterministic"
    ref, ref_lse = oracle_mla(x, ref_idx, tokens)
    for decode in (False, True):
        out, lse = dev.mla(idx, decode=decode)
        assert_attn_close(out, ref, lse, ref_lse, f"ragged decode={decode}")


@pytest.mark.parametrize("cached", [40000, 300000])
@pytest.mark.parametrize("pattern", ["zeros", "few_values", "random"])
def test_tie_stress_long_rows(pattern, cached):
    # rows longer than the LDS path (40,000: one workgroup per row; 300,000: the segmented
    # three-kernel path) with massive ties: every score equal (the candidate buffer overflows and
    # the row is resolved from the scores directly), a few distinct values, or random scores
    d = W.small_big_dims(n_q=3, cached=cached)
    x = W.generate(d)
    if pattern == "zeros":
        x.k_idx[:] = 0
    elif pattern == "few_values":
        rng = np.random.default_rng(5)
        x.k_idx[:] = 0
        x.k_idx[:, 0] = rng.integers(0, 3, size=x.k_idx.shape[0])
        x.q_idx[:] = 1
    say(f"[case] tie stress {pattern} cached={cached}")
    dev = Dev(x)
    tokens = np.arange(d.total_q)
    idx, sc = dev.topk()
    ref_idx, ref_sc = oracle_topk(x, tokens)
    assert_topk_equal(idx, sc, ref_idx, ref_sc, f"ties {pattern}")
    if pattern == "zeros":
        assert (idx == np.arange(2048)[None, :]).all()


@pytest.mark.parametrize("pattern", ["random", "zeros", "few_values"])
def test_many_long_rows_one_workgroup_per_row(pattern):
    # more query tokens than the segmented path takes, rows between the LDS and the register
    # limits: one workgroup per row; sampled tokens against the oracle, properties everywhere
    d = W.small_big_dims(n_q=200, cached=36000)
    x = W.generate(d)
    if pattern == "zeros":
        x.k_idx[:] = 0
    elif pattern == "few_values":
        rng = np.random.default_rng(9)
        x.k_idx[:] = 0
        x.k_idx[:, 0] = rng.integers(0, 3, size=x.k_idx.shape[0])
        x.q_idx[:] = 1
    say(f"[case] many long rows {pattern}")
    dev = Dev(x)
    idx, sc = dev.topk()
    tokens = np.array([0, 1, 57, 133, 198, 199])
    ref_idx, ref_sc = oracle_topk(x, tokens)
    assert_topk_equal(idx[tokens], sc[tokens], ref_idx, ref_sc, f"many rows {pattern}")
    pos = dev.plan.positions
    assert (idx >= 0).all() and (idx <= pos[:, None]).all()
    assert (np.diff(idx, axis=1) > 0).all()
    if pattern == "zeros":
        assert (idx == np.arange(d.top_k)[None, :]).all()
    idx2, sc2 = dev.topk()  # the workspace the first call left behind serves the second
    assert np.array_equal(idx, idx2) and np.array_equal(sc, sc2)


def test_tie_stress_short_rows():
    d = W.small_big_dims(n_q=40, cached=3000)
    x = W.generate(d)
    x.k_idx[:] = 0
    x.k_idx[::7, 3] = 1
    x.q_idx[:] = 2
    say("[case] tie stress short rows")
    dev = Dev(x)
    tokens = np.arange(d.total_q)
    idx, sc = dev.topk()
    ref_idx, ref_sc = oracle_topk(x, tokens)
    assert_topk_equal(idx, sc, ref_idx, ref_sc, "short ties")


def test_mla_with_oracle_indices_unsorted_and_padded():
    # kernel isolation: the oracle's selection (its own order) drives the GPU attention, with
    # some entries knocked out to -1 in the middle of rows
    d = W.small_big_dims(n_q=20, cached=2500)
    x = W.generate(d)
    tokens = np.arange(d.total_q)
    ref_idx, _ = oracle_topk(x, tokens)
    rng = np.random.default_rng(11)
    ref_idx = ref_idx.copy()
    ref_idx[rng.random(ref_idx.shape) < 0.1] = -1
    say("[case] mla with oracle indices")
    dev = Dev(x)
    ref, ref_lse = oracle_mla(x, ref_idx, tokens)
    for decode in (False, True):
        out, lse = dev.mla(ref_idx, decode=decode)
        assert_attn_close(out, ref, lse, ref_lse, f"oracle idx decode={decode}")


def test_mla_growing_logits_recompute():
    # The rope dims (a part of the key only, not of the value) of row s are scaled by
    # 2^floor(12 s / rows): the logits of the later selected rows grow thousands of times larger
    # than those of the first tile, far beyond what an fp16 P can span from the reference the
    # first tile sets, so the kernel must notice and recompute the split with the true maximum
    # (prefill: one split over all selected rows). Scaling by powers of two keeps the bf16 values
    # exact; they stay inside the fp16 range (|x| < 5 * 2^12), and the values stay N(0, 1).
    d = W.small_big_dims(n_q=4, cached=3000)
    x = W.generate(d)
    rows = x.kv.shape[0]
    rope = x.kv[:, 528:656].copy().view(np.uint16).astype(np.uint32) << 16
    grow = np.exp2(np.floor(12.0 * np.arange(rows) / rows)).astype(np.float32)
    scaled = (rope.view(np.float32) * grow[:, None]).view(np.uint32) >> 16
    x.kv[:, 528:656] = scaled.astype(np.uint16).view(np.uint8)
    say("[case] growing logits")
    dev = Dev(x)
    tokens = np.arange(d.total_q)
    idx, sc = dev.topk()
    ref_idx, ref_sc = oracle_topk(x, tokens)
    assert_topk_equal(idx, sc, ref_idx, ref_sc, "growing logits")
    ref, ref_lse = oracle_mla(x, ref_idx, tokens)
    for decode in (False, True):
        out, lse = dev.mla(idx, decode=decode)
        assert_attn_close(out, ref, lse, ref_lse, f"growing logits decode={decode}")


# ---- full-size workloads, sampled tokens -------------------------------------------------

def _sampled_full_config(cid, tokens, decode):
    d = W.config_dims(cid)
    say(f"[case] config {cid} ({W.CONFIG_NAMES[cid]}): generating")
    x = W.generate(d)
    dev = Dev(x)
    say(f"[case] config {cid}: top-k")
    idx, sc = dev.topk()
    tokens = np.asarray(sorted(set(int(t) for t in tokens if 0 <= t < d.total_q)))
    assert tokens.size >= min(256, d.total_q), tokens.size
    say(f"[case] config {cid}: oracle on {tokens.size} tokens")
    ref_idx, ref_sc = oracle_topk(x, tokens)
    assert_topk_equal(idx[tokens], sc[tokens], ref_idx, ref_sc, f"config {cid}")
    say(f"[case] config {cid}: sparse MLA decode={decode}")
    out, lse = dev.mla(idx, decode=decode)
    out = out.reshape(d.total_q, d.H, d.D_v)
    lse = lse.reshape(d.total_q, d.H)
    ref, ref_lse = oracle_mla(x, ref_idx, tokens)
    assert_attn_close(out[tokens], ref, lse[tokens], ref_lse, f"config {cid}")
    # properties at every token: finite outputs, sorted unique indices within [0, p]
    assert np.isfinite(lse).all()
    pos = dev.plan.positions
    valid = idx >= 0
    assert (np.where(valid, idx, 0) <= pos[:, None]).all()
    assert ((np.diff(np.where(valid, idx, np.iinfo(np.int32).max), axis=1) > 0) | ~valid[:, 1:]).all()
    assert (valid.sum(1) == np.minimum(pos + 1, d.top_k)).all()


def test_kv_append_rows_bit_exact_against_oracle_encoder():
    # 301 new tokens (ragged against the 4 rows of a workgroup) into prefilled caches: N(0,1)
    # rows plus blocks that are all zero, tiny, huge, all negative, and one whose quotients fall
    # exactly on E4M3 ties; every written row must equal the oracle's encoding byte for byte, and
    # every other row must be untouched
    import torch

    import oracle
    from sparse_mla_attention_indexer_amd import ops

    say("[case] kv append 301 rows")
    rng = np.random.default_rng(2024)
    n, R, D_I = 301, 1000, 128
    lat = rng.standard_normal((n, 576))
    lat[0] = 0.0
    lat[1, 128:256] = 0.0
    lat[2, 256:384] *= 1e-30
    lat[3, 0:128] *= 1e30
    lat[4, 384:512] = -np.abs(lat[4, 384:512])
    lat[5, 0:128] = 0.0
    lat[5, 0], lat[5, 1], lat[5, 2], lat[5, 3] = 448.0, 1.0625, 1.1875, 3 * 2.0 ** -10  # scale 1
    lat_t = torch.from_numpy(lat.astype(np.float32)).to(torch.bfloat16)
    bits = lat_t.view(torch.int16).numpy().view(np.uint16)
    rows = rng.permutation(R)[:n].astype(np.int64)
    k_new = rng.integers(-128, 128, (n, D_I), dtype=np.int8)
    dev = torch.device("cuda:0")
    kv = torch.full((R, 656), 0xA5, dtype=torch.uint8, device=dev)
    k_idx = torch.full((R, D_I), 0x5A, dtype=torch.int8, device=dev)
    ops.kv_append(lat_t.to(dev), torch.from_numpy(rows).to(dev), kv, torch.from_numpy(k_new).to(dev), k_idx)
    ops.kv_append(lat_t[:0].to(dev), torch.empty(0, dtype=torch.int64, device=dev), kv)  # no-op
    got_kv, got_k = kv.cpu().numpy(), k_idx.cpu().numpy()
    for i in range(n):
        ref = oracle.fp8_row_encode(bits[i])
        assert np.array_equal(got_kv[rows[i]], ref), (i, np.nonzero(got_kv[rows[i]] != ref)[0][:8])
        assert np.array_equal(got_k[rows[i]], k_new[i]), i
    rest = np.setdiff1d(np.arange(R), rows)
    assert (got_kv[rest] == 0xA5).all() and (got_k[rest] == 0x5A).all()
    # the special rows decode as expected too
    assert not got_kv[rows[0], :512].any()
    assert (got_kv[rows[5], :4] == np.array([0x7E, 0x38, 0x3A, 0x02], np.uint8)).all()


def test_config1_decode_full_size():
    _sampled_full_config(1, range(32), decode=True)


def _spread_and_seams(n_tok, n_even, extra):
    """n_even tokens spread evenly over [0, n_tok), plus `extra`: the query-tile seams (tiles of 4
    tokens, tile i paired with tile n - 1 - i, so the middle pair shares a seam), the ends."""
    tiles = n_tok // 4
    mid = 4 * (tiles // 2)
    seams = [3, 4, 7, 8, mid - 5, mid - 4, mid - 1, mid, mid + 3, mid + 4, n_tok - 5, n_tok - 4]
    ends = [0, 1, 2, n_tok - 2, n_tok - 1]
    return np.linspace(0, n_tok - 1, n_even).astype(np.int64).tolist() + seams + ends + list(extra)


def test_config2_chunked_full_size():
    # 2,048 tokens after 65,536 cached: every row spans many 4,096-key chunks of the plan
    _sampled_full_config(2, _spread_and_seams(2048, 248, []), decode=False)


def test_config3_prefill_full_size():
    # p + 1 = 2,047 / 2,048 / 2,049 (the top-k fills exactly), rows ending on both sides of every
    # 4,096-key chunk edge up to 32K, and the tile-pair seams
    edges = [e + o for e in range(4096, 32768, 4096) for o in (-1, 0)]
    _sampled_full_config(3, _spread_and_seams(32768, 232, [2046, 2047, 2048] + edges), decode=False)


def test_config4_million_full_size():
    _sampled_full_config(4, range(16), decode=True)
