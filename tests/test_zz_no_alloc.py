"""smla_sparse_mla_decode_noalloc (split partials in the library's built-in scratch) against
smla_sparse_mla_decode (split partials in a caller workspace): both run the same kernels with the
same split plan, so outputs and lse must agree bit for bit. Two calls in a row on one GPU, the
second with fewer query tokens (it reuses the scratch the first left behind), then the largest
partial count the split rule produces (255 query tokens, 2 splits each: 510 of the 512 slots).
"""
import numpy as np
import pytest
import torch

from sparse_mla_attention_indexer_amd import ops
from sparse_mla_attention_indexer_amd import workload as W

pytestmark = pytest.mark.gpu

from gpu_harness import Dev, assert_attn_close, oracle_mla, say  # noqa: E402


def _both(dev, idx_np):
    d = dev.x.dims
    idx = torch.from_numpy(np.ascontiguousarray(idx_np, np.int32)).to(dev.device)
    tq = dev.plan.total_q
    ref_out, ref_lse = ops.sparse_mla(dev.plan, dev.q, dev.kv, d.kv_format, d.D_v, idx, d.sm_scale,
                                      decode=True)
    out = torch.full((tq, 64, d.D_v), float("nan"), dtype=torch.bfloat16, device=dev.device)
    lse = torch.full((tq, 64), float("nan"), dtype=torch.float32, device=dev.device)
    ops.sparse_mla(dev.plan, dev.q, dev.kv, d.kv_format, d.D_v, idx, d.sm_scale, decode=True,
                   out=out, lse=lse, noalloc=True)
    torch.cuda.synchronize()
    as_bits = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    return as_bits(out), lse.cpu().numpy(), as_bits(ref_out), ref_lse.cpu().numpy()


def _case(label, batch, n_q, cached, seed, oracle_tokens):
    d = W.small_big_dims(batch=batch, n_q=n_q, cached=cached, seed=seed)
    x = W.generate(d)
    dev = Dev(x)
    idx, _ = dev.topk(with_scores=False)
    tq = int(d.total_q)
    splits = int(min(-(-256 // tq), -(-d.top_k // 32)))
    say(f"[case] {label}: total_q={tq} splits={splits} partials={tq * splits if splits > 1 else 0}")
    out, lse, ref_out, ref_lse = _both(dev, idx)
    assert np.array_equal(out, ref_out), f"{label}: outputs differ from smla_sparse_mla_decode"
    assert np.array_equal(lse.view(np.uint32), ref_lse.view(np.uint32)), f"{label}: lse differs"
    if oracle_tokens:
        tokens = np.asarray(oracle_tokens)
        ref, rl = oracle_mla(x, idx[tokens], tokens)
        assert_attn_close(out.reshape(tq, 64, -1)[tokens], ref,
                          lse.reshape(tq, 64)[tokens], rl, f"{label} vs oracle")


def test_noalloc_two_calls_second_smaller():
    _case("first call", batch=2, n_q=4, cached=3000, seed=0x5EED7100, oracle_tokens=(0, 7))
    _case("second call, fewer tokens", batch=1, n_q=3, cached=2200, seed=0x5EED7200,
          oracle_tokens=(2,))


def test_noalloc_most_partials():
    _case("255 tokens", batch=1, n_q=255, cached=2600, seed=0x5EED7300, oracle_tokens=(0, 254))
