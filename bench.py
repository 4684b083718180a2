#!/usr/bin/env python3
"""Throughput of one layer of the hot path (indexer scores -> exact top-k -> sparse MLA) on one
MI355X, in query tokens per second, with the dominant kernel's roofline fraction and the CPU
oracle timed on the host beside it.

A step is one pass of the whole path over one batch of seeded synthetic inputs resident in HBM:
smla_indexer_scores_topk then smla_sparse_mla_decode (decode workloads) or _prefill. The headline
workload is the largest: one 32,768-token prompt, fully causal. The decode batch (32 x 1 token
after 65,536), the 2,048-token chunk after 65,536 and the million-token MTP decode (4 x 4 after
1,048,576) run beside it as legs, each with its own roofline.

Steps are timed cold: before each step, outside its timed span, a 1 GiB buffer is written so that
neither the L2 caches nor the 256 MB last-level cache hold anything of the previous step, and then
512 MB of another buffer are read, so that the write's dirty lines go back to HBM before the step
rather than during it (the caches then hold clean data the step never touches); each step's span
is taken with HIP events on the stream the library launches on. Decode legs also
rotate among four seeded query sets, so consecutive steps select different rows. The warm figure
(steps back to back, no scrub) is reported beside the cold one.

    python bench.py [--steps K] [--warmup W] [--config 0..4] [--legs 1,2,4 | --legs none]
                    [--no-cpu-baseline]
    python bench.py --copy-calibration    # a plain 256 MiB device copy, for counter scaling

HBM traffic of a dominant kernel comes from rocprofv3 FETCH_SIZE / WRITE_SIZE counters taken
on `bench.py --config N --legs none` and scaled by what the counters read for the plain copy; the
summary under profiles/ records the hash of the kernel's sources, and the figure is reported only
while the sources still match.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "query-tokens/s per layer (indexer+top-k+sparse MLA); % of MFMA / HBM roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA
DECODE_CONFIGS = (1, 4)
HEADLINE_CONFIG = 3
SIDE_LEGS = (1, 2, 4)
SCRUB_BYTES = 1 << 30        # written between timed steps: > 4 x the 256 MB last-level cache
DRAIN_BYTES = 1 << 29        # then read: > 2 x that cache, so none of the write stays dirty
ROTATIONS = 4                # seeded query sets a decode leg cycles through
# file-name tags of the workloads in profiles/
WORKLOAD_TAGS = {0: "tiny_1x512", 1: "decode_32x65536", 2: "chunk_2048after65536",
                 3: "prefill_32768", 4: "decode_4x4after1048576"}
STAGES = ("indexer", "topk", "mla", "combine")
APPEND_BYTES_PER_ROW = 1152 + 656 + 128 + 128 + 8
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense FP8 MFMA


def workload_name(d):
    return (f"{d.batch} request(s) x {d.n_q} query token(s) after {d.cached} cached tokens; "
            f"{d.H} heads, {d.D_qk}/{d.D_v} dims, "
            f"{'656-byte FP8' if d.kv_format == 1 else 'bf16'} latent rows, "
            f"{d.H_I}x{d.D_I} int8 indexer, top-k {d.top_k}")


class HipEvents:
    """hipEvent_t handles via the HIP runtime (timing on the library's own launch stream)."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        rc = self.rt.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return e.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.rt.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def destroy(self, e):
        self.rt.hipEventDestroy(e)


# sources whose code decides a kernel's memory traffic
KERNEL_SOURCES = {
    "indexer_mfma_kernel": ("sparse_mla_attention_indexer_amd/csrc/indexer.hip",
                            "sparse_mla_attention_indexer_amd/csrc/smla_internal.h"),
    "indexer_mfma_kernel_multi": ("sparse_mla_attention_indexer_amd/csrc/indexer.hip",
                                  "sparse_mla_attention_indexer_amd/csrc/smla_internal.h"),
    "mla_fp8_kernel": ("sparse_mla_attention_indexer_amd/csrc/sparse_mla.hip",
                       "sparse_mla_attention_indexer_amd/csrc/smla_internal.h"),
}


def sources_sha256(kernel):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profiled_traffic(kernel, tag):
    """HBM bytes per launch from the committed counter summary, or None when there is none or the
    kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}.{tag}.pmc.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"^src_sha256:\s*([0-9a-f]{64})", text, re.M)
    val = re.search(r"^traffic_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not sha or not val or sha.group(1) != sources_sha256(kernel):
        return None
    return float(val.group(1))


def copy_calibration():
    """A plain device-to-device copy of 256 MiB, five times: the reference for counter scaling."""
    import torch

    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(7)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 5}), flush=True)


def append_measurement(dev, steps):
    """The cache-append step (smla_kv_append) beside the headline: the decode step's new rows and
    a bulk append of 65,536 rows (HBM-bound: 2,072 algorithmic bytes per row = 1,152 B bf16 latent
    in + 656 B FP8 row out + 128 B key in + 128 B key out + 8 B row index), timed with torch
    events on the current stream the library launches on. Not part of the headline metric."""
    import torch

    from sparse_mla_attention_indexer_amd import ops

    out = {}
    R = 1 << 17
    kv = torch.zeros((R, 656), dtype=torch.uint8, device=dev)
    k_idx = torch.zeros((R, 128), dtype=torch.int8, device=dev)
    g = torch.Generator(device="cpu").manual_seed(5)
    for label, n in (("decode_step", 32), ("bulk", 1 << 16)):
        lat = torch.randn((n, 576), generator=g).to(torch.bfloat16).to(dev)
        k_new = torch.randint(-128, 128, (n, 128), generator=g, dtype=torch.int8).to(dev)
        rows = torch.randperm(R, generator=g)[:n].to(torch.int64).to(dev)
        for _ in range(3):
            ops.kv_append(lat, rows, kv, k_new, k_idx)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(steps):
            ops.kv_append(lat, rows, kv, k_new, k_idx)
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / steps
        gbs = n * APPEND_BYTES_PER_ROW / (us * 1e-6) / 1e9
        out[label] = {"rows": n, "us": round(us, 2), "achieved": round(gbs, 1), "unit": "GB/s",
                      "frac": round(gbs / HBM_PEAK_GBS, 4)}
    out["bytes_per_row"] = APPEND_BYTES_PER_ROW
    return out


def stage_times(step, steps, before=None):
    """Average per-stage kernel time (ms) over `steps` calls of step(k), from HIP events the
    library records on its own launch stream around each stage; before(k) (the cache scrub) runs
    ahead of each step, outside every stage's span."""
    from sparse_mla_attention_indexer_amd import _lib

    hip = HipEvents()
    L = _lib.lib()
    ev = [[(hip.create(), hip.create()) for _ in STAGES] for _ in range(steps)]
    import torch

    torch.cuda.synchronize()
    for k in range(steps):
        if before is not None:
            before(k)
        begin = (ctypes.c_void_p * len(STAGES))(*[e[0] for e in ev[k]])
        end = (ctypes.c_void_p * len(STAGES))(*[e[1] for e in ev[k]])
        _lib.check("smla_set_stage_events", L.smla_set_stage_events(begin, end, len(STAGES)))
        step(k)
    torch.cuda.synchronize()
    L.smla_set_stage_events(None, None, 0)
    return ev, hip


def fp8_indexer_measurement(dev, d, plan, steps, warmup, attend):
    """The whole step with FP8 indexer keys (128 E4M3 values + an fp32 scale per key, 132 B) in
    place of the workload's int8 keys: FP8 indexer, top-k and the same sparse MLA (`attend(idx)`),
    so that the caches see what they see in the headline step (an indexer timed alone finds part
    of its keys still in the 256 MB last-level cache). Beside the headline, not part of it.
    Algorithmic bytes of the indexer: every visible key once (132 B) plus each token's E4M3 query
    (8,192 B) and fp32 weights (256 B); HBM-bound below the FP8 ridge of 5.0 PFLOP/s / 8 TB/s =
    625 FLOP/B, else against the FP8 peak."""
    import numpy as np
    import torch

    from sparse_mla_attention_indexer_amd import ops
    from sparse_mla_attention_indexer_amd import workload as W

    x8 = W.fp8_indexer_inputs(d)
    q8 = torch.from_numpy(x8.q).to(dev)
    k8 = torch.from_numpy(x8.k).to(dev)
    ks = torch.from_numpy(x8.k_scale).to(dev)
    w8 = torch.from_numpy(x8.w).to(dev)
    del x8
    idx = torch.empty((d.total_q, d.top_k), dtype=torch.int32, device=dev)
    ws = ops.topk_workspace(plan, d.H_I, d.D_I, d.top_k)

    def step(k=0):
        ops.indexer_topk_fp8(plan, q8, k8, ks, w8, d.top_k, with_scores=False, idx=idx, workspace=ws)
        attend(idx)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    step_ms = (time.perf_counter() - t0) * 1e3 / steps
    ev, hip = stage_times(step, steps)
    ms = {}
    for s, name in enumerate(STAGES[:2]):
        ms[name] = sum(hip.elapsed_ms(*ev[k][s]) for k in range(steps)) / steps
    for row in ev:
        for a, b in row:
            hip.destroy(a)
            hip.destroy(b)
    pairs = float(np.sum(plan.positions + 1))
    nbytes = d.total_rows * (d.D_I + 4) + d.total_q * d.H_I * (d.D_I + 4)
    flops = 2.0 * d.H_I * d.D_I * pairs
    sec = ms["indexer"] * 1e-3
    if flops / nbytes < FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        ach = nbytes / sec / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    else:
        ach = flops / sec / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s (fp8)", "frac": round(ach / FP8_PEAK_TFLOPS, 4)}
    roof["kernel_ms"] = round(ms["indexer"], 4)
    return {"key": "128 x e4m3 + fp32 scale (132 B)", "value": round(d.total_q / (step_ms * 1e-3), 1),
            "unit": "query-tokens/s", "ms_per_step": round(step_ms, 4),
            "stages_ms": {k: round(v, 4) for k, v in ms.items()},
            "roofline": roof, "algorithmic_bytes": nbytes, "flops": flops}


def dcp_measurement(dev, x, d, steps, warmup, n_sh=8):
    """The single-GPU DCP simulation on a decode batch: the KV cache of every request cut round
    robin into n_sh shards (shard l holds tokens l, l + n_sh, ...; a request's several query
    tokens get their local positions), each shard's indexer + top-k and sparse MLA at its real
    shape, and the exact merges (top-k merge with the shards' local lists, LSE merge).
    Reports one shard's step, the merges, and their sum: what one GPU of a DCP group would spend
    on compute per step (the all-gathers between GPUs are not modelled)."""
    import numpy as np
    import torch

    from sparse_mla_attention_indexer_amd import ops

    q = torch.from_numpy(x.q.view(np.int16)).view(torch.bfloat16).to(dev)
    q_idx = torch.from_numpy(x.q_idx).to(dev)
    w = torch.from_numpy(x.w).to(dev)
    row0 = np.concatenate([[0], np.cumsum(x.kv_len)[:-1]])
    shards = []
    for sh in range(n_sh):
        lens, pos = ops.dcp_shard_positions(x.n_q, x.kv_len, n_sh, sh)
        rows = np.concatenate([row0[b] + np.arange(sh, int(kl), n_sh) for b, kl in enumerate(x.kv_len)])
        plan = ops.BatchPlan(x.n_q, lens, dev, positions=pos)
        kv = torch.from_numpy(np.ascontiguousarray(x.kv[rows])).to(dev)
        k_idx = torch.from_numpy(np.ascontiguousarray(x.k_idx[rows])).to(dev)
        ws_t = ops.topk_workspace(plan, d.H_I, d.D_I, d.top_k)
        ws_m = ops.mla_workspace(plan, d.H, d.D_v, d.top_k, True)
        shards.append((plan, kv, k_idx, ws_t, ws_m))
    lists_i = torch.empty((n_sh, d.total_q, d.top_k), dtype=torch.int32, device=dev)
    lists_s = torch.empty_like(lists_i)
    local = torch.empty_like(lists_i)
    outs = torch.empty((n_sh, d.total_q, d.H, d.D_v), dtype=torch.bfloat16, device=dev)
    lses = torch.empty((n_sh, d.total_q, d.H), dtype=torch.float32, device=dev)
    idx = torch.empty((d.total_q, d.top_k), dtype=torch.int32, device=dev)
    sc = torch.empty_like(idx)
    out = torch.empty((d.total_q, d.H, d.D_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((d.total_q, d.H), dtype=torch.float32, device=dev)

    def shard_select(sh):
        plan, _, k_idx, ws_t, _ = shards[sh]
        ops.indexer_topk(plan, q_idx, k_idx, w, d.top_k, idx=lists_i[sh], score=lists_s[sh], workspace=ws_t)

    def shard_attend(sh):
        plan, kv, _, _, ws_m = shards[sh]
        ops.sparse_mla(plan, q, kv, d.kv_format, d.D_v, local[sh], d.sm_scale, decode=True,
                       out=outs[sh], lse=lses[sh], workspace=ws_m)

    def merge_select():
        ops.topk_merge(lists_i, lists_s, d.top_k, idx=idx, score=sc, local=local)

    def merge_attend():
        ops.lse_merge(outs, lses, out=out, lse=lse)

    def whole():
        for sh in range(n_sh):
            shard_select(sh)
        merge_select()
        for sh in range(n_sh):
            shard_attend(sh)
        merge_attend()

    def timed(fn):
        for _ in range(warmup):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    whole()  # every buffer holds a real selection before the parts are timed alone
    shard_ms = timed(lambda: (shard_select(0), shard_attend(0)))
    merge_ms = timed(lambda: (merge_select(), merge_attend()))
    whole_ms = timed(whole)
    return {"shards": n_sh, "shard_rows_per_request": int(np.ceil(int(x.kv_len[0]) / n_sh)),
            "shard_step_ms": round(shard_ms, 4), "merge_ms": round(merge_ms, 4),
            "per_gpu_compute_ms": round(shard_ms + merge_ms, 4),
            "one_gpu_all_shards_ms": round(whole_ms, 4),
            "note": "one shard's indexer + top-k + sparse MLA at its real shape, plus the merges; "
                    "the cross-GPU all-gathers are not modelled"}


def hot_resolve_measurement(dev, x, d, plan, q, select, attend, steps, warmup, resident=16384):
    """Hybrid offload on the decode batch: each request keeps its last `resident` rows on the GPU,
    the older ones only in pinned host memory, and a hot buffer of 2 x top_k slots in its released
    rows. Times the resolve cold (every offloaded selection a miss, copied from host memory) and
    warm (the same selection again: all hits), and the whole warm step (top-k, resolve, sparse
    MLA over the resolved rows)."""
    import numpy as np
    import torch

    from sparse_mla_attention_indexer_amd import ops
    from sparse_mla_attention_indexer_amd import workload as W

    B = d.batch
    rf = np.maximum(x.kv_len - resident, 0).astype(np.int32)
    n_slots = 2 * d.top_k
    if (rf < n_slots).any() or d.kv_format != W.KV_FP8_656:
        return None
    row0 = np.concatenate([[0], np.cumsum(x.kv_len)[:-1]]).astype(np.int64)
    host = torch.from_numpy(x.kv).pin_memory()
    kv = torch.from_numpy(x.kv).to(dev)
    for b in range(B):  # the device copies of offloaded rows are gone
        kv[int(row0[b]): int(row0[b]) + int(rf[b])].fill_(0xEE)
    t_rf = torch.from_numpy(rf).to(dev)
    t_hb = torch.zeros(B, dtype=torch.int32, device=dev)
    t_h0 = torch.from_numpy(row0).to(dev)
    tok = torch.full((B, n_slots), -1, dtype=torch.int32, device=dev)
    age = torch.full_like(tok, -1)
    idx = select()
    out_idx = torch.empty_like(idx)
    nc = torch.empty(B, dtype=torch.int32, device=dev)
    state = {"step": 0}

    def resolve():
        ops.hot_resolve(plan, idx, t_rf, t_hb, tok, age, state["step"], host, t_h0, kv,
                        idx_out=out_idx, n_copied=nc)
        state["step"] += 1

    def events(n, before, fn):
        tot = 0.0
        for _ in range(n):
            before()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            tot += a.elapsed_time(b)
        return tot / n

    def reset():
        tok.fill_(-1)
        age.fill_(-1)

    for _ in range(warmup):
        reset()
        resolve()
    cold_ms = events(steps, reset, resolve)
    copied = int(nc.sum().item())
    warm_ms = events(steps, lambda: None, resolve)
    assert int(nc.sum().item()) == 0

    def whole():
        select()
        resolve()
        attend(out_idx, kv)

    for _ in range(warmup):
        whole()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        whole()
    b.record()
    torch.cuda.synchronize()
    step_ms = a.elapsed_time(b) / steps
    return {"resident_rows_per_request": resident, "slots_per_request": n_slots,
            "cold_resolve_ms": round(cold_ms, 4), "cold_rows_copied": copied,
            "cold_host_read_GBps": round(copied * 656 / (cold_ms * 1e-3) / 1e9, 2),
            "warm_resolve_ms": round(warm_ms, 4), "warm_step_ms": round(step_ms, 4),
            "note": "rows below kv_len - resident only in pinned host memory; cold = every "
                    "offloaded selection a miss, warm = the same selection again"}


def algorithmic(d, positions):
    """Algorithmic work of one step (unique bytes; FLOPs/ops), per stage."""
    import numpy as np

    rows_sel = np.minimum(positions + 1, d.top_k)
    pairs = float(np.sum(positions + 1))
    n_rows = float(np.sum(rows_sel))
    qo = d.total_q * d.H * 2 * (d.D_qk + d.D_v)
    return {
        # every key read once per request, every query once, the weights
        "indexer_bytes": d.total_rows * d.D_I + d.total_q * d.H_I * d.D_I + 4 * d.H_I,
        "indexer_ops": 2.0 * d.H_I * d.D_I * pairs,
        # the pages' accounting per query: selected rows (656 B + 4 B index) + bf16 q and out;
        # every gathered row counts as read from HBM
        "mla_bytes": n_rows * (d.row_bytes + 4) + qo,
        # unique bytes: q and out, the indices, and every latent row of the batch once (prefill
        # re-reads its few MB of rows from cache)
        "mla_unique_bytes": qo + n_rows * 4 + d.total_rows * d.row_bytes,
        "mla_flops": n_rows * d.H * 2.0 * (d.D_qk + d.D_v),
    }


def rooflines(d, positions, stage_ms, decode, tag):
    """Roofline objects of the indexer and the sparse MLA, the dominant kernel's, and the step's
    roofline ceiling (indexer and MLA each at its bound, top-k counted as free)."""
    alg = algorithmic(d, positions)
    ridge_i8 = INT8_PEAK_TOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    ridge_bf16 = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    multi = d.n_q > 1
    idx_kernel = "indexer_mfma_kernel_multi" if multi else "indexer_mfma_kernel"
    idx_s = stage_ms["indexer"] * 1e-3
    if alg["indexer_ops"] / alg["indexer_bytes"] < ridge_i8:
        a = alg["indexer_bytes"] / idx_s / 1e9
        idx = {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
               "frac": round(a / HBM_PEAK_GBS, 4)}
        idx_floor = alg["indexer_bytes"] / (HBM_PEAK_GBS * 1e9)
    else:
        a = alg["indexer_ops"] / idx_s / 1e12
        idx = {"bound": "mfma", "achieved": round(a, 1), "peak": INT8_PEAK_TOPS, "unit": "TOP/s (int8)",
               "frac": round(a / INT8_PEAK_TOPS, 4)}
        idx_floor = alg["indexer_ops"] / (INT8_PEAK_TOPS * 1e12)
    idx.update({"traffic": profiled_traffic(idx_kernel, tag), "kernel": idx_kernel,
                "kernel_ms": round(stage_ms["indexer"], 4), "algorithmic_bytes": alg["indexer_bytes"],
                "ops": alg["indexer_ops"]})
    mla_ms = stage_ms["mla"] + stage_ms.get("combine", 0.0)
    mla_s = mla_ms * 1e-3
    if decode:  # no reuse between tokens: every gathered row from HBM (footnote accounting)
        nbytes = alg["mla_bytes"]
        a = nbytes / mla_s / 1e9
        mla = {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
               "frac": round(a / HBM_PEAK_GBS, 4), "accounting": "selected rows + q + out per token"}
        mla_floor = max(nbytes / (HBM_PEAK_GBS * 1e9), alg["mla_flops"] / (BF16_PEAK_TFLOPS * 1e12))
    else:
        nbytes = alg["mla_unique_bytes"]
        bound_hbm = alg["mla_flops"] / nbytes < ridge_bf16
        if bound_hbm:
            a = nbytes / mla_s / 1e9
            mla = {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                   "frac": round(a / HBM_PEAK_GBS, 4)}
        else:
            a = alg["mla_flops"] / mla_s / 1e12
            mla = {"bound": "mfma", "achieved": round(a, 1), "peak": BF16_PEAK_TFLOPS,
                   "unit": "TFLOP/s (bf16)", "frac": round(a / BF16_PEAK_TFLOPS, 4)}
        mla["accounting"] = "unique bytes: q + out + indices + every latent row once"
        mla["footnote_hbm_GBps"] = round(alg["mla_bytes"] / mla_s / 1e9, 1)
        mla_floor = max(nbytes / (HBM_PEAK_GBS * 1e9), alg["mla_flops"] / (BF16_PEAK_TFLOPS * 1e12))
    mla.update({"traffic": profiled_traffic("mla_fp8_kernel", tag) if not decode or "combine" not in stage_ms
                else None,
                "kernel": "mla_fp8_kernel" + (" + mla_combine_kernel" if "combine" in stage_ms else ""),
                "kernel_ms": round(mla_ms, 4), "algorithmic_bytes": nbytes, "flops": alg["mla_flops"]})
    dominant = idx if stage_ms["indexer"] >= mla_ms else mla
    return idx, mla, dict(dominant), (idx_floor + mla_floor) * 1e3


def cpu_baseline(x, d, sample_tokens):
    import numpy as np

    import oracle

    threads = oracle.default_threads()
    tokens = np.asarray(sample_tokens, np.int64)
    # whole passes over the sample until about a second of wall time (tens of CPU-seconds)
    reps, t0 = 0, time.perf_counter()
    while True:
        idx, _ = oracle.indexer_topk_batch(x.n_q, x.kv_len, x.q_idx, x.k_idx, x.w, d.top_k, tokens,
                                           nthreads=threads)
        full = np.full((d.total_q, d.top_k), -1, np.int32)
        full[tokens] = idx
        oracle.sparse_mla_batch(x.n_q, x.kv_len, x.q, x.kv, d.kv_format, d.D_v, full, d.sm_scale,
                                tokens, nthreads=threads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 1.0 or reps >= 50:
            break
    return {"value": reps * tokens.size / dt, "unit": "query-tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{reps} pass(es) over {tokens.size} of {d.total_q} query tokens of the same "
                      f"workload (indexer + top-k + fp64 attention), {dt:.2f} s wall on "
                      f"{threads} threads"}


def measured_peaks(dev):
    """What this GPU reaches on plain library work, for context beside the nominal peaks: a 1 GiB
    device copy (read + write bytes / time) and square bf16 and int8 GEMMs of 8,192 (hipBLASLt)."""
    import torch

    out = {}
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(3)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(10):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    out["hbm_copy_GBps"] = round(2 * n * 10 / (a.elapsed_time(b) * 1e-3) / 1e9, 1)
    del src, dst
    m = 8192
    x = torch.randn((m, m), device=dev).to(torch.bfloat16)
    y = torch.randn((m, m), device=dev).to(torch.bfloat16)
    for _ in range(3):
        torch.matmul(x, y)
    torch.cuda.synchronize()
    a.record()
    for _ in range(10):
        torch.matmul(x, y)
    b.record()
    torch.cuda.synchronize()
    out["bf16_gemm_TFLOPs"] = round(2.0 * m ** 3 * 10 / (a.elapsed_time(b) * 1e-3) / 1e12, 1)
    del x, y
    try:
        xi = torch.randint(-8, 8, (m, m), dtype=torch.int8, device=dev)
        yi = torch.randint(-8, 8, (m, m), dtype=torch.int8, device=dev)
        for _ in range(3):
            torch._int_mm(xi, yi)
        torch.cuda.synchronize()
        a.record()
        for _ in range(10):
            torch._int_mm(xi, yi)
        b.record()
        torch.cuda.synchronize()
        out["int8_gemm_TOPs"] = round(2.0 * m ** 3 * 10 / (a.elapsed_time(b) * 1e-3) / 1e12, 1)
        del xi, yi
    except Exception as e:  # int8 GEMM may be missing from this torch build
        out["int8_gemm_TOPs"] = None
        out["int8_gemm_note"] = f"torch._int_mm unavailable: {type(e).__name__}"
    torch.cuda.empty_cache()
    out["note"] = "library kernels (torch copy, hipBLASLt GEMMs); frac is taken against the nominal peaks"
    return out


def run_metadata():
    import platform
    import subprocess

    import torch

    meta = {"python": platform.python_version(), "torch": torch.__version__,
            "hip": getattr(torch.version, "hip", None)}
    try:
        meta["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        meta["rocm"] = None
    cpu = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    meta["cpu_model"] = cpu
    meta["host_cpus"] = os.cpu_count()
    meta["host_cpus_allowed"] = len(os.sched_getaffinity(0))
    p = torch.cuda.get_device_properties(0)
    meta["gpu"] = {"name": torch.cuda.get_device_name(0), "arch": getattr(p, "gcnArchName", None),
                   "cus": p.multi_processor_count, "memory_GiB": round(p.total_memory / 2 ** 30, 1)}
    try:
        rev = subprocess.run(["git", "rev-parse", "HEAD"], cwd=ROOT, capture_output=True, text=True,
                             timeout=10)
        meta["git_rev"] = rev.stdout.strip() if rev.returncode == 0 else None
    except (OSError, subprocess.SubprocessError):
        meta["git_rev"] = None
    h = hashlib.sha256()
    for sub in ("include", "sparse_mla_attention_indexer_amd/csrc"):
        base = os.path.join(ROOT, sub)
        for name in sorted(os.listdir(base)):
            if name.endswith((".h", ".hip", ".cpp")):
                with open(os.path.join(base, name), "rb") as f:
                    h.update(name.encode() + b"\0" + f.read())
    meta["src_sha256"] = h.hexdigest()
    return meta


class Leg:
    """One workload on the GPU: inputs, buffers and the step (indexer + top-k, then sparse MLA)."""

    def __init__(self, config, dev, log):
        import numpy as np
        import torch

        from sparse_mla_attention_indexer_amd import ops
        from sparse_mla_attention_indexer_amd import workload as W

        self.config, self.dev = config, dev
        d = self.d = W.config_dims(config)
        self.decode = config in DECODE_CONFIGS
        log(f"generating workload {config} ({W.CONFIG_NAMES[config]})")
        x = self.x = W.generate(d)
        self.plan = ops.BatchPlan(x.n_q, x.kv_len, dev)
        as_bf16 = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        if d.kv_format == W.KV_FP8_656:
            self.kv = torch.from_numpy(x.kv).to(dev)
        else:
            self.kv = torch.from_numpy(x.kv.view(np.int16).reshape(d.total_rows, d.D_qk)).view(
                torch.bfloat16).to(dev)
        self.k_idx = torch.from_numpy(x.k_idx).to(dev)
        self.w = torch.from_numpy(x.w).to(dev)
        # query sets: the workload's own, and for decode legs three more seeded ones, so that
        # consecutive steps select different rows
        self.q = [as_bf16(x.q)]
        self.q_idx = [torch.from_numpy(x.q_idx).to(dev)]
        if self.decode:
            for r in range(1, ROTATIONS):
                xr = W.generate(d, seed=int(d.seed) + 0x1000 * r, parts=("q", "q_idx"))
                self.q.append(as_bf16(xr.q))
                self.q_idx.append(torch.from_numpy(xr.q_idx).to(dev))
        self.idx = torch.empty((d.total_q, d.top_k), dtype=torch.int32, device=dev)
        self.out = torch.empty((d.total_q, d.H, d.D_v), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((d.total_q, d.H), dtype=torch.float32, device=dev)
        self.ws_topk = ops.topk_workspace(self.plan, d.H_I, d.D_I, d.top_k)
        self.ws_mla = ops.mla_workspace(self.plan, d.H, d.D_v, d.top_k, self.decode)
        torch.cuda.synchronize()

    def step(self, k=0):
        from sparse_mla_attention_indexer_amd import ops

        d, r = self.d, k % len(self.q)
        ops.indexer_topk(self.plan, self.q_idx[r], self.k_idx, self.w, d.top_k, with_scores=False,
                         idx=self.idx, workspace=self.ws_topk)
        ops.sparse_mla(self.plan, self.q[r], self.kv, d.kv_format, d.D_v, self.idx, d.sm_scale,
                       decode=self.decode, out=self.out, lse=self.lse, workspace=self.ws_mla)

    def attend(self, sel, kv=None, k=0):
        from sparse_mla_attention_indexer_amd import ops

        d = self.d
        ops.sparse_mla(self.plan, self.q[k % len(self.q)], self.kv if kv is None else kv, d.kv_format,
                       d.D_v, sel, d.sm_scale, decode=self.decode, out=self.out, lse=self.lse,
                       workspace=self.ws_mla)


def time_leg(leg, steps, warmup, scrub, log):
    """scrub: (write buffer, drain buffer); see the module docstring."""
    """Cold per-step spans (the reported figures), cold per-stage kernel times, and the warm rate
    of steps back to back."""
    import numpy as np
    import torch

    for k in range(warmup):
        leg.step(k)
    torch.cuda.synchronize()

    wbuf, drain = scrub

    def cold(k):
        wbuf.fill_(k & 0x7F)
        drain.max()  # a read of other data: the write's dirty lines leave the caches first

    log(f"timing {steps} cold steps")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        cold(k)
        ev[k][0].record()
        leg.step(k)
        ev[k][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    spans = np.array([a.elapsed_time(b) for a, b in ev])

    # per-stage kernel time: as many cold steps again with HIP events the library records on its
    # own launch stream around each stage (kept out of the spans above)
    sev, hip = stage_times(leg.step, steps, before=cold)
    stage_ms = {}
    has_combine = leg.decode and leg.ws_mla.numel() > 256
    for s, name in enumerate(STAGES):
        if name == "combine" and not has_combine:
            continue
        stage_ms[name] = sum(hip.elapsed_ms(*sev[k][s]) for k in range(steps)) / steps
    for row in sev:
        for a, b in row:
            hip.destroy(a)
            hip.destroy(b)

    log(f"timing {steps} warm steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        leg.step(k)
    torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - t0) * 1e3 / steps
    return {"ms": float(spans.mean()), "median_ms": float(np.median(spans)), "min_ms": float(spans.min()),
            "wall_ms_incl_scrub": wall * 1e3 / steps, "warm_ms": warm_ms, "stage_ms": stage_ms}


def leg_result(leg, t, steps, warmup):
    d = leg.d
    tag = WORKLOAD_TAGS.get(leg.config, "")
    idx_roof, mla_roof, dominant, ceiling_ms = rooflines(d, leg.plan.positions, t["stage_ms"],
                                                         leg.decode, tag)
    return {
        "config": {"workload": workload_name(d), "config_id": leg.config, "batch": d.batch,
                   "query_tokens": d.total_q, "cached_tokens": d.cached, "heads": d.H,
                   "top_k": d.top_k, "decode_entry": leg.decode, "seed": hex(int(d.seed)),
                   "query_sets": len(leg.q)},
        "value": round(d.total_q / (t["ms"] * 1e-3), 1), "unit": "query-tokens/s",
        "steps": steps, "warmup": warmup,
        "ms_per_step": round(t["ms"], 4), "median_ms": round(t["median_ms"], 4),
        "min_ms": round(t["min_ms"], 4),
        "warm": {"ms_per_step": round(t["warm_ms"], 4),
                 "value": round(d.total_q / (t["warm_ms"] * 1e-3), 1)},
        "stages_ms": {k: round(v, 4) for k, v in t["stage_ms"].items()},
        "roofline": dominant,
        "indexer_roofline": idx_roof,
        "mla_roofline": mla_roof,
        "step_roofline": {"ceiling_ms": round(ceiling_ms, 4),
                          "frac": round(ceiling_ms / t["ms"], 4),
                          "note": "indexer and sparse MLA each at its bound, top-k free"},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=HEADLINE_CONFIG,
                    help="headline workload 0..4 (default 3: the 32,768-token prefill)")
    ap.add_argument("--legs", default=",".join(map(str, SIDE_LEGS)),
                    help="comma-separated side workloads, or 'none'")
    ap.add_argument("--leg-steps", type=int, default=50,
                    help="timed steps of each side workload (decode steps take ~0.1-0.25 ms)")
    ap.add_argument("--leg-warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the cache-append, DCP, hybrid-offload and FP8-key measurements")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 256 MiB device copy (counter scaling reference)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (no collectives); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from sparse_mla_attention_indexer_amd import _lib, ops  # noqa: F401  (loads the library)
    from sparse_mla_attention_indexer_amd import workload as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    _lib.lib()
    dev = torch.device("cuda:0")
    log = lambda m: print(f"[bench] {m}", file=sys.stderr, flush=True)
    legs = [] if args.legs.strip() in ("", "none") else [int(c) for c in args.legs.split(",")]
    legs = [c for c in legs if c != args.config]

    meta = run_metadata()
    log("measuring copy and GEMM rates")
    meta["measured_peaks"] = measured_peaks(dev)
    scrub = (torch.empty(SCRUB_BYTES, dtype=torch.uint8, device=dev),
             torch.zeros(DRAIN_BYTES // 4, dtype=torch.int32, device=dev))

    leg = Leg(args.config, dev, log)
    d = leg.d
    t = time_leg(leg, args.steps, args.warmup, scrub, log)
    head = leg_result(leg, t, args.steps, args.warmup)
    result = {
        "metric": METRIC, "value": head["value"], "unit": "query-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8+bf16",
        "dtypes": {"indexer": "int8 x int8 -> int32 (MFMA)",
                   "kv": "fp8 e4m3 codes + fp32 block scales per 128 dims",
                   "attention": "bf16 MFMA of bf16 q with exact e4m3 codes, fp32 block scales and "
                                "softmax; PV in fp16 (bf16 fallback), fp32 accumulate"},
        "data": "synthetic",
        "config": head["config"],
        "timing": "cold: 1 GiB written, then 512 MB of other data read, before each step, outside its HIP-event span"
                  + ("; 4 rotating query sets" if leg.decode else ""),
        "median_ms": head["median_ms"], "min_ms": head["min_ms"], "warm": head["warm"],
        "stages_ms": head["stages_ms"],
        "roofline": head["roofline"],
        "indexer_roofline": head["indexer_roofline"],
        "mla_roofline": head["mla_roofline"],
        "step_roofline": head["step_roofline"],
        "meta": meta,
    }
    extras = not args.no_extras and d.kv_format == W.KV_FP8_656
    if extras and d.H_I == 64 and d.D_I == 128:
        log("FP8-key indexer")
        result["indexer_fp8"] = fp8_indexer_measurement(dev, d, leg.plan, min(args.steps, 10), 2,
                                                        leg.attend)
    if not args.no_cpu_baseline:
        sample = np.arange(d.total_q) if d.total_q <= 32 else np.linspace(0, d.total_q - 1, 32).astype(np.int64)
        log(f"oracle on {sample.size} tokens")
        result["cpu_baseline"] = cpu_baseline(leg.x, d, sample)
    del leg
    torch.cuda.empty_cache()

    result["legs"] = {}
    for c in legs:
        lg = Leg(c, dev, log)
        tl = time_leg(lg, args.leg_steps, args.leg_warmup, scrub, log)
        r = leg_result(lg, tl, args.leg_steps, args.leg_warmup)
        if extras and lg.decode and lg.d.kv_format == W.KV_FP8_656:
            log("DCP simulation")
            r["dcp_sim"] = dcp_measurement(dev, lg.x, lg.d, args.leg_steps, args.leg_warmup)
        if extras and lg.decode and (lg.x.n_q == 1).all() and lg.d.kv_format == W.KV_FP8_656:
            log("hybrid offload resolve")

            def select():
                ops.indexer_topk(lg.plan, lg.q_idx[0], lg.k_idx, lg.w, lg.d.top_k, with_scores=False,
                                 idx=lg.idx, workspace=lg.ws_topk)
                return lg.idx

            hot = hot_resolve_measurement(dev, lg.x, lg.d, lg.plan, lg.q[0], select,
                                          lambda sel, kv_h: lg.attend(sel, kv_h), args.leg_steps,
                                          args.leg_warmup)
            if hot is not None:
                r["hot_resolve"] = hot
        result["legs"][WORKLOAD_TAGS[c]] = r
        del lg
        torch.cuda.empty_cache()
    if extras:
        result["append"] = append_measurement(dev, args.leg_steps)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
