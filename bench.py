#!/usr/bin/env python3
"""Throughput of one layer of the hot path (indexer scores -> exact top-k -> sparse MLA) on one
MI355X, in query tokens per second, with the dominant kernel's roofline fraction and the CPU
oracle timed on the host beside it.

A step is one pass of the whole path over one batch of seeded synthetic inputs resident in HBM:
smla_indexer_scores_topk then smla_sparse_mla_decode (decode workloads) or _prefill. The default
workload is the decode batch: 32 requests x 1 query token over 65,536 cached tokens each.

    python bench.py [--steps K] [--warmup W] [--config 0..4] [--no-cpu-baseline]
    python bench.py --copy-calibration    # a plain 256 MiB device copy, for counter scaling

HBM traffic of the dominant kernel comes from rocprofv3 FETCH_SIZE / WRITE_SIZE counters taken
on this same command and scaled by what the counters read for the plain copy; the summary under
profiles/ records the hash of the kernel's sources, and the figure is reported only while the
sources still match.
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


def stage_times(step, steps):
    """Average per-stage kernel time (ms) over `steps` calls of step(), from HIP events the library
    records on its own launch stream around each stage."""
    from sparse_mla_attention_indexer_amd import _lib

    hip = HipEvents()
    L = _lib.lib()
    ev = [[(hip.create(), hip.create()) for _ in STAGES] for _ in range(steps)]
    import torch

    torch.cuda.synchronize()
    for k in range(steps):
        begin = (ctypes.c_void_p * len(STAGES))(*[e[0] for e in ev[k]])
        end = (ctypes.c_void_p * len(STAGES))(*[e[1] for e in ev[k]])
        _lib.check("smla_set_stage_events", L.smla_set_stage_events(begin, end, len(STAGES)))
        step()
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

    def step():
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
    """The single-GPU DCP simulation on the decode batch: the KV cache of every request cut round
    robin into n_sh shards (shard l holds tokens l, l + n_sh, ...), each shard's indexer + top-k and
    sparse MLA at its real shape, and the exact merges (top-k merge, local indices, LSE merge).
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
        lens, rows = [], []
        for b, kl in enumerate(x.kv_len):
            g = np.arange(sh, int(kl), n_sh)
            lens.append(g.size)
            rows.append(row0[b] + g)
        rows = np.concatenate(rows)
        plan = ops.BatchPlan(np.ones(d.batch, np.int32), np.array(lens, np.int64), dev)
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
        ops.topk_merge(lists_i, lists_s, d.top_k, idx=idx, score=sc)
        ops.dcp_local_indices(idx, n_sh, out=local)

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
    return {
        # every key read once per request, every query once, the weights
        "indexer_bytes": d.total_rows * d.D_I + d.total_q * d.H_I * d.D_I + 4 * d.H_I,
        "indexer_ops": 2.0 * d.H_I * d.D_I * pairs,
        # the pages' accounting per query: selected rows (656 B + 4 B index) + bf16 q and out
        "mla_bytes": float(np.sum(rows_sel)) * (d.row_bytes + 4) + d.total_q * d.H * 2 * (d.D_qk + d.D_v),
        "mla_flops": float(np.sum(rows_sel)) * d.H * 2.0 * (d.D_qk + d.D_v),
    }


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


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=1, help="workload 0..4 (default 1: decode)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 256 MiB device copy (counter scaling reference)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (no collectives); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from sparse_mla_attention_indexer_amd import _lib, ops
    from sparse_mla_attention_indexer_amd import workload as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    dev = torch.device("cuda:0")
    d = W.config_dims(args.config)
    decode = args.config in DECODE_CONFIGS
    print(f"[bench] generating workload {args.config} ({W.CONFIG_NAMES[args.config]})", file=sys.stderr, flush=True)
    x = W.generate(d)
    plan = ops.BatchPlan(x.n_q, x.kv_len, dev)
    q = torch.from_numpy(x.q.view(np.int16)).view(torch.bfloat16).to(dev)
    if d.kv_format == W.KV_FP8_656:
        kv = torch.from_numpy(x.kv).to(dev)
    else:
        kv = torch.from_numpy(x.kv.view(np.int16).reshape(d.total_rows, d.D_qk)).view(torch.bfloat16).to(dev)
    q_idx = torch.from_numpy(x.q_idx).to(dev)
    k_idx = torch.from_numpy(x.k_idx).to(dev)
    w = torch.from_numpy(x.w).to(dev)
    idx = torch.empty((d.total_q, d.top_k), dtype=torch.int32, device=dev)
    out = torch.empty((d.total_q, d.H, d.D_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((d.total_q, d.H), dtype=torch.float32, device=dev)
    ws_topk = ops.topk_workspace(plan, d.H_I, d.D_I, d.top_k)
    ws_mla = ops.mla_workspace(plan, d.H, d.D_v, d.top_k, decode)
    torch.cuda.synchronize()

    def step():
        ops.indexer_topk(plan, q_idx, k_idx, w, d.top_k, with_scores=False, idx=idx,
                         workspace=ws_topk)
        ops.sparse_mla(plan, q, kv, d.kv_format, d.D_v, idx, d.sm_scale, decode=decode, out=out,
                       lse=lse, workspace=ws_mla)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # headline: K steps back to back, nothing but the library's launches in the timed region
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    # per-stage kernel time: K more steps with HIP events the library records on its own launch
    # stream around each stage (event markers cost a few microseconds each, so they stay out of
    # the headline region)
    ev, hip = stage_times(step, args.steps)

    stage_ms = {}
    for s, name in enumerate(STAGES):
        if name == "combine" and not (decode and ws_mla.numel() > 256):
            continue
        stage_ms[name] = sum(hip.elapsed_ms(*ev[k][s]) for k in range(args.steps)) / args.steps
    for row in ev:
        for a, b in row:
            hip.destroy(a)
            hip.destroy(b)

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = d.total_q / (ms_per_step * 1e-3)
    alg = algorithmic(d, plan.positions)
    idx_gbs = alg["indexer_bytes"] / (stage_ms["indexer"] * 1e-3) / 1e9
    idx_tops = alg["indexer_ops"] / (stage_ms["indexer"] * 1e-3) / 1e12
    mla_ms = stage_ms["mla"] + stage_ms.get("combine", 0.0)
    mla_gbs = alg["mla_bytes"] / (mla_ms * 1e-3) / 1e9
    mla_tflops = alg["mla_flops"] / (mla_ms * 1e-3) / 1e12
    # the indexer dominates the step; it is HBM-bound when its ops per key byte fall below the
    # int8 ridge (5.0 POP/s / 8 TB/s = 625)
    idx_hbm = alg["indexer_ops"] / alg["indexer_bytes"] < INT8_PEAK_TOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    traffic = profiled_traffic("indexer_mfma_kernel", WORKLOAD_TAGS.get(args.config, ""))
    if idx_hbm:
        roof = {"bound": "hbm", "achieved": round(idx_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(idx_gbs / HBM_PEAK_GBS, 4),
                "traffic": None if traffic is None else round(traffic),
                "kernel": "indexer_mfma_kernel", "kernel_ms": round(stage_ms["indexer"], 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(idx_tops, 1), "peak": INT8_PEAK_TOPS,
                "unit": "TOP/s (int8)", "frac": round(idx_tops / INT8_PEAK_TOPS, 4),
                "traffic": None if traffic is None else round(traffic),
                "kernel": "indexer_mfma_kernel", "kernel_ms": round(stage_ms["indexer"], 4)}
    mla_hbm = alg["mla_flops"] / alg["mla_bytes"] < BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    mla_roof = ({"bound": "hbm", "achieved": round(mla_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": round(mla_gbs / HBM_PEAK_GBS, 4)} if mla_hbm else
                {"bound": "mfma", "achieved": round(mla_tflops, 1), "peak": BF16_PEAK_TFLOPS,
                 "unit": "TFLOP/s", "frac": round(mla_tflops / BF16_PEAK_TFLOPS, 4)})
    mla_roof["kernel_ms"] = round(mla_ms, 4)

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "query-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8+fp16",
        "dtypes": {"indexer": "int8 x int8 -> int32", "kv": "fp8 e4m3 + fp32 block scales",
                   "attention": "fp16 MFMA on dequantised rows, fp32 accumulate and softmax"},
        "data": "synthetic",
        "config": {"workload": workload_name(d), "config_id": args.config, "batch": d.batch,
                   "query_tokens": d.total_q, "cached_tokens": d.cached, "heads": d.H,
                   "top_k": d.top_k, "decode_entry": decode},
        "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "roofline": roof,
        "mla_roofline": mla_roof,
    }
    if d.kv_format == W.KV_FP8_656:
        result["append"] = append_measurement(dev, args.steps)
    if decode and (x.n_q == 1).all() and d.kv_format == W.KV_FP8_656:
        print("[bench] DCP simulation", file=sys.stderr, flush=True)
        result["dcp_sim"] = dcp_measurement(dev, x, d, args.steps, args.warmup)
    if decode and (x.n_q == 1).all() and d.kv_format == W.KV_FP8_656:
        print("[bench] hybrid offload resolve", file=sys.stderr, flush=True)

        def select():
            ops.indexer_topk(plan, q_idx, k_idx, w, d.top_k, with_scores=False, idx=idx,
                             workspace=ws_topk)
            return idx

        hot = hot_resolve_measurement(
            dev, x, d, plan, q, select,
            lambda sel, kv_h: ops.sparse_mla(plan, q, kv_h, d.kv_format, d.D_v, sel, d.sm_scale,
                                             decode=True, out=out, lse=lse, workspace=ws_mla),
            args.steps, args.warmup)
        if hot is not None:
            result["hot_resolve"] = hot
    if d.H_I == 64 and d.D_I == 128:
        print("[bench] FP8-key indexer", file=sys.stderr, flush=True)
        result["indexer_fp8"] = fp8_indexer_measurement(
            dev, d, plan, args.steps, args.warmup,
            lambda sel: ops.sparse_mla(plan, q, kv, d.kv_format, d.D_v, sel, d.sm_scale, decode=decode,
                                       out=out, lse=lse, workspace=ws_mla))
    if not args.no_cpu_baseline:
        sample = np.arange(d.total_q) if d.total_q <= 32 else np.linspace(0, d.total_q - 1, 32).astype(np.int64)
        print(f"[bench] oracle on {sample.size} tokens", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(x, d, sample)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
