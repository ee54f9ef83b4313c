"""Decode-step benchmark for paged KV-cache attention on one MI355X.

A step is one pass of the whole hot path over one synthetic batch: the
slot-mapped cache write of every sequence's new token (INT8 quantize-on-write
for the INT8 cache), then split-context paged decode attention, then (for
sequences cut into more than one partition) the merge of the partial softmax
results in a second launch.  Inputs are resident in HBM before timing starts.

Prints ONE JSON line.  `value` is algorithmic bytes moved per step / wall time
per step (GB/s); `roofline` reports the dominant kernel (paged decode) from HIP
events on the stream it runs on; `cpu_baseline` times the CPU oracle on a
bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 100] [--warmup 20] [--config llama7b]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
METRIC = "decode attention KV GB/s and % of HBM peak; KV-tokens/s at LLaMA-7B shape"
WORKLOAD_NAMES = {
    "tiny": "tiny-fp32-mha-decode",
    "llama7b": "llama7b-mha-fp16-paged-decode",
    "gqa": "gqa-32q8kv-bf16-paged-decode",
    "long": "long-32k-fp16-split-decode",
    "int8": "llama7b-mha-int8kv-paged-decode",
    "fp8": "llama7b-mha-fp8e4m3kv-paged-decode",
    "int4": "llama7b-mha-int4kv-paged-decode",
    "window": "llama7b-mha-fp16-sliding-window-4096-decode",
    "verify": "llama7b-mha-fp16-speculative-verify-8-queries",
    "prefill": "llama7b-mha-fp16-chunked-prefill-512",
    "sampling": "llama7b-parallel-sampling-shared-prefix-decode",
    "int8-write": "llama7b-int8kv-cache-write-64-new-tokens",
    "gqa8": "gqa-64q8kv-bf16-paged-decode",
    "gqa8-int8": "gqa-64q8kv-int8kv-paged-decode",
    "tp8": "llama7b-mha-fp16-decode-one-gpu-share-of-8-by-kv-head",
    "dp8": "llama7b-mha-fp16-decode-one-gpu-share-of-8-by-sequence",
    "cp8": "long-32k-fp16-decode-one-gpu-share-of-8-by-context",
}
# the device code of a kernel: its source file, the device helpers and the
# argument struct it is launched with (host-side edits elsewhere leave the
# hash, and so the validity of recorded counters, unchanged)
KERNEL_SOURCES = ["paged_decode.hip", "pkv_device.h", "struct DecodeArgs"]
MULTI_SOURCES = ["paged_multi.hip", "pkv_device.h", "struct MultiArgs"]


def kernel_sha(sources=None) -> str:
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_264_amd", "csrc")
    for f in sources or KERNEL_SOURCES:
        if f.startswith("struct "):
            with open(os.path.join(csrc, "pkv_internal.h")) as fh:
                m = re.search(re.escape(f) + r" \{.*?\n\};", fh.read(), re.S)
            h.update(m.group(0).encode())
        else:
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", default="llama7b", choices=sorted(WORKLOAD_NAMES))
    p.add_argument("--partition-size", type=int, default=None)
    p.add_argument("--step", choices=["fused", "separate"], default="fused",
                   help="fused: one pkv_paged_attn_decode_append call per step; separate: "
                        "pkv_kv_cache_write, then the two decode phases")
    p.add_argument("--seed", type=int, default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="target CPU time of the oracle baseline sample")
    p.add_argument("--sampling-decode", choices=["shared", "plain"], default="shared",
                   help="sampling workload: shared = pkv_paged_attn_decode_shared_prefix (each "
                        "prompt's shared blocks read once per group), plain = the fused decode "
                        "of every sequence over its whole context")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain 1 GiB device copy (for HBM counter calibration)")
    return p.parse_args()


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 5}))


def traffic_for(key: str, alg_bytes: int, sources=None):
    """HBM bytes per decode launch from committed rocprofv3 counter runs, if
    they were taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None, None
    with open(path) as f:
        data = json.load(f)
    rec = data.get(key)
    if not rec or rec.get("kernel_sha") != kernel_sha(sources):
        return None, None
    t = float(rec["fetch_bytes_per_launch"]) + float(rec["write_bytes_per_launch"])
    return t, t / alg_bytes


def timed_steps(step, steps, stream):
    """The contract's timed region: `steps` steps bracketed by
    torch.cuda.synchronize() on both sides, wall clock around it, plus two
    HIP events on the launch stream at its ends (nothing is recorded between
    the steps, so the region holds the launches alone).  Returns (wall ms per
    step, GPU ms per step)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) * 1e3 / steps, e0.elapsed_time(e1) / steps


def per_launch_events(step, steps):
    """A pass after the timed region with HIP events around the measured
    launch of every step (its distribution; recording events between launches
    adds a few microseconds to each step, so this pass is not the timed one).
    `step(ev0, ev1)` records ev0 / ev1 around the launch.  Returns ms list."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in evs:
        step(a, b)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the decode path is built and measured on a "
              f"single MI355X (got --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.config == "sampling":
        bench_sampling(args)
        return
    if args.config == "int8-write":
        bench_cache_write(args)
        return
    if "q_len" in __import__("workloads").CONFIGS.get(args.config, {}):
        bench_multi(args)
        return

    import numpy as np
    import torch

    import paged_kv_cache_264_amd as pkv
    import workloads as W

    torch.cuda.set_device(0)
    cfg = W.CONFIGS[args.config]
    batch = W.make_batch(args.config, device="cuda", seed=args.seed, poison=False)
    if batch.k_src is not None and batch.k_src.shape[0] > 0:
        pkv.kv_cache_write(batch.k_src, batch.v_src, batch.k_cache, batch.v_cache,
                           batch.slot_src, batch.k_scale, batch.v_scale)
    P = args.partition_size if args.partition_size is not None else cfg.get("partition_size", 0)
    mbs = batch.block_tables.shape[1]
    mbs_eff = min(mbs, int(cfg.get("window", 0)) // W.BLOCK_SIZE + 2) if cfg.get("window") \
        else mbs
    P_eff = P or pkv.default_partition_size(batch.B, batch.Hq, batch.Hkv, mbs_eff,
                                            batch.k_cache.dtype)
    out = torch.empty_like(batch.q)
    NP = pkv.num_partitions(mbs_eff, P_eff)
    partials = (torch.empty((batch.B, batch.Hq, NP), dtype=torch.float32, device="cuda"),
                torch.empty((batch.B, batch.Hq, NP), dtype=torch.float32, device="cuda"),
                torch.empty((batch.B, batch.Hq, NP, batch.D), dtype=torch.float32, device="cuda"))
    lens = batch.layout.context_lens
    window = int(cfg.get("window", 0))
    block_tables = batch.block_tables
    if window:
        # tokens a sequence attends to; blocks wholly before the window are
        # released (-1), as a block manager would have done
        bt = batch.layout.block_tables.copy()
        for b, n in enumerate(lens):
            if n > window:
                bt[b, :(int(n) - window) // W.BLOCK_SIZE] = -1
        block_tables = torch.from_numpy(bt).cuda()
        lens = np.minimum(lens, window)
    e_kv = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1, "f8": 1, "u4": 0.5}[cfg["cache"]]
    e_q = {"f32": 4, "f16": 2, "bf16": 2}[cfg["dtype"]]
    int8 = cfg["cache"] in W.SCALED     # quantized codes + per-row scale (or min, range)
    meta = {"i8": 4, "f8": 4, "u4": 8}.get(cfg["cache"], 0)
    dec_bytes = W.algorithmic_bytes(lens, batch.Hq, batch.Hkv, batch.D, e_kv, e_q, int8, meta)
    n_new = int((batch.slot_new >= 0).sum())
    # the new rows written into the cache (codes + scales for quantized caches)
    store_bytes = int(n_new * batch.Hkv * 2 * (batch.D * e_kv + meta))
    if args.step == "fused":
        # the new token's K/V are read from the input instead of the cache: the
        # decode byte count already holds them; add the stores
        launch_bytes = dec_bytes + store_bytes
        step_bytes = launch_bytes
    else:
        launch_bytes = dec_bytes
        # separate cache write: read the new rows, store them, read the slots
        step_bytes = dec_bytes + store_bytes + n_new * batch.Hkv * 2 * batch.D * e_q + n_new * 8
    kv_tokens = int(lens.sum())
    stream = torch.cuda.current_stream()

    # The step is what pkv_paged_attn_decode enqueues, called phase by phase so
    # that HIP events bracket the decode kernel alone: cache write, phase 1
    # (split-context decode; single-partition sequences finish here), phase 2
    # (merge of the longer ones).
    ws = torch.empty(pkv.decode_workspace_size(batch.B, batch.Hq, batch.Hkv, batch.D, mbs_eff,
                                               P_eff, batch.k_cache.dtype),
                     dtype=torch.uint8, device="cuda")

    def step_fused(ev0=None, ev1=None):
        if ev0 is not None:
            ev0.record(stream)
        if window:
            pkv.paged_attn_decode_sliding(batch.q, batch.k_cache, batch.v_cache, block_tables,
                                          batch.context_lens, batch.scale, window,
                                          k_new=batch.k_new, v_new=batch.v_new, out=out,
                                          k_scale=batch.k_scale, v_scale=batch.v_scale,
                                          partition_size=P_eff, workspace=ws)
        else:
            pkv.paged_attn_decode_append(batch.q, batch.k_new, batch.v_new, batch.k_cache,
                                         batch.v_cache, batch.block_tables, batch.context_lens,
                                         batch.scale, out=out, k_scale=batch.k_scale,
                                         v_scale=batch.v_scale, partition_size=P_eff,
                                         workspace=ws)
        if ev1 is not None:
            ev1.record(stream)

    def step_separate(ev0=None, ev1=None):
        pkv.kv_cache_write(batch.k_new, batch.v_new, batch.k_cache, batch.v_cache,
                           batch.slot_new, batch.k_scale, batch.v_scale)
        if ev0 is not None:
            ev0.record(stream)
        pkv.paged_attn_decode_partials(batch.q, batch.k_cache, batch.v_cache, batch.block_tables,
                                       batch.context_lens, batch.scale, P_eff,
                                       k_scale=batch.k_scale, v_scale=batch.v_scale, out=out,
                                       partials=partials)
        if ev1 is not None:
            ev1.record(stream)
        if NP > 1:
            pkv.paged_attn_reduce(*partials, batch.context_lens, P_eff, out=out,
                                  skip_single_partition=True)

    if window and args.step != "fused":
        print("the sliding-window workload runs the fused step only", file=sys.stderr)
        sys.exit(2)
    step = step_fused if args.step == "fused" else step_separate

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    if args.step == "fused":
        # one decode launch per step (plus the merge launch when NP > 1): the
        # events at the ends of the timed region give the average launch
        ms_per_step, gpu_ms = timed_steps(step, args.steps, stream)
        dec_avg_ms = gpu_ms
        timing = ("HIP events at the ends of the timed region on the launch stream, divided by "
                  "the steps (one decode launch per step" +
                  (" and one merge launch" if NP > 1 else "") + "; gaps between launches "
                  "included)")
    else:
        # three launches per step: events around the decode launch inside the
        # timed region
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        it = iter(evs)
        ms_per_step, gpu_ms = timed_steps(lambda: step(*next(it)), args.steps, stream)
        dec_avg_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
        timing = "HIP events around every decode launch of the timed region"
    assert torch.isfinite(out.float()).all()
    dec_ms = per_launch_events(step, args.steps)
    achieved = launch_bytes / (dec_avg_ms * 1e-3) / 1e9
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    # The library runs decodes with 16-bit q of 8 to 63 q heads per kv head
    # over a cache of q's dtype, or 4 to 63 over an INT8, FP8 or 4-bit one (no
    # window) on the matrix cores: the multi-query kernel, which also stores (and quantizes) the
    # new token; phase 1 alone keeps the decode kernel.
    g = batch.Hq // batch.Hkv
    quant = cfg["cache"] in ("i8", "f8", "u4")
    mfma_route = (args.step == "fused" and not window and (4 if quant else 8) <= g < 64 and
                  cfg["dtype"] in ("f16", "bf16") and (cfg["cache"] == cfg["dtype"] or quant))
    sources = MULTI_SOURCES if mfma_route else KERNEL_SOURCES
    traffic, traffic_ratio = traffic_for(f"{args.config}/{args.step}", launch_bytes, sources)
    if mfma_route:
        kernel_label = "paged_multi_kernel" + (" + paged_reduce_kernel (events span both)"
                                               if NP > 1 else "")
        launches = {"kv_cache_write_kernel": 0, "paged_multi_kernel": 1,
                    "paged_reduce_kernel": 1 if NP > 1 else 0}
    else:
        kernel_label = "paged_decode_kernel" + (" + paged_reduce_kernel (events span both)"
                                                if (NP > 1 and args.step == "fused") else "")
        launches = {"kv_cache_write_kernel": 0 if args.step == "fused" else 1,
                    "paged_decode_kernel": 1, "paged_reduce_kernel": 1 if NP > 1 else 0}

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["cache"] if cfg["cache"] in W.SCALED else cfg["dtype"],
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD_NAMES[args.config],
            "num_seqs": batch.B, "num_q_heads": batch.Hq, "num_kv_heads": batch.Hkv,
            "head_dim": batch.D, "block_size": W.BLOCK_SIZE,
            "context_lens": (f"U[{cfg['ctx'][0]},{cfg['ctx'][1]}]" if isinstance(cfg["ctx"], tuple)
                             else cfg["ctx"] if len(set(cfg["ctx"])) > 1 else
                             f"{cfg['ctx'][0]} x {len(cfg['ctx'])}"),
            "sum_context_tokens": kv_tokens, "q_dtype": cfg["dtype"], "kv_dtype": cfg["cache"],
            "partition_size": P_eff, "seed": batch.seed, "parallelism": "single-gpu",
            "step": args.step,
            **({"sliding_window": window, "attended_tokens": kv_tokens} if window else {}),
        },
        "kv_tokens_per_s": round(kv_tokens / (ms_per_step * 1e-3), 1),
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "ms_per_step_gpu_events": round(gpu_ms, 5),
        "decode_kernel_us": round(dec_avg_ms * 1e3, 2),
        "decode_kernel_timing": timing,
        "per_launch_events_us_mean_p10_p50_p90": (
            [round(float(np.mean(dec_ms)) * 1e3, 2)] +
            [round(float(np.percentile(dec_ms, q)) * 1e3, 2) for q in (10, 50, 90)]),
        "decode_alg_bytes": dec_bytes,
        "launch_alg_bytes": launch_bytes,
        "step_alg_bytes": step_bytes,
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None if traffic is None else int(traffic),
            "traffic_unit": "bytes/launch",
            "traffic_over_alg": None if traffic_ratio is None else round(traffic_ratio, 4),
            "kernel": kernel_label,
            "kernel_sha": kernel_sha(sources),
            "launches_per_step": launches,
        },
    }
    if batch.k_cache.element_size() * batch.D * W.BLOCK_SIZE == 4096 and not window:
        result["practical_ceiling"] = practical_ceiling(batch, stream, dec_bytes)
        result["practical_ceiling"]["decode_frac_of_tile_read"] = round(
            achieved / result["practical_ceiling"]["tile_read_gbs"], 4)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = run_cpu_baseline(batch, args.config, args.cpu_seconds,
                                                  e_kv, e_q, int8, window)
    print(json.dumps(result), flush=True)


def practical_ceiling(batch, stream, dec_bytes, reps=10):
    """Context for the decode's rate: the HBM read rate, on this GPU in this
    run, of (1) a plain streaming read of the same number of bytes from the
    pool and (2) the decode's own tile reads (the batch's K/V tiles through
    its block tables, longest sequences first, one work-group per (sequence,
    kv head), in the decode's order of work-groups) without any arithmetic."""
    import numpy as np
    import torch

    import paged_kv_cache_264_amd as pkv

    lens = batch.layout.context_lens
    order = np.argsort(-lens, kind="stable")

    def head(t):
        # the decode's order of a sequence's kv heads (with a multiple of 16
        # heads, the 8 XCDs read adjacent pairs of them)
        if batch.Hkv % 16:
            return t
        return (t & ~15) | ((t >> 3) & 1) | ((t & 7) << 1)

    items = torch.from_numpy(np.array([(s, head(t)) for s in order for t in range(batch.Hkv)],
                                      np.int32)).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    half = min(dec_bytes // 2, batch.k_cache.numel() * batch.k_cache.element_size())
    k_flat = batch.k_cache.view(-1).view(torch.uint8)[:half]
    v_flat = batch.v_cache.view(-1).view(torch.uint8)[:half]

    def run(fn):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    t_stream = run(lambda: (pkv.stream_read(k_flat, sink), pkv.stream_read(v_flat, sink)))
    t_tile = run(lambda: pkv.tile_read(batch.k_cache, batch.v_cache, batch.block_tables,
                                       batch.context_lens, items, sink))
    tile_bytes = int(lens.astype(np.int64).sum()) * batch.Hkv * 2 * batch.D * \
        batch.k_cache.element_size()
    return {"stream_read_gbs": round(2 * half / t_stream / 1e9, 1),
            "tile_read_gbs": round(tile_bytes / t_tile / 1e9, 1),
            "note": "read-only kernels (pkv_stream_read: the same byte count read contiguously; "
                    "pkv_tile_read: the batch's K/V tiles through its block tables), no "
                    "arithmetic, HIP events over 10 launches after 3"}


def matrix_core_ceiling(stream, kernel_tflops, reps=5):
    """Context for the chunked-prefill kernel's rate, measured on this GPU in
    this run: the rate the matrix cores sustain on back-to-back independent
    16x16x32 fp16 MFMAs (4 waves per SIMD on every CU, no memory traffic),
    and the LDS read rate of the kernel's two operand reads on each of its
    tile layouts (the K layout serves the 16-byte K reads, the V layout the
    V^T transpose reads; either read on the other layout meets bank
    conflicts)."""
    import torch

    import paged_kv_cache_264_amd as pkv

    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count

    def run(fn):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    groups, rounds = 4 * cus, 2000
    t = run(lambda: pkv.mfma_rate(groups, rounds, sink))
    mfma_tflops = groups * 4 * rounds * 8 * 16384 / t / 1e12
    lds = {}
    names = ["k_read_k_layout", "k_read_v_layout", "vt_read_v_layout", "vt_read_k_layout"]
    for pattern, name in enumerate(names):
        lgroups, lrounds = 2 * cus, 4000
        t = run(lambda: pkv.lds_read_rate(pattern, lgroups, lrounds, sink))
        lds[name] = round(lgroups * 8 * lrounds * 8192 / t / 1e9 / cus, 1)
    return {"mfma_f16_tflops": round(mfma_tflops, 1),
            "kernel_frac_of_mfma_rate": round(kernel_tflops / mfma_tflops, 4),
            "lds_read_gbs_per_cu": lds,
            "note": "pkv_mfma_rate (8 independent 16x16x32 fp16 MFMAs per wave and round, 4 waves "
                    "per SIMD, no memory traffic) and pkv_lds_read_rate (the kernel's operand "
                    "reads, 8 KiB per wave and round, 4 waves per SIMD); HIP events over 5 "
                    "launches after 2"}


def bench_multi(args):
    """Several query tokens per sequence (speculative verification, chunked
    prefill).  A step: the cache write of the B * q_len new tokens' K/V, then
    multi-query causal attention over the paged cache."""
    import numpy as np
    import torch

    import paged_kv_cache_264_amd as pkv
    import workloads as W

    torch.cuda.set_device(0)
    cfg = W.CONFIGS[args.config]
    batch = W.make_batch(args.config, device="cuda", seed=args.seed, poison=False)
    ql = int(cfg["q_len"])
    lens = batch.layout.context_lens.astype(np.int64)
    qlens = np.minimum(lens, ql)
    qsl_np = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    T = int(qsl_np[-1])
    qsl = torch.from_numpy(qsl_np).cuda()
    q = W.token_rows(T, batch.Hq, batch.D, cfg["dtype"], batch.seed, W.S_STEP_Q, "cuda")
    k_new = W.token_rows(T, batch.Hkv, batch.D, cfg["dtype"], batch.seed, W.S_NEWK, "cuda")
    v_new = W.token_rows(T, batch.Hkv, batch.D, cfg["dtype"], batch.seed, W.S_NEWV, "cuda")
    slots = torch.from_numpy(np.concatenate(
        [W.slots_for(batch.layout, b, np.arange(int(n) - int(k), int(n)))
         for b, (n, k) in enumerate(zip(lens, qlens))])).cuda()
    out = torch.empty_like(q)
    mbs = batch.block_tables.shape[1]
    P = args.partition_size or pkv._load().pkv_multi_default_partition_size(
        batch.B, ql, batch.Hq, batch.Hkv, mbs)
    ws = torch.empty(max(pkv._load().pkv_multi_workspace_size(T, batch.Hq, batch.D, mbs, P), 256),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    e = 2
    kv_bytes = int(lens.sum()) * batch.Hkv * 2 * batch.D * e
    launch_bytes = (kv_bytes + T * batch.Hq * batch.D * e * 2
                    + int(sum(W.blocks_needed(int(n)) for n in lens)) * 4 + 8 * batch.B)
    write_bytes = T * batch.Hkv * 2 * batch.D * e * 2 + T * 8
    step_bytes = launch_bytes + write_bytes
    flops = W.multi_query_flops(lens, ql, batch.Hq, batch.D)

    def step(ev0=None, ev1=None):
        pkv.kv_cache_write(k_new, v_new, batch.k_cache, batch.v_cache, slots)
        if ev0 is not None:
            ev0.record(stream)
        pkv.paged_attn_multi(q, batch.k_cache, batch.v_cache, batch.block_tables,
                             batch.context_lens, qsl, batch.scale, ql, out=out, partition_size=P,
                             workspace=ws)
        if ev1 is not None:
            ev1.record(stream)

    def attend():
        pkv.paged_attn_multi(q, batch.k_cache, batch.v_cache, batch.block_tables,
                             batch.context_lens, qsl, batch.scale, ql, out=out, partition_size=P,
                             workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed region: K steps (cache write + attention), events at its ends only
    ms_per_step, gpu_ms_per_step = timed_steps(step, args.steps, stream)
    assert torch.isfinite(out.float()).all()
    # the attention launch's own duration, in the steps as timed (each after
    # its cache write): events around it in every step of a second pass (the
    # events add a few microseconds to a launch, so this pass is not the
    # timed one)
    k_list = per_launch_events(step, args.steps)
    k_ms = float(np.mean(k_list))
    # context: the attention launches alone, back to back, events at the ends
    _, k_b2b_ms = timed_steps(attend, args.steps, stream)
    hbm = launch_bytes / (k_ms * 1e-3) / 1e9
    tflops = flops / (k_ms * 1e-3) / 1e12
    ridge = 2500.0 / HBM_PEAK_GBS * 1e3          # flop per byte where fp16 MFMA meets HBM
    mfma_bound = flops / launch_bytes > ridge
    roof = ({"bound": "mfma", "achieved": round(tflops, 2), "peak": 2500.0, "unit": "TFLOP/s",
             "frac": round(tflops / 2500.0, 4)} if mfma_bound else
            {"bound": "hbm", "achieved": round(hbm, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(hbm / HBM_PEAK_GBS, 4)})
    roof.update({"traffic": None, "kernel": "paged_multi_kernel" + (
        " + paged_reduce_kernel (events span both)" if pkv.num_partitions(mbs, P) > 1 else ""),
        "kernel_sha": kernel_sha(MULTI_SOURCES), "flop_per_byte": round(flops / launch_bytes, 2)})
    result = {
        "metric": METRIC, "value": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg["dtype"], "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[args.config], "num_seqs": batch.B,
                   "queries_per_seq": ql, "query_tokens": T, "num_q_heads": batch.Hq,
                   "num_kv_heads": batch.Hkv, "head_dim": batch.D, "block_size": W.BLOCK_SIZE,
                   "context_lens": f"U[{cfg['ctx'][0]},{cfg['ctx'][1]}]",
                   "sum_context_tokens": int(lens.sum()), "partition_size": P,
                   "seed": batch.seed, "parallelism": "single-gpu",
                   "step": "kv_cache_write of the query tokens + multi-query attention"},
        "query_tokens_per_s": round(T / (ms_per_step * 1e-3), 1),
        "ms_per_step_gpu_events": round(gpu_ms_per_step, 5),
        "multi_kernel_us": round(k_ms * 1e3, 2),
        "multi_kernel_timing": "HIP events around the attention launch of every step (cache "
                               "write, then attention), in a pass after the timed region",
        "per_launch_events_us_mean_p10_p50_p90": [round(k_ms * 1e3, 3)] + [
            round(float(np.percentile(k_list, q)) * 1e3, 3) for q in (10, 50, 90)],
        "multi_kernel_us_back_to_back": round(k_b2b_ms * 1e3, 2),
        "kernel_hbm_gbs": round(hbm, 1), "kernel_tflops": round(tflops, 2),
        "launch_alg_bytes": launch_bytes, "launch_flops": flops,
        "roofline": roof,
    }
    if mfma_bound:
        result["practical_ceiling"] = matrix_core_ceiling(stream, tflops)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = run_multi_cpu_baseline(batch, q, qsl_np, ql, args.cpu_seconds,
                                                        flops, launch_bytes)
    print(json.dumps(result), flush=True)


def run_multi_cpu_baseline(batch, q, qsl_np, ql, target_s, flops, launch_bytes):
    """The multi-query oracle on the first sequences, sized to ~target_s."""
    import numpy as np
    import torch

    import oracle
    import workloads as W

    lens = batch.layout.context_lens
    threads = oracle.num_threads(len(os.sched_getaffinity(0)))

    def h(t):
        t = t.contiguous().cpu()
        return t.view(torch.int16).numpy().view(np.uint16)

    def run(n_seq):
        blocks = np.concatenate([batch.layout.block_tables[s, :W.blocks_needed(lens[s])]
                                 for s in range(n_seq)]).astype(np.int64)
        remap = np.full(batch.num_blocks, -1, np.int64)
        remap[blocks] = np.arange(len(blocks))
        bt = batch.layout.block_tables[:n_seq].copy()
        bt[bt >= 0] = remap[bt[bt >= 0]]
        idx = torch.from_numpy(blocks).cuda()
        T = int(qsl_np[n_seq])
        args = (h(q[:T]), "f16", h(batch.k_cache[idx]), h(batch.v_cache[idx]), "f16",
                bt.astype(np.int32), lens[:n_seq].astype(np.int32), qsl_np[:n_seq + 1],
                batch.scale)
        t = time.perf_counter()
        oracle.paged_multi(*args)
        return time.perf_counter() - t

    t_one = max(run(1), 1e-4)
    n_seq = max(1, min(batch.B, int(target_s / t_one)))
    t_s = run(n_seq)
    frac = float(lens[:n_seq].sum()) / float(lens.sum())
    return {"value": round(launch_bytes * frac / t_s / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"first {n_seq} of {batch.B} sequences ({int(qsl_np[n_seq])} query tokens), "
                      f"one fp64 oracle pass of {t_s:.2f} s",
            "tflops": round(flops * frac / t_s / 1e12, 6), "seconds": round(t_s, 3)}


def bench_sampling(args):
    """Decode with prefix sharing: 16 LLaMA-7B-shaped prompts (U[512, 2048]
    tokens) continued by 4 samples each (64 sequences).  A step is what a
    serving loop does per generated token: the native block manager reserves
    one slot per sequence (copy-on-write of shared partial blocks on the first
    step), its block tables go to the GPU through pinned double buffers, the
    block copies run, then the fused append + decode kernel.  Also times
    pkv_copy_blocks on 1024 block pairs, and reports the pool memory used
    with and without sharing."""
    import types

    import numpy as np
    import torch

    import paged_kv_cache_264_amd as pkv
    import workloads as W

    torch.cuda.set_device(0)
    cfg = W.SAMPLING["sampling"]
    BS = W.BLOCK_SIZE
    Hq, Hkv, D = cfg["Hq"], cfg["Hkv"], cfg["D"]
    n = cfg["samples"]
    prompt_lens = W.sampling_prompt_lens(cfg)
    B = len(prompt_lens) * n
    gen = args.warmup + args.steps
    NB = int(sum(n * -(-(int(L) + gen) // BS) for L in prompt_lens)) + 64
    NB = max(NB, 2048 + 64)
    mbs = max(-(-(int(L) + gen) // BS) for L in prompt_lens)
    seed = cfg["seed"] if args.seed is None else args.seed
    dt = W.TORCH_DTYPE[cfg["dtype"]]
    kc = torch.zeros((NB, Hkv, BS, D), dtype=dt, device="cuda")
    vc = torch.zeros_like(kc)
    bm = pkv.BlockManager(NB)
    for p, L in enumerate(prompt_lens):
        sid = p * n
        bm.add_sequence(sid)
        slots, _ = bm.append([sid], [int(L)])
        k = W.token_rows(int(L), Hkv, D, cfg["dtype"], seed * 100 + p, W.S_TOKEN_K, "cuda")
        v = W.token_rows(int(L), Hkv, D, cfg["dtype"], seed * 100 + p, W.S_TOKEN_V, "cuda")
        pkv.kv_cache_write(k, v, kc, vc, torch.from_numpy(slots).cuda())
        for c in range(1, n):
            bm.fork(sid, sid + c)
    seqs = list(range(B))
    ones = [1] * B
    q = W.token_rows(B, Hq, D, cfg["dtype"], seed, W.S_STEP_Q, "cuda")
    k_new = W.token_rows(B, Hkv, D, cfg["dtype"], seed, W.S_NEWK, "cuda")
    v_new = W.token_rows(B, Hkv, D, cfg["dtype"], seed, W.S_NEWV, "cuda")
    out = torch.empty_like(q)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    P = pkv.default_partition_size(B, Hq, Hkv, mbs, kc.dtype)
    ws = torch.empty(pkv.decode_workspace_size(B, Hq, Hkv, D, mbs, P, kc.dtype),
                     dtype=torch.uint8, device="cuda")
    shared = args.sampling_decode == "shared"
    # the shared prefix of a prompt's samples: its whole blocks (the partial
    # last block is copied on write at the first step)
    prefix_d = torch.from_numpy(np.repeat((prompt_lens // BS * BS).astype(np.int32), n)).cuda()
    group_d = torch.from_numpy((np.arange(len(prompt_lens) + 1) * n).astype(np.int32)).cuda()
    ws_sp = torch.empty(max(pkv.shared_prefix_workspace_size(B, len(prompt_lens), n, Hq, Hkv, D,
                                                             mbs), 256),
                        dtype=torch.uint8, device="cuda")
    pin_t = [torch.empty((B, mbs), dtype=torch.int32, pin_memory=True) for _ in range(2)]
    pin_l = [torch.empty((B,), dtype=torch.int32, pin_memory=True) for _ in range(2)]
    ev_up = [None, None]
    tables = torch.empty((B, mbs), dtype=torch.int32, device="cuda")
    lens_d = torch.empty((B,), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    e_kv = 2
    state = dict(copies=0, host_s=0.0, lens_sum=0)
    store_bytes = B * Hkv * 2 * D * e_kv

    step_lens = []

    def step(i, ev0=None, ev1=None, count=False):
        t = time.perf_counter()
        _, pairs = bm.append(seqs, ones)
        t_mid = time.perf_counter()
        buf = i % 2
        if ev_up[buf] is not None:
            ev_up[buf].synchronize()        # the pinned buffer's last upload is done
        t_tab = time.perf_counter()
        bm.block_tables(seqs, mbs, out=(pin_t[buf], pin_l[buf]))
        state["host_s"] += (t_mid - t) + (time.perf_counter() - t_tab)
        if len(pairs):
            state["copies"] += len(pairs)
            pkv.copy_blocks(kc, vc, torch.from_numpy(pairs).cuda())
        tables.copy_(pin_t[buf], non_blocking=True)
        lens_d.copy_(pin_l[buf], non_blocking=True)
        ev_up[buf] = torch.cuda.Event()
        ev_up[buf].record(stream)
        if count:
            step_lens.append(pin_l[buf].numpy().copy())
        if ev0 is not None:
            ev0.record(stream)
        if shared:
            pkv.paged_attn_decode_shared_prefix(q, kc, vc, tables, lens_d, prefix_d, group_d,
                                                scale, n, k_new=k_new, v_new=v_new, out=out,
                                                workspace=ws_sp)
        else:
            pkv.paged_attn_decode_append(q, k_new, v_new, kc, vc, tables, lens_d, scale,
                                         out=out, partition_size=P, workspace=ws)
        if ev1 is not None:
            ev1.record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    state["host_s"] = 0.0
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j, (e0, e1) in enumerate(evs):
        step(args.warmup + j, e0, e1, count=True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    assert torch.isfinite(out.float()).all()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    dec_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    # Bytes per step.  Per-sequence (the metric's count): every sequence's
    # context K/V, as if nothing were shared.  Unique (the HBM minimum): each
    # physical block once, for the tokens valid in it; the tables of a timed
    # step are prefixes of the final tables (no copies after the first step).
    final_tables, _ = bm.block_tables(seqs, mbs)
    tok_bytes = Hkv * 2 * D * e_kv
    side = B * Hq * D * 2 * 2 + 4 * B
    seq_bytes, uniq_bytes = 0, 0
    for lens_h in step_lens:
        lens_h = lens_h.astype(np.int64)
        seq_bytes += W.algorithmic_bytes(lens_h, Hq, Hkv, D, e_kv, 2) + store_bytes
        nblk = -(-lens_h // BS)
        ids, valid = [], []
        for b in range(B):
            if nblk[b] == 0:
                continue
            ids.append(final_tables[b, :nblk[b]])
            v = np.full(nblk[b], BS, np.int64)
            v[-1] = lens_h[b] - BS * (nblk[b] - 1)
            valid.append(v)
        ids = np.concatenate(ids)
        valid = np.concatenate(valid)
        best = np.zeros(NB, np.int64)
        np.maximum.at(best, ids, valid)
        uniq_bytes += int(best.sum()) * tok_bytes + side + 4 * len(ids) + store_bytes
        state["lens_sum"] += int(lens_h.sum())
    launch_bytes = seq_bytes / args.steps
    unique_bytes = uniq_bytes / args.steps
    value = launch_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = unique_bytes / (dec_ms * 1e-3) / 1e9

    final_lens = np.asarray([bm.sequence_length(s) for s in seqs])
    used = NB - bm.num_free_blocks
    unshared = int(sum(-(-int(x) // BS) for x in final_lens))
    block_bytes = Hkv * BS * D * e_kv * 2

    # copy-on-write kernel alone: 1024 whole-block copies (K and V)
    n_pairs = 1024
    pairs = torch.from_numpy(np.stack([np.arange(n_pairs), np.arange(n_pairs, 2 * n_pairs)],
                                      1).astype(np.int32)).cuda()
    for _ in range(3):
        pkv.copy_blocks(kc, vc, pairs)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    c0.record(stream)
    for _ in range(reps):
        pkv.copy_blocks(kc, vc, pairs)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_us = c0.elapsed_time(c1) * 1e3 / reps
    copy_bytes = n_pairs * block_bytes * 2          # read + write

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD_NAMES["sampling"], "prompts": len(prompt_lens),
            "samples_per_prompt": n, "num_seqs": B, "num_q_heads": Hq, "num_kv_heads": Hkv,
            "head_dim": D, "block_size": BS, "prompt_lens": "U[512,2048]",
            "mean_context_tokens": round(state["lens_sum"] / args.steps / B, 1),
            "partition_size": P, "seed": seed, "parallelism": "single-gpu",
            "step": "block-manager append + table upload + fused decode",
            "decode": ("shared-prefix (prompt blocks once per group, own positions per "
                       "sequence, merge)" if shared else "plain (every sequence's whole context)"),
        },
        "kv_tokens_per_s": round(state["lens_sum"] / args.steps / (ms_per_step * 1e-3), 1),
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "decode_kernel_us": round(dec_ms * 1e3, 2),
        "launch_alg_bytes": int(launch_bytes),
        "launch_unique_bytes": int(unique_bytes),
        "per_sequence_gbs_in_kernel": round(launch_bytes / (dec_ms * 1e-3) / 1e9, 1),
        "host_block_manager_us_per_step": round(state["host_s"] / args.steps * 1e6, 2),
        "cow_copies_first_step": state["copies"],
        "pool_blocks_used": used,
        "pool_blocks_without_sharing": unshared,
        "memory_saved_frac": round(1.0 - used / unshared, 4),
        "copy_blocks": {"pairs": n_pairs, "us": round(copy_us, 2),
                        "achieved": round(copy_bytes / (copy_us * 1e-6) / 1e9, 1),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(copy_bytes / (copy_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
            "kernel": ("paged_multi_kernel + paged_decode_kernel (events span the two; the "
                       "decode merges the prompt partials in its epilogue)" if shared
                       else "paged_decode_kernel"),
            "kernel_sha": kernel_sha(),
            "note": "achieved = unique bytes (each physical block once) / kernel time; value "
                    "counts every sequence's context, so shared prompt blocks count once per "
                    "sample there",
        },
    }
    if not args.no_cpu_baseline:
        tb, lens = bm.block_tables(seqs, mbs)
        fake = types.SimpleNamespace(
            layout=types.SimpleNamespace(context_lens=lens.astype(np.int64), block_tables=tb),
            num_blocks=NB, q=q, k_cache=kc, v_cache=vc, k_scale=None, v_scale=None, B=B, Hq=Hq,
            Hkv=Hkv, D=D, scale=scale)
        result["cpu_baseline"] = run_cpu_baseline(fake, "sampling", args.cpu_seconds, e_kv, 2,
                                                  False)
    print(json.dumps(result), flush=True)


def run_cpu_baseline(batch, cfg_name, target_s, e_kv, e_q, int8, window=0):
    """Time the CPU oracle (as it stands) on the first sequences of the same
    batch, sized to about `target_s` seconds, and express it in the metric's
    unit (algorithmic GB/s)."""
    import numpy as np
    import torch

    import oracle
    import workloads as W

    lens = batch.layout.context_lens
    threads = oracle.num_threads(len(os.sched_getaffinity(0)))

    def view_for(n_seq):
        seqs = np.arange(n_seq)
        blocks = np.concatenate([batch.layout.block_tables[s, :W.blocks_needed(lens[s])]
                                 for s in seqs]).astype(np.int64)
        remap = np.full(batch.num_blocks, -1, np.int64)
        remap[blocks] = np.arange(len(blocks))
        bt = batch.layout.block_tables[:n_seq].copy()
        bt[bt >= 0] = remap[bt[bt >= 0]]
        idx = torch.from_numpy(blocks).cuda()

        def h(t):
            t = t.contiguous().cpu()
            if t.dtype in (torch.float16, torch.bfloat16):
                return t.view(torch.int16).numpy().view(np.uint16)
            if t.dtype == torch.float8_e4m3fn:
                return t.view(torch.uint8).numpy()
            return t.numpy()

        dt = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16",
              torch.int8: "i8", torch.float8_e4m3fn: "f8", torch.uint8: "u4"}
        kw = {}
        if int8:
            kw = dict(k_scale=h(batch.k_scale[idx]), v_scale=h(batch.v_scale[idx]))
        return dict(q=h(batch.q[:n_seq]), q_dtype=dt[batch.q.dtype], k_cache=h(batch.k_cache[idx]),
                    v_cache=h(batch.v_cache[idx]), cache_dtype=dt[batch.k_cache.dtype],
                    block_tables=bt.astype(np.int32), context_lens=lens[:n_seq].astype(np.int32),
                    scale=batch.scale, window=window, **kw)

    # probe on one sequence, then size the sample
    v1 = view_for(1)
    t = time.perf_counter()
    oracle.paged_decode(**v1)
    t_one = max(time.perf_counter() - t, 1e-4)
    att = np.minimum(lens, window) if window else lens     # tokens attended to
    per_tok = t_one / max(int(att[0]), 1)
    n_seq = 1
    while n_seq < batch.B and per_tok * att[:n_seq + 1].sum() < target_s:
        n_seq += 1
    v = view_for(n_seq)
    # passes over the sample until about target_s seconds of oracle work (the
    # whole batch can take well under a second); the median pass is reported
    passes = []
    while True:
        t = time.perf_counter()
        oracle.paged_decode(**v)
        passes.append(time.perf_counter() - t)
        if sum(passes) >= target_s or len(passes) >= 50:
            break
    t_s = float(np.median(passes))
    sub = att[:n_seq]
    meta = 8 if e_kv == 0.5 else (4 if int8 else 0)
    alg = W.algorithmic_bytes(sub, batch.Hq, batch.Hkv, batch.D, e_kv, e_q, int8, meta)

    # the same oracle on one thread, on a sample sized to about a third of
    # target_s (the first sequences, whole)
    n1 = 1
    per_tok1 = per_tok * threads
    while n1 < n_seq and per_tok1 * att[:n1 + 1].sum() < target_s / 3:
        n1 += 1
    v1 = view_for(n1) if n1 != n_seq else v
    t = time.perf_counter()
    oracle.paged_decode(**v1, nthreads=1)
    t1_s = time.perf_counter() - t
    oracle.num_threads(threads)
    sub1 = att[:n1]
    alg1 = W.algorithmic_bytes(sub1, batch.Hq, batch.Hkv, batch.D, e_kv, e_q, int8, meta)
    return {
        "value": round(alg / t_s / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": f"first {n_seq} of {batch.B} sequences (all {batch.Hq} q heads, "
                  f"{int(sub.sum())} context tokens), median of {len(passes)} fp64 oracle passes "
                  f"({sum(passes):.1f} s in all)",
        "kv_tokens_per_s": round(float(sub.sum()) / t_s, 1),
        "seconds": round(t_s, 3),
        "passes": len(passes),
        "single_thread": {
            "value": round(alg1 / t1_s / 1e9, 5), "unit": "GB/s", "cores": 1,
            "sample": f"first {n1} of {batch.B} sequences ({int(sub1.sum())} context tokens), "
                      f"one fp64 oracle pass on one thread",
            "kv_tokens_per_s": round(float(sub1.sum()) / t1_s, 1), "seconds": round(t1_s, 3)},
    }


def bench_cache_write(args):
    """The INT8 workload's cache write alone: the decode step's 64 new tokens
    (one per sequence, at position context_len - 1, slots from the block
    tables) quantized on write into the INT8 pool (absmax per (slot, kv head),
    round half to even).  A step is one pkv_kv_cache_write launch."""
    import numpy as np
    import torch

    import paged_kv_cache_264_amd as pkv
    import workloads as W

    torch.cuda.set_device(0)
    cfg = W.CONFIGS["int8"]
    batch = W.make_batch("int8", device="cuda", seed=args.seed, poison=False)
    stream = torch.cuda.current_stream()
    T = int((batch.slot_new >= 0).sum())
    e_src = 2
    # read the fp16 rows and the slots, write the codes and one fp32 scale per row
    alg = T * batch.Hkv * 2 * (batch.D * e_src + batch.D * 1 + 4) + T * 8

    def step(ev0=None, ev1=None):
        if ev0 is not None:
            ev0.record(stream)
        pkv.kv_cache_write(batch.k_new, batch.v_new, batch.k_cache, batch.v_cache,
                           batch.slot_new, batch.k_scale, batch.v_scale)
        if ev1 is not None:
            ev1.record(stream)

    for _ in range(args.warmup):
        step()
    ms_per_step, gpu_ms = timed_steps(step, args.steps, stream)
    per = per_launch_events(step, args.steps)
    # A launch takes a few microseconds, less than the binding needs to
    # enqueue one from Python, so the steps above time the host.  The
    # kernel's own rate: REPS launches captured in a HIP graph and replayed
    # back to back (the write is idempotent: same rows, same slots), timed
    # with events on the replay stream.
    reps = 50
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        step()                                 # first launch outside the capture
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            for _ in range(reps):
                step()
    torch.cuda.synchronize()
    for _ in range(3):
        graph.replay()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    g0.record(stream)
    for _ in range(args.steps):
        graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    launch_ms = g0.elapsed_time(g1) / (args.steps * reps)
    achieved = alg / (launch_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC, "value": round(alg / (ms_per_step * 1e-3) / 1e9, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "i8", "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES["int8-write"], "new_tokens": T,
                   "num_kv_heads": batch.Hkv, "head_dim": batch.D, "block_size": W.BLOCK_SIZE,
                   "src_dtype": cfg["dtype"], "kv_dtype": "i8", "seed": batch.seed,
                   "slot_mapping": "position context_len-1 of each sequence, from its block "
                                   "table", "parallelism": "single-gpu"},
        "step_gpu_us": round(gpu_ms * 1e3, 3),
        "write_kernel_us": round(launch_ms * 1e3, 3),
        "write_kernel_timing": f"{reps} launches captured in a HIP graph, replayed {args.steps} "
                               f"times back to back, HIP events around the replays",
        "per_launch_events_us_mean_p10_p50_p90": (
            [round(float(np.mean(per)) * 1e3, 3)] +
            [round(float(np.percentile(per, q)) * 1e3, 3) for q in (10, 50, 90)]),
        "launch_alg_bytes": alg,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "kv_cache_write_kernel",
                     "kernel_sha": kernel_sha(["kv_cache_write.hip", "pkv_device.h",
                                               "struct CacheWriteArgs"]),
                     "note": "1.6 MB per launch: the launch is bound by its fixed latency "
                             "(start-up and one round trip to HBM), not by HBM bandwidth; in "
                             "the decode step the same write is fused into the decode launch"},
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
