#!/usr/bin/env python3
"""Paged-attention decode benchmark on one MI355X.

One step = one pass of the whole hot path over one batch: pa_plan (work
list), the persistent partition kernel and the log-sum-exp reduce. Inputs are
seeded synthetic workloads (workloads.CONFIGS) already resident in HBM; before
every step a 1 GiB read (a reduction over a scratch tensor) evicts L2 and the
256 MB Infinity Cache, outside the timed events, so KV really streams from
HBM. The flush reads rather than writes: a write flush would leave up to
256 MB of dirty lines whose write-back competes with the timed kernel.

Three timed passes, each of warmups-then-samples with the median reported
(the method of Ascend/RecSDK issue #1281, section "测试方法"): HIP events on
the launch stream around the whole step (the headline: nothing else between
them), around pa_decode with its plan built beforehand (decode latency), and
around each of the three kernels (the breakdown and the partition kernel's
roofline; these extra events cost a few microseconds of their own).

The JSON line's `value` is KV-read GB/s of the whole step on the headline
workload (the long-context head_dim-256 decode, the largest workload);
`config.decode_frac_of_peak` gives the decode-level fraction of 8 TB/s (plan
built beforehand) of every workload the 70% bar applies to; `per_config`
carries every workload; `roofline` is the partition kernel's algorithmic KV
bytes over its mean event duration against 8 TB/s; `cpu_baseline` times the
CPU oracle on a bounded sample of the headline workload, whose outputs also
check the GPU's. `append` times the
KV-cache append (the write side, pa_cache_append) at a decode-sized shape (C4's
32 sequences x 4 new tokens, latency-bound) and at two prefill-sized shapes
(HBM-bound), with the same flush and events. `decode_loop` times back-to-back
decode steps (context bump, append, plan, decode) launched eagerly, replayed
as one graph per step, and unrolled eight to a graph, and with one plan for
eight steps. `prefill` times the chunked-prefill shapes (192 and 256 query
rows per kv head, one K/V pass) against the HBM and bf16 MFMA rooflines.

`--scale-sweep` replaces the step bench with a sweep of the partition kernel
over context lengths scaled 1/8 .. 2x, fitting time = fixed + bytes / rate per
workload (one JSON line of fits and points). `--plan-sweep` times pa_plan
alone over batch sizes up to 16384 sequences x 8 kv heads.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged-attn decode latency (µs) and KV-read HBM GB/s (% of peak), 1 GPU"
HBM_PEAK_GBS = 8000.0
HEADLINE = "C5_long_ctx_d256"
# workloads the 70%-of-HBM bar applies to (batched GQA, fp8 persistent, long context)
BAR_WORKLOADS = ("C3_batched_gqa", "C4_fp8_q1_per_token", "C4_fp8_q4_per_token",
                 "C4_fp8_q1_per_tensor", "C4_fp8_q4_per_tensor", "C5_long_ctx_d256")
FLUSH_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "partition_kernel_hbm_traffic_all_workloads.md")
MFMA_FILE = os.path.join(ROOT, "profiles", "partition_kernel_mfma_busy_all_workloads.md")
KERNEL_SOURCES = ("pa_decode.hip", "pa_common.h")


def kernel_source_digest():
    """sha256 over the partition kernel's sources with line comments and blank
    lines dropped, so that a comment edit keeps a counter record valid."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_attention_decode_block_amd", "csrc", f)) as fh:
            for ln in fh:
                ln = re.sub(r"//.*", "", ln).rstrip()
                if ln:
                    h.update(ln.encode() + b"\n")
    return h.hexdigest()


def recorded_traffic(workload):
    """HBM bytes per partition launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary (already scaled by the copy-kernel calibration), or
    None when there is no record for the workload or the kernel sources have
    changed since the counters were taken."""
    digest = kernel_source_digest()
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    for ln in lines:
        f = ln.split()
        if len(f) == 5 and f[0] == "traffic" and f[1] == workload:
            if f[2] != digest:
                return None
            return {"read_bytes": int(f[3]), "written_bytes": int(f[4]),
                    "total_bytes": int(f[3]) + int(f[4])}
    return None


def recorded_mfma(workload):
    """MFMA busy fraction of the partition kernel (rocprofv3 MfmaUtil / 100) and
    the bf16 MFMA flops one launch executes (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512),
    from the committed counter summary, or None when there is no record for the
    workload or the kernel sources have changed since the counters were taken."""
    digest = kernel_source_digest()
    try:
        lines = open(MFMA_FILE).read().splitlines()
    except OSError:
        return None
    for ln in lines:
        f = ln.split()
        if len(f) == 5 and f[0] == "mfma" and f[1] == workload:
            if f[2] != digest:
                return None
            return {"busy_frac": round(float(f[3]) / 100, 4), "flops_per_launch": int(f[4])}
    return None


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=51)
    p.add_argument("--warmup", type=int, default=16)
    p.add_argument("--seed", type=int, default=2026)
    p.add_argument("--only", default="", help="comma list of workloads (default: all)")
    p.add_argument("--grid-multiplier", type=int, default=0)
    p.add_argument("--partition", type=int, default=0)
    p.add_argument("--no-flush", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--no-append", action="store_true", help="skip the KV-cache append timings")
    p.add_argument("--no-prefill", action="store_true",
                   help="skip the chunked-prefill timings (many query rows per kv head)")
    p.add_argument("--no-loop", action="store_true",
                   help="skip the decode-loop timings (eager vs graph-captured steps)")
    p.add_argument("--scale-sweep", action="store_true",
                   help="instead of the step bench: time the partition kernel at context "
                        "lengths scaled by 1/8 .. 2 and fit time = fixed + bytes / rate")
    p.add_argument("--plan-sweep", action="store_true",
                   help="instead of the step bench: time pa_plan alone over batch sizes from "
                        "64 x 8 to 16384 x 8 (sequences x kv heads)")
    p.add_argument("--tune", action="store_true",
                   help="instead of the step bench: time every (grid multiplier, partition size, "
                        "fused or separate reduce) per workload and write the tuning table")
    p.add_argument("--tune-out", default="",
                   help="where --tune writes the table (default: the package's tuning.csv)")
    p.add_argument("--tune-margin", type=float, default=0.02,
                   help="a setting other than the default must be faster by this fraction, "
                        "in graph replays and in eager launches alike")
    p.add_argument("--read-probe", action="store_true",
                   help="instead of the step bench: HBM read rate of the K/V load layouts alone "
                        "(pa_debug_read_probe) over a 4 GiB buffer, contiguous and page-scattered")
    p.add_argument("--prefill-only", action="store_true",
                   help="instead of the step bench: only the chunked-prefill timings (one JSON "
                        "line), e.g. for counter runs over those kernels alone")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run one 512 MiB device copy first (a known-size kernel for scaling "
                        "rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# workloads whose configuration states the partition size (split-KV
# partitions of 256 tokens); the others leave it to the library (its tuning
# table, else 256)
PARTITION_STATED = ("C2_single_seq", "C4_fp8_q1_per_token", "C4_fp8_q4_per_token",
                    "C4_fp8_q1_per_tensor", "C4_fp8_q4_per_tensor")


def partition_of(name, spec):
    return spec.partition_size if name in PARTITION_STATED else 0


def tuned_entry(name, dims, cus):
    """The tuning-table row pa_plan applies to these dims, if any."""
    from paged_attention_decode_block_amd import tuning
    return tuning.lookup(tuning.read_table(), tuning.shape_key(dims, cus))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the decode runs on a single MI355X and has no "
              f"multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_attention_decode_block_amd as pa
    import workloads as W

    dev = torch.device("cuda:0")
    names = [n for n in W.CONFIGS] if not args.only else args.only.split(",")
    if HEADLINE not in names and not args.only:
        names.insert(0, HEADLINE)
    flush = None
    if not args.no_flush:
        flush_src = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev).view(256, -1)
        flush_dst = torch.empty(flush_src.shape[1], dtype=torch.float32, device=dev)

        def flush():
            torch.sum(flush_src, dim=0, out=flush_dst)
    cus = pa.pa_query_device(0)
    if args.scale_sweep:
        scale_sweep(args, flush)
        return
    if args.plan_sweep:
        plan_sweep(args, flush)
        return
    if args.tune:
        tune(args, flush)
        return
    if args.read_probe:
        read_probe(args)
        return
    if args.calibrate_copy:
        src = torch.ones(1 << 27, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: 536870912 bytes read, 536870912 bytes written")
        del src, dst
    if args.prefill_only:
        print(json.dumps({"metric": "chunked-prefill pa_decode: KV GB/s and MFMA TFLOP/s, 1 GPU",
                          "steps": args.steps, "warmup": args.warmup,
                          "prefill": prefill_bench(args, flush)}), flush=True)
        return
    results = {}
    keep = {}
    for name in names:
        spec = W.CONFIGS[name]
        t0 = time.time()
        w = W.generate(spec, args.seed)
        log(f"{name}: drew inputs in {time.time() - t0:.1f}s, ctx sum {int(w.context_lens.sum())}")
        d = {k: getattr(w, k).to(dev) for k in ("q", "k_cache", "v_cache", "block_table",
                                                 "context_lens")}
        d["kv_scales"] = None if w.kv_scales is None else w.kv_scales.to(dev)
        kvd = pa.PA_KV_FP8_E4M3FN if spec.kv_dtype == W.KV_FP8 else pa.PA_KV_BF16
        mode = {W.SCALE_NONE: pa.PA_SCALE_NONE, W.SCALE_PER_TENSOR: pa.PA_SCALE_PER_TENSOR,
                W.SCALE_PER_TOKEN_HEAD: pa.PA_SCALE_PER_TOKEN_HEAD}[spec.kv_scale_mode]
        dims = pa.make_dims(batch=spec.batch, q_len=spec.q_len, num_q_heads=spec.num_q_heads,
                            num_kv_heads=spec.num_kv_heads, head_dim=spec.head_dim,
                            page_size=spec.page_size, num_pages=w.num_pages,
                            max_pages_per_seq=spec.max_pages_per_seq, kv_dtype=kvd,
                            kv_scale_mode=mode,
                            partition_size=args.partition or partition_of(name, spec),
                            grid_multiplier=args.grid_multiplier)
        ws = torch.empty(pa.pa_workspace_bytes(dims, cus), dtype=torch.uint8, device=dev)
        out = torch.empty_like(d["q"])
        stream = torch.cuda.current_stream()

        def plan_call():
            return pa.pa_plan(dims, d["context_lens"], workspace=ws, stream=stream)

        def partition_call(plan):
            pa.pa_decode_partition(plan, d["q"], d["k_cache"], d["v_cache"], d["block_table"],
                                   d["context_lens"], spec.q_len, spec.scale, mode,
                                   d["kv_scales"], out, stream=stream)

        def reduce_call(plan):
            pa.pa_decode_reduce(plan, spec.q_len, mode, out, stream=stream)

        def decode_call(plan):
            pa.pa_decode(plan, d["q"], d["k_cache"], d["v_cache"], d["block_table"],
                         d["context_lens"], spec.q_len, spec.scale, mode, d["kv_scales"], out,
                         stream=stream)

        def timed(body, n_events):
            """args.steps samples of body(events), each after a cache flush;
            returns the events of every sample."""
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_events)]
                   for _ in range(args.steps)]
            torch.cuda.synchronize()
            for i in range(args.steps):
                if flush is not None:
                    flush()
                body(evs[i])
            torch.cuda.synchronize()
            return evs

        def whole_step(ev):
            ev[0].record(stream)
            decode_call(plan_call())
            ev[1].record(stream)

        def decode_only(ev):
            plan = plan_call()
            ev[0].record(stream)
            decode_call(plan)
            ev[1].record(stream)

        def per_kernel(ev):
            ev[0].record(stream)
            plan = plan_call()
            ev[1].record(stream)
            partition_call(plan)
            ev[2].record(stream)
            reduce_call(plan)
            ev[3].record(stream)

        for _ in range(args.warmup):
            if flush is not None:
                flush()
            decode_call(plan_call())
        torch.cuda.synchronize()
        # 1. the step alone between two events (the headline); 2. the decode
        # with its plan built before the first event; 3. events around every
        # kernel (they add a few microseconds of their own to a step)
        t_wall = time.perf_counter()
        ev_step = timed(whole_step, 2)
        wall = time.perf_counter() - t_wall
        ev_dec = timed(decode_only, 2)
        ev_k = timed(per_kernel, 4)
        plan = plan_call()
        status = pa.pa_plan_status(plan)
        assert status == 0, f"{name}: device status {status}"
        ms = lambda a, b: a.elapsed_time(b) * 1e3  # noqa: E731
        step_us = [ms(e[0], e[1]) for e in ev_step]
        dec_us = [ms(e[0], e[1]) for e in ev_dec]
        plan_us = [ms(e[0], e[1]) for e in ev_k]
        part_us = [ms(e[1], e[2]) for e in ev_k]
        red_us = [ms(e[2], e[3]) for e in ev_k]
        kvb = w.kv_bytes()
        med = statistics.median
        r = {
            "kv_bytes": kvb,
            "step_us": med(step_us), "decode_us": med(dec_us), "plan_us": med(plan_us),
            "partition_us": med(part_us), "reduce_us": med(red_us),
            "partition_us_mean": statistics.fmean(part_us),
            "step_us_p10": float(np.percentile(step_us, 10)),
            "step_us_p90": float(np.percentile(step_us, 90)),
            "decode_us_p10": float(np.percentile(dec_us, 10)),
            "decode_us_p90": float(np.percentile(dec_us, 90)),
            "wall_us_per_step_incl_flush": wall / args.steps * 1e6,
            "step_GBps": kvb / med(step_us) / 1e3,
            "decode_GBps": kvb / med(dec_us) / 1e3,
            "partition_GBps": kvb / statistics.fmean(part_us) / 1e3,
        }
        r["step_frac_of_peak"] = r["step_GBps"] / HBM_PEAK_GBS
        r["decode_frac_of_peak"] = r["decode_GBps"] / HBM_PEAK_GBS
        r["variant"] = int(plan.c.variant)
        r["grid"] = int(plan.c.grid)
        r["chosen"] = {"grid_multiplier": int(plan.c.dims.grid_multiplier),
                       "partition_size": int(plan.c.dims.partition_size),
                       "reduce": "fused" if plan.c.dims.flags & pa.PA_FLAG_FUSED_REDUCE
                       else "separate",
                       "source": "tuning table" if tuned_entry(name, dims, cus) else "default"}
        results[name] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
        log(f"{name}: step {r['step_us']:.1f}us (plan {r['plan_us']:.1f}, partition "
            f"{r['partition_us']:.1f}, reduce {r['reduce_us']:.1f}) -> {r['step_GBps']:.0f} GB/s "
            f"step, {r['decode_GBps']:.0f} GB/s decode")
        if name == HEADLINE:
            keep = dict(w=w, out=out.cpu(), spec=spec)
        del d, ws, out, w
        torch.cuda.empty_cache()

    append = None if args.no_append else append_bench(args, flush)
    prefill = None if args.no_prefill else prefill_bench(args, flush)
    loops = None if args.no_loop else decode_loop_bench(args)

    head = HEADLINE if HEADLINE in results else names[0]
    hr = results[head]
    spec = W.CONFIGS[head]
    cpu = None
    parity = None
    if keep and not args.no_cpu_baseline:
        cpu, parity = cpu_baseline(keep, args.cpu_seconds)
    recorded = not args.partition and not args.grid_multiplier
    traffic = recorded_traffic(head) if recorded else None
    mfma = recorded_mfma(head) if recorded else None
    line = {
        "metric": METRIC,
        "value": round(hr["step_GBps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(hr["step_us"] / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{head}: batch {spec.batch}, q_len {spec.q_len}, {spec.num_q_heads} query "
                        f"heads / {spec.num_kv_heads} kv heads, head_dim {spec.head_dim}, page "
                        f"{spec.page_size}, context U[{spec.ctx_lo},{spec.ctx_hi}], partition "
                        f"{args.partition or spec.partition_size}, seed {args.seed}",
            "kv_bytes": hr["kv_bytes"],
            "latency_us": hr["step_us"],
            "decode_latency_us": hr["decode_us"],
            "frac_of_hbm_peak": round(hr["step_frac_of_peak"], 4),
            "decode_frac_of_peak": {n: results[n]["decode_frac_of_peak"] for n in BAR_WORKLOADS
                                    if n in results},
            "decode_frac_definition": "algorithmic KV bytes / median HIP-event time of pa_decode "
                                      "(partition + reduce, plan built before the first event) "
                                      "/ 8 TB/s",
            "timing": "median of HIP-event step times (plan + partition + reduce, two events "
                      "per step) on the launch stream; 1 GiB read flush of L2 / Infinity Cache "
                      "before each step, outside the events",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "partition",
            "achieved": round(hr["partition_GBps"], 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(hr["partition_GBps"] / HBM_PEAK_GBS, 4),
            "traffic": traffic["total_bytes"] if traffic else None,
            "traffic_detail": traffic,
            "traffic_source": ("rocprofv3 FETCH_SIZE / WRITE_SIZE per partition dispatch, scaled by "
                               "a 512 MiB copy, from the committed record for these kernel sources "
                               "(profiles/partition_kernel_hbm_traffic_all_workloads.md); null when "
                               "the sources changed since"),
            "bytes_per_launch": hr["kv_bytes"],
            "mean_launch_us": hr["partition_us_mean"],
            "mfma_busy_frac": mfma["busy_frac"] if mfma else None,
            "mfma_source": ("rocprofv3 MfmaUtil, SQ_INSTS_VALU_MFMA_MOPS_BF16, committed record for "
                            "these kernel sources (profiles/partition_kernel_mfma_busy_"
                            "all_workloads.md); null when the sources changed since"),
            "mfma_tflops": (round(mfma["flops_per_launch"] / hr["partition_us_mean"] / 1e6, 2)
                            if mfma else None),
        },
        "cpu_baseline": cpu,
        "parity_sample": parity,
        "per_config": results,
        "append": append,
        "prefill": prefill,
        "decode_loop": loops,
    }
    print(json.dumps(line), flush=True)


# KV-cache append shapes: (batch, new tokens per sequence, kv heads, head dim,
# page size, fp8 per-token-head scales or bf16)
APPEND_SHAPES = {
    "decode_c4_fp8_per_token": (32, 4, 1, 128, 1024, True),
    "prefill_fp8_per_token": (32, 4096, 1, 128, 1024, True),
    "prefill_bf16_c3_heads": (64, 512, 8, 128, 16, False),
}


def append_bench(args, flush):
    """pa_cache_append timed per launch (median of HIP-event samples after a
    read flush). Algorithmic bytes: the new K/V rows read (bf16) plus the cache
    rows written (and the per-token scales)."""
    import numpy as np
    import torch

    import paged_attention_decode_block_amd as pa

    dev = torch.device("cuda:0")
    gen = torch.Generator(device="cpu").manual_seed(args.seed)
    res = {}
    for name, (B, q_len, hkv, D, ps, fp8) in APPEND_SHAPES.items():
        maxp = -(-q_len // ps) + 2
        num_pages = B * maxp
        ctx = torch.randint(q_len, maxp * ps + 1, (B,), generator=gen, dtype=torch.int32)
        bt = torch.randperm(num_pages, generator=gen, dtype=torch.int32).view(B, maxp)
        nk = torch.randn(B, q_len, hkv, D, generator=gen).to(torch.bfloat16).to(dev)
        nv = torch.randn(B, q_len, hkv, D, generator=gen).to(torch.bfloat16).to(dev)
        elt = 1 if fp8 else 2
        kc = torch.zeros(num_pages, hkv, ps, D, dtype=torch.uint8 if fp8 else torch.bfloat16,
                         device=dev)
        vc = torch.zeros_like(kc)
        sc = torch.zeros(2, num_pages, hkv, ps, dtype=torch.float32, device=dev) if fp8 else None
        dims = pa.make_dims(batch=B, q_len=q_len, num_q_heads=hkv, num_kv_heads=hkv, head_dim=D,
                            page_size=ps, num_pages=num_pages, max_pages_per_seq=maxp,
                            kv_dtype=pa.PA_KV_FP8_E4M3FN if fp8 else pa.PA_KV_BF16,
                            kv_scale_mode=pa.PA_SCALE_PER_TOKEN_HEAD if fp8 else pa.PA_SCALE_NONE)
        ctx_d, bt_d = ctx.to(dev), bt.to(dev)
        rows = B * q_len * hkv
        nbytes = rows * D * 2 * 2 + rows * D * elt * 2 + (rows * 8 if fp8 else 0)
        us = []
        for it in range(args.warmup + args.steps):
            if flush:
                flush()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            pa.pa_cache_append(dims, nk, nv, bt_d, ctx_d, kc, vc, sc)
            e1.record()
            torch.cuda.synchronize()
            if it >= args.warmup:
                us.append(e0.elapsed_time(e1) * 1e3)
        t = statistics.median(us)
        res[name] = {"rows": rows, "bytes": nbytes, "us": round(t, 3),
                     "GBps": round(nbytes / t / 1e3, 2),
                     "frac_of_hbm_peak": round(nbytes / t / 1e3 / HBM_PEAK_GBS, 4)}
        log(f"append {name}: {rows} rows, {nbytes} bytes in {t:.1f} us -> {nbytes / t / 1e3:.0f} GB/s")
        del nk, nv, kc, vc, sc
    torch.cuda.empty_cache()
    return res


def prefill_bench(args, flush):
    """pa_decode on the chunked-prefill shapes (workloads.PREFILL: 192 and 256
    query rows per kv head, which one kernel serves while reading each K/V
    chunk once), plan built beforehand, median of HIP-event samples after a
    read flush. Reported against both rooflines: KV bytes / time against
    8 TB/s, and the algorithmic MFMA flops (QK^T and PV over every visible key
    of every row, 4 * head_dim flops per row and key) / time against the bf16
    dense peak of 2.5 PFLOP/s."""
    import numpy as np
    import torch

    import paged_attention_decode_block_amd as pa
    import workloads as W

    dev = torch.device("cuda:0")
    cus = pa.pa_query_device(0)
    res = {}
    for name, spec in W.PREFILL.items():
        if args.only and name not in args.only.split(","):
            continue
        w = W.generate(spec, args.seed)
        d = {k: getattr(w, k).to(dev) for k in ("q", "k_cache", "v_cache", "block_table",
                                                 "context_lens")}
        kvs = None if w.kv_scales is None else w.kv_scales.to(dev)
        mode = {W.SCALE_NONE: pa.PA_SCALE_NONE, W.SCALE_PER_TENSOR: pa.PA_SCALE_PER_TENSOR,
                W.SCALE_PER_TOKEN_HEAD: pa.PA_SCALE_PER_TOKEN_HEAD}[spec.kv_scale_mode]
        dims = pa.make_dims(batch=spec.batch, q_len=spec.q_len, num_q_heads=spec.num_q_heads,
                            num_kv_heads=spec.num_kv_heads, head_dim=spec.head_dim,
                            page_size=spec.page_size, num_pages=w.num_pages,
                            max_pages_per_seq=spec.max_pages_per_seq,
                            kv_dtype=pa.PA_KV_FP8_E4M3FN if spec.kv_dtype == W.KV_FP8
                            else pa.PA_KV_BF16, kv_scale_mode=mode,
                            partition_size=spec.partition_size)
        ws = torch.empty(pa.pa_workspace_bytes(dims, cus), dtype=torch.uint8, device=dev)
        out = torch.empty_like(d["q"])
        plan = pa.pa_plan(dims, d["context_lens"], workspace=ws)
        us = []
        for it in range(args.warmup + args.steps):
            if flush is not None:
                flush()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            pa.pa_decode(plan, d["q"], d["k_cache"], d["v_cache"], d["block_table"],
                         d["context_lens"], spec.q_len, spec.scale, mode, kvs, out)
            e1.record()
            torch.cuda.synchronize()
            if it >= args.warmup:
                us.append(e0.elapsed_time(e1) * 1e3)
        assert pa.pa_plan_status(plan) == 0, f"prefill {name}: device status"
        t = statistics.median(us)
        ctx = w.context_lens.numpy().astype(np.int64)
        # keys seen by query i of sequence b: ctx_b - q_len + i + 1
        keys = int(sum(spec.q_len * (c - spec.q_len) + spec.q_len * (spec.q_len + 1) // 2
                       for c in ctx))
        flops = 4 * spec.head_dim * spec.num_q_heads * keys
        kvb = w.kv_bytes()
        res[name] = {"rows_per_kv_head": spec.rows, "q_block": int(plan.c.q_block),
                     "kv_passes": -(-spec.q_len // int(plan.c.q_block)),
                     "us": round(t, 2), "kv_bytes": kvb,
                     "GBps": round(kvb / t / 1e3, 1),
                     "frac_of_hbm_peak": round(kvb / t / 1e3 / HBM_PEAK_GBS, 4),
                     "mfma_flops": flops, "TFLOPs": round(flops / t / 1e6, 1),
                     "frac_of_bf16_mfma_peak": round(flops / t / 1e6 / 2500.0, 4)}
        log(f"prefill {name}: {spec.rows} rows per kv head, {res[name]['kv_passes']} K/V pass(es), "
            f"{t:.1f} us -> {kvb / t / 1e3:.0f} GB/s, {flops / t / 1e6:.0f} TFLOP/s")
        del d, kvs, ws, out, w
        torch.cuda.empty_cache()
    return res


# Decode loops timed eagerly and as graphs: workloads and steps per graph
LOOP_WORKLOADS = ("C1_tiny", "C2_single_seq", "C3_batched_gqa")
LOOP_STEPS = 8


# (workload, context scale factors) of the scale sweep; C5 stops at its own
# size (twice would need 17 GB of bf16 K/V drawn on the host)
SWEEP = (("C3_batched_gqa", (0.125, 0.25, 0.5, 1.0, 2.0)),
         ("C4_fp8_q1_per_token", (0.125, 0.25, 0.5, 1.0, 2.0)),
         ("C4_fp8_q4_per_token", (0.125, 0.25, 0.5, 1.0, 2.0)),
         ("C5_long_ctx_d256", (0.125, 0.25, 0.5, 1.0)))


def scale_sweep(args, flush):
    """Partition-kernel time against KV bytes: each workload with its context
    lengths (range and capacity) scaled by each factor, the rest of its shape
    unchanged. A least-squares line time = fixed + bytes / rate splits a
    launch's cost into a per-launch part (dispatch, the dependent fetches
    before the first K/V bytes, ramp-up and tail, segment merges) and the
    steady streaming rate. Median of HIP-event samples, read flush before
    each. Prints one JSON line."""
    import numpy as np
    import torch

    import paged_attention_decode_block_amd as pa
    import workloads as W

    dev = torch.device("cuda:0")
    cus = pa.pa_query_device(0)
    stream = torch.cuda.current_stream()
    mode_of = {W.SCALE_NONE: pa.PA_SCALE_NONE, W.SCALE_PER_TENSOR: pa.PA_SCALE_PER_TENSOR,
               W.SCALE_PER_TOKEN_HEAD: pa.PA_SCALE_PER_TOKEN_HEAD}
    fits, points = {}, []
    for name, factors in SWEEP:
        base = W.CONFIGS[name]
        xs, ys = [], []
        for f in factors:
            hi = int(base.ctx_hi * f)
            lo = max(int(base.ctx_lo * f), base.q_len)
            spec = W.scaled(base, ctx_lo=lo, ctx_hi=hi, max_ctx=0)
            w = W.generate(spec, args.seed)
            d = {k: getattr(w, k).to(dev) for k in ("q", "k_cache", "v_cache", "block_table",
                                                     "context_lens")}
            kvs = None if w.kv_scales is None else w.kv_scales.to(dev)
            mode = mode_of[spec.kv_scale_mode]
            dims = pa.make_dims(batch=spec.batch, q_len=spec.q_len, num_q_heads=spec.num_q_heads,
                                num_kv_heads=spec.num_kv_heads, head_dim=spec.head_dim,
                                page_size=spec.page_size, num_pages=w.num_pages,
                                max_pages_per_seq=spec.max_pages_per_seq,
                                kv_dtype=pa.PA_KV_FP8_E4M3FN if spec.kv_dtype == W.KV_FP8
                                else pa.PA_KV_BF16,
                                kv_scale_mode=mode, partition_size=spec.partition_size)
            ws = torch.empty(pa.pa_workspace_bytes(dims, cus), dtype=torch.uint8, device=dev)
            out = torch.empty_like(d["q"])
            plan = pa.pa_plan(dims, d["context_lens"], workspace=ws, stream=stream)
            ts = []
            for i in range(args.warmup + args.steps):
                if flush is not None:
                    flush()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                pa.pa_decode_partition(plan, d["q"], d["k_cache"], d["v_cache"], d["block_table"],
                                       d["context_lens"], spec.q_len, spec.scale, mode, kvs, out,
                                       stream=stream)
                e1.record(stream)
                e1.synchronize()
                if i >= args.warmup:
                    ts.append(e0.elapsed_time(e1) * 1e3)
            torch.cuda.synchronize()
            assert pa.pa_plan_status(plan) == 0, f"{name} x{f}: device status"
            t = statistics.median(ts)
            b = w.kv_bytes()
            xs.append(b)
            ys.append(t)
            points.append({"workload": name, "factor": f, "ctx": [lo, hi], "kv_bytes": b,
                           "partition_us": round(t, 2), "GBps": round(b / t / 1e3, 1)})
            log(f"sweep {name} x{f}: {b} bytes, {t:.1f} us, {b / t / 1e3:.0f} GB/s")
            del d, kvs, ws, out, w
            torch.cuda.empty_cache()
        A = np.vstack([np.ones(len(xs)), np.asarray(xs, float)]).T
        (fixed, inv), *_ = np.linalg.lstsq(A, np.asarray(ys, float), rcond=None)
        rate = 1.0 / inv / 1e3
        fits[name] = {"fixed_us": round(float(fixed), 2), "steady_GBps": round(float(rate), 1),
                      "steady_frac_of_peak": round(float(rate) / HBM_PEAK_GBS, 4)}
        log(f"sweep {name}: fixed {fixed:.1f} us, steady {rate:.0f} GB/s")
    print(json.dumps({"metric": "partition kernel time vs KV bytes (context lengths scaled)",
                      "unit": "us", "steps": args.steps, "warmup": args.warmup,
                      "fits": fits, "points": points}), flush=True)


# (sequences, kv heads) of the plan sweep: the benchmark's batch, the limits of
# the plan kernel's LDS tables (4096 and 8192 sequences, 4096 and 16336
# pairs) and batches past them
PLAN_SWEEP = ((64, 8), (512, 8), (512, 1), (4096, 1), (4097, 1), (1024, 8), (8192, 1),
              (16384, 1), (4096, 8), (16384, 8))


def plan_sweep(args, flush):
    """pa_plan device time against batch size: context lengths U[512, 8192]
    (seed 2026), page 16, partition 256, q_len 1, group 4; median of HIP-event
    samples around the plan alone, read flush before each. Prints one JSON
    line."""
    import numpy as np
    import torch

    import paged_attention_decode_block_amd as pa

    dev = torch.device("cuda:0")
    cus = pa.pa_query_device(0)
    stream = torch.cuda.current_stream()
    rng = np.random.default_rng(args.seed)
    points = []
    for B, hkv in PLAN_SWEEP:
        ctx_np = rng.integers(512, 8193, size=B).astype(np.int32)
        ctx = torch.from_numpy(ctx_np).to(dev)
        dims = pa.make_dims(batch=B, q_len=1, num_q_heads=4 * hkv, num_kv_heads=hkv, head_dim=128,
                            page_size=16, num_pages=B * 512, max_pages_per_seq=512,
                            kv_dtype=pa.PA_KV_BF16, kv_scale_mode=pa.PA_SCALE_NONE)
        ws = torch.empty(pa.pa_workspace_bytes(dims, cus), dtype=torch.uint8, device=dev)
        ts = []
        for i in range(args.warmup + args.steps):
            if flush is not None:
                flush()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            plan = pa.pa_plan(dims, ctx, workspace=ws, stream=stream)
            e1.record(stream)
            e1.synchronize()
            if i >= args.warmup:
                ts.append(e0.elapsed_time(e1) * 1e3)
        assert pa.pa_plan_status(plan) == 0, f"plan {B} x {hkv}: device status"
        t = statistics.median(ts)
        points.append({"sequences": B, "kv_heads": hkv, "pairs": B * hkv,
                       "items": int(hkv * ((ctx_np.astype(np.int64) + 255) // 256).sum()),
                       "plan_us": round(t, 2)})
        log(f"plan sweep {B} x {hkv}: {t:.1f} us")
        del ws, ctx
    print(json.dumps({"metric": "pa_plan time vs batch size", "unit": "us", "steps": args.steps,
                      "warmup": args.warmup, "points": points}), flush=True)


def read_probe(args):
    """HBM read rate of the partition pass's two K/V lane layouts, alone
    (pa_debug_read_probe): 16-row blocks of 128, 256 and 512-byte rows (fp8
    and bf16 rows at head_dim 128 and 256) read from a 4 GiB buffer with
    non-temporal 16-byte loads, in block order (contiguous) and in a seeded
    random permutation (page-scattered, as a block table places pages), by 4
    and 8 waves per CU; median of 10 HIP-event timings after 2 warm-ups.
    Prints one JSON line."""
    import torch

    import paged_attention_decode_block_amd as pa

    dev = torch.device("cuda:0")
    cus = pa.pa_query_device(0)
    total = 4 << 30
    buf = torch.ones(total, dtype=torch.uint8, device=dev)
    sink = torch.empty(cus * 16 * 64, dtype=torch.float32, device=dev)
    gen = torch.Generator(device="cpu").manual_seed(args.seed)
    points = []
    for row_bytes in (128, 256, 512):
        nblk = total // (16 * row_bytes)
        orders = {"contiguous": torch.arange(nblk, dtype=torch.int32),
                  "page-scattered": torch.randperm(nblk, generator=gen, dtype=torch.int32)}
        for order, blocks_h in orders.items():
            blocks = blocks_h.to(dev)
            for waves in (4, 8):
                per = nblk // (cus * waves) // 2 * 2
                nbytes = per * cus * waves * 16 * row_bytes
                rate = {}
                for linear in (True, False):
                    ts = []
                    for it in range(12):
                        e0 = torch.cuda.Event(enable_timing=True)
                        e1 = torch.cuda.Event(enable_timing=True)
                        e0.record()
                        pa.pa_debug_read_probe(buf, blocks, row_bytes, linear, waves, sink)
                        e1.record()
                        e1.synchronize()
                        if it >= 2:
                            ts.append(e0.elapsed_time(e1) * 1e3)
                    rate["linear" if linear else "rows"] = round(nbytes / statistics.median(ts) / 1e3, 1)
                points.append({"row_bytes": row_bytes, "block_bytes": 16 * row_bytes, "order": order,
                               "waves_per_cu": waves, "bytes": nbytes, "GBps": rate})
                log(f"read probe {row_bytes} B rows, {order}, {waves} waves: linear "
                    f"{rate['linear']:.0f} GB/s, rows {rate['rows']:.0f} GB/s")
            del blocks
    print(json.dumps({"metric": "HBM read rate of the K/V load layouts (non-temporal 16-byte loads)",
                      "unit": "GB/s", "peak": HBM_PEAK_GBS, "points": points}), flush=True)


def tune(args, flush):
    """The offline tuner of the persistent grid ("[Kernel][Perf] Optimize
    paged-attention metadata decode", ROCm/FlyDSL PR #910, "Pull request
    overview": a tuned per-shape grid table written by a graph-based tuner).
    Per workload, pa_decode (plan built beforehand) runs with every candidate
    (grid multiplier, partition size, fused or separate reduce), captured once
    in a HIP graph and replayed after a read flush, and launched eagerly the
    same way; medians of HIP-event samples. The fastest candidate by graph
    replay enters the table for the workload's shape class if it beats the
    default (one workgroup per CU, 256 tokens, separate reduce) by the margin
    in both timings; otherwise the default is recorded. Partition sizes vary
    only where the workload's configuration leaves them open. Prints one JSON
    line and writes the table."""
    import torch

    import paged_attention_decode_block_amd as pa
    import workloads as W
    from paged_attention_decode_block_amd import tuning

    dev = torch.device("cuda:0")
    cus = pa.pa_query_device(0)
    stream = torch.cuda.current_stream()
    out_path = args.tune_out or tuning.TABLE
    table = tuning.read_table(out_path) if os.path.exists(out_path) else []
    names = [n for n in W.CONFIGS] if not args.only else args.only.split(",")
    report = {}
    default = (1, 256, 0)
    for name in names:
        spec = W.CONFIGS[name]
        w = W.generate(spec, args.seed)
        d = {k: getattr(w, k).to(dev) for k in ("q", "k_cache", "v_cache", "block_table",
                                                 "context_lens")}
        kvs = None if w.kv_scales is None else w.kv_scales.to(dev)
        mode = {W.SCALE_NONE: pa.PA_SCALE_NONE, W.SCALE_PER_TENSOR: pa.PA_SCALE_PER_TENSOR,
                W.SCALE_PER_TOKEN_HEAD: pa.PA_SCALE_PER_TOKEN_HEAD}[spec.kv_scale_mode]
        kvd = pa.PA_KV_FP8_E4M3FN if spec.kv_dtype == W.KV_FP8 else pa.PA_KV_BF16
        partitions = (256,) if name in PARTITION_STATED else (128, 256, 512)
        out = torch.empty_like(d["q"])
        times = {}
        key = None
        for mult in (1, 2):
            for P in partitions:
                for fused in (0, 1):
                    dims = pa.make_dims(batch=spec.batch, q_len=spec.q_len,
                                        num_q_heads=spec.num_q_heads,
                                        num_kv_heads=spec.num_kv_heads, head_dim=spec.head_dim,
                                        page_size=spec.page_size, num_pages=w.num_pages,
                                        max_pages_per_seq=spec.max_pages_per_seq, kv_dtype=kvd,
                                        kv_scale_mode=mode, partition_size=P,
                                        grid_multiplier=mult,
                                        flags=pa.PA_FLAG_FUSED_REDUCE if fused
                                        else pa.PA_FLAG_SEPARATE_REDUCE)
                    key = tuning.shape_key(dims, cus)
                    ws = torch.empty(pa.pa_workspace_bytes(dims, cus), dtype=torch.uint8,
                                     device=dev)
                    plan = pa.pa_plan(dims, d["context_lens"], workspace=ws, stream=stream)

                    def call():
                        pa.pa_decode(plan, d["q"], d["k_cache"], d["v_cache"], d["block_table"],
                                     d["context_lens"], spec.q_len, spec.scale, mode, kvs, out,
                                     stream=torch.cuda.current_stream())

                    call()
                    torch.cuda.synchronize()
                    side = torch.cuda.Stream()
                    side.wait_stream(torch.cuda.current_stream())
                    graph = torch.cuda.CUDAGraph()
                    with torch.cuda.stream(side):
                        with torch.cuda.graph(graph, stream=side):
                            call()
                    torch.cuda.current_stream().wait_stream(side)
                    res = {}
                    for label, body in (("graph", graph.replay), ("eager", call)):
                        ts = []
                        for i in range(args.warmup + args.steps):
                            if flush is not None:
                                flush()
                            e0 = torch.cuda.Event(enable_timing=True)
                            e1 = torch.cuda.Event(enable_timing=True)
                            e0.record()
                            body()
                            e1.record()
                            e1.synchronize()
                            if i >= args.warmup:
                                ts.append(e0.elapsed_time(e1) * 1e3)
                        res[label] = statistics.median(ts)
                    assert pa.pa_plan_status(plan) == 0, f"tune {name} {(mult, P, fused)}"
                    times[(mult, P, fused)] = res
                    log(f"tune {name} mult={mult} P={P} fused={fused}: graph "
                        f"{res['graph']:.1f} us, eager {res['eager']:.1f} us")
                    del graph, ws, plan
        best = min(times, key=lambda c: times[c]["graph"])
        base = times[default]
        m = 1 - args.tune_margin
        if best != default and not (times[best]["graph"] < m * base["graph"]
                                    and times[best]["eager"] < m * base["eager"]):
            best = default
        e = tuning.Entry(*key, grid_multiplier=best[0], partition_size=best[1],
                         fused_reduce=best[2], decode_us=round(times[best]["eager"], 2),
                         workload=name)
        table = tuning.upsert(table, e)
        report[name] = {"key": list(key), "chosen": list(best),
                        "times_us": {f"m{c[0]}_p{c[1]}_{'fused' if c[2] else 'separate'}": v
                                     for c, v in times.items()}}
        log(f"tune {name}: chose mult={best[0]} P={best[1]} fused={best[2]}")
        del d, kvs, out, w
        torch.cuda.empty_cache()
    tuning.write_table(table, out_path)
    print(json.dumps({"metric": "pa_decode time per tuning candidate", "unit": "us",
                      "steps": args.steps, "warmup": args.warmup, "margin": args.tune_margin,
                      "table": out_path, "workloads": report}), flush=True)


def decode_loop_bench(args):
    """Back-to-back decode steps of a serving loop, each = context lengths +=
    q_len on the device, pa_cache_append of the new tokens, pa_plan and
    pa_decode (five launches). Timed over LOOP_STEPS steps between two HIP
    events: eager launches, one graph replay per step, and all steps unrolled
    in one graph; then with one plan for all LOOP_STEPS steps (the decode reads
    the grown lengths itself), eager and as one graph; reported per step
    (median over samples). No flush
    inside the loop: consecutive steps read the same cache, as a serving loop
    does, so small caches are served from L2 / the Infinity Cache (C3's 1.1 GB
    is not). The steps' inputs stay in fixed buffers. Before each sample the
    context lengths are reset, so every sample rewrites the same slots."""
    import torch

    import paged_attention_decode_block_amd as pa
    import workloads as W

    dev = torch.device("cuda:0")
    res = {}
    S = LOOP_STEPS
    for name in LOOP_WORKLOADS:
        spec = W.CONFIGS[name]
        loop = W.decode_loop(spec, args.seed, S)
        w = loop.start
        kc, vc = w.k_cache.to(dev), w.v_cache.to(dev)
        sc = None if w.kv_scales is None else w.kv_scales.to(dev)
        bt = w.block_table.to(dev)
        ctx0 = w.context_lens.to(dev)
        ctx = ctx0.clone()
        q, nk, nv = loop.q.to(dev), loop.new_k.to(dev), loop.new_v.to(dev)
        out = torch.empty_like(q)
        dims = pa.make_dims(batch=spec.batch, q_len=spec.q_len, num_q_heads=spec.num_q_heads,
                            num_kv_heads=spec.num_kv_heads, head_dim=spec.head_dim,
                            page_size=spec.page_size, num_pages=w.num_pages,
                            max_pages_per_seq=spec.max_pages_per_seq,
                            kv_dtype={W.KV_BF16: pa.PA_KV_BF16,
                                      W.KV_FP8: pa.PA_KV_FP8_E4M3FN}[spec.kv_dtype],
                            kv_scale_mode={W.SCALE_NONE: pa.PA_SCALE_NONE,
                                           W.SCALE_PER_TENSOR: pa.PA_SCALE_PER_TENSOR,
                                           W.SCALE_PER_TOKEN_HEAD: pa.PA_SCALE_PER_TOKEN_HEAD}[
                                spec.kv_scale_mode])
        mode = dims.kv_scale_mode
        ws = torch.empty(pa.pa_workspace_bytes(dims, pa.pa_query_device(0)), dtype=torch.uint8,
                         device=dev)
        status = torch.zeros(1, dtype=torch.int32, device=dev)

        def step(i):
            ctx.add_(spec.q_len)
            pa.pa_cache_append(dims, nk[i], nv[i], bt, ctx, kc, vc, sc, status)
            plan = pa.pa_plan(dims, ctx, workspace=ws)
            pa.pa_decode(plan, q[i], kc, vc, bt, ctx, spec.q_len, spec.scale, mode, sc, out[i])

        def capture(fn):
            st = torch.cuda.Stream()
            st.wait_stream(torch.cuda.current_stream())
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(st):
                with torch.cuda.graph(g, stream=st):
                    fn()
            torch.cuda.current_stream().wait_stream(st)
            return g

        # plan reuse: one plan at the first step's lengths serves all S steps
        # (the decode reads the grown context lengths itself)
        held = {}

        def step_reuse(i):
            ctx.add_(spec.q_len)
            pa.pa_cache_append(dims, nk[i], nv[i], bt, ctx, kc, vc, sc, status)
            if i == 0:
                held["plan"] = pa.pa_plan(dims, ctx, workspace=ws)
            pa.pa_decode(held["plan"], q[i], kc, vc, bt, ctx, spec.q_len, spec.scale, mode, sc,
                         out[i])

        g_one = capture(lambda: step(0))
        g_all = capture(lambda: [step(i) for i in range(S)])
        g_reuse = capture(lambda: [step_reuse(i) for i in range(S)])

        def eager():
            for i in range(S):
                step(i)

        def eager_reuse():
            for i in range(S):
                step_reuse(i)

        def one():
            for _ in range(S):
                g_one.replay()

        def unrolled():
            g_all.replay()

        def unrolled_reuse():
            g_reuse.replay()

        r = {"steps_per_sample": S, "launches_per_step": 5,
             "plan_once_launches_per_step": 4 + 1 / S}
        for label, body in (("eager", eager), ("graph_per_step", one), ("graph_unrolled", unrolled),
                            ("eager_plan_once", eager_reuse),
                            ("graph_unrolled_plan_once", unrolled_reuse)):
            us = []
            for it in range(3 + max(5, args.steps // 3)):
                ctx.copy_(ctx0)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                body()
                e1.record()
                torch.cuda.synchronize()
                if it >= 3:
                    us.append(e0.elapsed_time(e1) * 1e3 / S)
            r[label + "_us_per_step"] = round(statistics.median(us), 3)
        torch.cuda.synchronize()
        if int(status.item()) != 0:
            raise RuntimeError(f"decode loop {name}: append status {int(status.item())}")
        res[name] = r
        log(f"decode loop {name}: eager {r['eager_us_per_step']:.1f} us/step, graph per step "
            f"{r['graph_per_step_us_per_step']:.1f}, {S} steps in one graph "
            f"{r['graph_unrolled_us_per_step']:.1f}; one plan per {S} steps: eager "
            f"{r['eager_plan_once_us_per_step']:.1f}, one graph "
            f"{r['graph_unrolled_plan_once_us_per_step']:.1f}")
        del g_one, g_all, g_reuse, kc, vc, sc, q, nk, nv, out, ws
        torch.cuda.empty_cache()
    return res


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None where unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(keep, seconds):
    """The CPU oracle, as it stands, on a bounded sample of the headline
    workload's sequences; its outputs also check the GPU's on that sample."""
    import numpy as np
    import torch

    import oracle
    import workloads as W

    w, spec, gout = keep["w"], keep["spec"], keep["out"]
    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        cores = max([i["num_threads"] for i in threadpool_info()] or [1])
    except Exception:  # no introspection: the affinity set bounds what BLAS uses
        cores = affinity
    ctx = w.context_lens.tolist()
    # sequences in order, passes repeated until the time target (at most 20 passes)
    order = [b for _ in range(20) for b in range(spec.batch)]
    done, t_total, kv_total, worst = [], 0.0, 0, 0.0
    for b in order:
        sub = W.Workload(W.scaled(spec, batch=1), w.seed, w.q[b:b + 1], w.k_cache, w.v_cache,
                         w.block_table[b:b + 1], w.context_lens[b:b + 1], w.kv_scales, w.num_pages)
        t0 = time.perf_counter()
        want, _ = oracle.decode(sub.q, sub.k_cache, sub.v_cache, sub.block_table,
                                sub.context_lens, spec.q_len, spec.scale, spec.page_size,
                                spec.kv_dtype, spec.kv_scale_mode, sub.kv_scales)
        t_total += time.perf_counter() - t0
        kv_total += sub.kv_bytes()
        got = gout[b:b + 1].float().numpy().astype(np.float64)
        tol = 2e-2 if spec.kv_dtype == W.KV_FP8 else 8e-3
        bad = np.abs(got - want) > tol + tol * np.abs(want)
        worst = max(worst, float(np.abs(got - want).max()))
        if bad.any() or not np.isfinite(got).all():
            raise SystemExit(f"parity failure on sequence {b} of the benchmark workload")
        done.append(b)
        if t_total >= seconds:
            break
    passes = len(done) / spec.batch
    log(f"cpu oracle: {len(done)} sequences ({passes:.2f} passes), {kv_total / 1e6:.1f} MB KV in "
        f"{t_total:.1f}s on {cores} threads")
    cpu = {"value": round(kv_total / t_total / 1e9, 4), "unit": "GB/s", "cores": cores,
           "kind": "oracle",
           "sample": f"{len(done)} sequence decodes ({passes:.2f} passes over the {spec.batch} "
                     f"sequences of the headline workload, {sum(ctx[b] for b in done)} context "
                     f"tokens, {kv_total} KV bytes), float64 NumPy oracle, {t_total:.1f}s",
           "oracle_ms_per_sequence": round(1e3 * t_total / max(len(done), 1), 3),
           "cpu_model": cpu_model(),
           "threads": {"blas_threads_used": cores, "affinity_cpus": affinity,
                       "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS"),
                       "OPENBLAS_NUM_THREADS": os.environ.get("OPENBLAS_NUM_THREADS")}}
    parity = {"sequences_checked": len(set(done)), "max_abs_err": worst,
              "tolerance": ("atol = rtol = 2e-2 (fp8 KV)" if spec.kv_dtype == W.KV_FP8
                            else "atol = rtol = 8e-3 (bf16 KV)")}
    return cpu, parity


if __name__ == "__main__":
    main()
