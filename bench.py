"""Benchmark of paged MLA decode attention on one MI355X.

A step is one pass of the whole hot path over one batch: the split-KV
scheduler, the split-KV decode kernel (page gather -> LDS, scores and values
on bf16 MFMA, fp32 online softmax) and the LSE combine.  Inputs are resident
in HBM before timing starts.  Between timed steps a separate 1 GiB buffer is
read (outside the timed events) so that L2 and the 256 MB Infinity Cache hold
no KV pages and no dirty lines: every step reads its KV from HBM.

Prints one JSON line (rank 0).  `value` is algorithmic HBM GB/s of the whole
step; `roofline` reports the dominant kernel (mla_decode_splitkv) measured
with HIP events on the stream it is launched on.

By default the five configurations of the metric (tiny, membound, ridge,
ragged, long) run one after another, each with W warm-up and K timed steps;
the line is that of the long-context configuration (the largest one by
bytes), with a `per_config` map holding every configuration's step and
kernel times, GB/s, TFLOP/s, roofline fractions and traffic ratio.
`--workload X` times one workload alone.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload KEY]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MLA decode attention TFLOPS + HBM GB/s (% of roofline), 1 MI355X"
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA


# HBM bytes per launch of the decode kernel, from two rocprofv3 --pmc runs of
# this script (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch), each scaled
# by what the same counter reads for a plain 1 GiB int32 elementwise copy
# (--copy-calib-mib 1024): FETCH_SIZE reads 0.5 GiB for it, WRITE_SIZE 1 GiB.
# mfma_util: rocprofv3's MfmaUtil for the decode kernel (a third --pmc run:
# sum of SQ_VALU_MFMA_BUSY_CYCLES over the SIMDs / (GRBM_GUI_ACTIVE of the
# busiest XCD x 1024 SIMDs); a 32x32x16 bf16 product counts 32 busy cycles).
# Keyed by workload ("<workload>/fp8" for the FP8 cache); valid only for the
# kernel source it was measured on
# (sha256 of csrc/mla_kernels.hip), otherwise reported as null.
HBM_TRAFFIC = {
    "membound": {
        "kernel_sha256": "4625f0bb5924a795928211bd350bb7683e98adda00c009bef9bca9dfb8d1325c",
        "fetch_bytes": 307010352,
        "write_bytes": 4210688,
        "fetch_scale": 1.99986,
        "write_scale": 1.0,
        "mfma_util": 0.0846
    },
    "ridge": {
        "kernel_sha256": "4625f0bb5924a795928211bd350bb7683e98adda00c009bef9bca9dfb8d1325c",
        "fetch_bytes": 722688215,
        "write_bytes": 47804982,
        "fetch_scale": 1.99993,
        "write_scale": 1.0,
        "mfma_util": 0.4112
    },
    "long": {
        "kernel_sha256": "4625f0bb5924a795928211bd350bb7683e98adda00c009bef9bca9dfb8d1325c",
        "fetch_bytes": 774460937,
        "write_bytes": 34871011,
        "fetch_scale": 1.99992,
        "write_scale": 1.0,
        "mfma_util": 0.4426
    },
    "ragged": {
        "kernel_sha256": "4625f0bb5924a795928211bd350bb7683e98adda00c009bef9bca9dfb8d1325c",
        "fetch_bytes": 528448095,
        "write_bytes": 65792118,
        "fetch_scale": 1.99992,
        "write_scale": 1.0,
        "mfma_util": 0.4441
    },
    "draft": {
        "kernel_sha256": "4625f0bb5924a795928211bd350bb7683e98adda00c009bef9bca9dfb8d1325c",
        "fetch_bytes": 228788065,
        "write_bytes": 47370240,
        "fetch_scale": 1.99989,
        "write_scale": 1.0,
        "mfma_util": 0.4374
    },
    "prefill": {
        "kernel_sha256": "4625f0bb5924a795928211bd350bb7683e98adda00c009bef9bca9dfb8d1325c",
        "fetch_bytes": 424529934,
        "write_bytes": 92635136,
        "fetch_scale": 1.99992,
        "write_scale": 1.0,
        "mfma_util": 0.5074
    },
    "sparse": {
        "kernel_sha256": "4625f0bb5924a795928211bd350bb7683e98adda00c009bef9bca9dfb8d1325c",
        "fetch_bytes": 161516376,
        "write_bytes": 33686010,
        "fetch_scale": 1.99985,
        "write_scale": 1.0,
        "mfma_util": 0.2062
    },
    "membound/fp8": {
        "kernel_sha256": "4625f0bb5924a795928211bd350bb7683e98adda00c009bef9bca9dfb8d1325c",
        "fetch_bytes": 173876914,
        "write_bytes": 4210688,
        "fetch_scale": 1.99989,
        "write_scale": 1.0,
        "mfma_util": 0.1155
    },
    "ridge/fp8": {
        "kernel_sha256": "4625f0bb5924a795928211bd350bb7683e98adda00c009bef9bca9dfb8d1325c",
        "fetch_bytes": 428502401,
        "write_bytes": 47764992,
        "fetch_scale": 1.99992,
        "write_scale": 1.0,
        "mfma_util": 0.311
    },
    "long/fp8": {
        "kernel_sha256": "4625f0bb5924a795928211bd350bb7683e98adda00c009bef9bca9dfb8d1325c",
        "fetch_bytes": 442176301,
        "write_bytes": 34869789,
        "fetch_scale": 1.99992,
        "write_scale": 1.0,
        "mfma_util": 0.3282
    },
    "ragged/fp8": {
        "kernel_sha256": "4625f0bb5924a795928211bd350bb7683e98adda00c009bef9bca9dfb8d1325c",
        "fetch_bytes": 328802698,
        "write_bytes": 65792000,
        "fetch_scale": 1.99992,
        "write_scale": 1.0,
        "mfma_util": 0.3188
    },
    "draft/fp8": {
        "kernel_sha256": "4625f0bb5924a795928211bd350bb7683e98adda00c009bef9bca9dfb8d1325c",
        "fetch_bytes": 151826040,
        "write_bytes": 47370240,
        "fetch_scale": 1.99993,
        "write_scale": 1.0,
        "mfma_util": 0.3182
    },
    "prefill/fp8": {
        "kernel_sha256": "4625f0bb5924a795928211bd350bb7683e98adda00c009bef9bca9dfb8d1325c",
        "fetch_bytes": 283635462,
        "write_bytes": 92635146,
        "fetch_scale": 1.99992,
        "write_scale": 1.0,
        "mfma_util": 0.3576
    },
    "sparse/fp8": {
        "kernel_sha256": "4625f0bb5924a795928211bd350bb7683e98adda00c009bef9bca9dfb8d1325c",
        "fetch_bytes": 102086588,
        "write_bytes": 33685600,
        "fetch_scale": 1.99992,
        "write_scale": 1.0,
        "mfma_util": 0.1755
    }
}


def _kernel_source_sha() -> str:
    import hashlib
    p = os.path.join(ROOT, "mla_paged_kv_04_amd", "csrc", "mla_kernels.hip")
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(workload: str, kv: str = "bf16"):
    rec = HBM_TRAFFIC.get(workload if kv == "bf16" else f"{workload}/{kv}")
    if rec is None or rec["kernel_sha256"] != _kernel_source_sha():
        return None
    return rec


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(inp, budget_s: float = 12.0) -> dict:
    """The fp64 oracle, as it stands, on a bounded sample of the workload:
    whole requests in order until about `budget_s` seconds have elapsed."""
    import numpy as np
    from oracle import decode, decode_fp8, decode_sparse, decode_sparse_fp8
    from workloads import algorithmic_counts, sparse_counts
    if inp.indices is not None:
        sparse_ref = decode_sparse_fp8 if inp.kv_format == "fp8" else decode_sparse

        def oracle_decode(q, kc, bt, sl, scale, causal, requests):
            return sparse_ref(q, kc, bt, sl, inp.indices, scale, causal, requests=requests)
    else:
        oracle_decode = decode_fp8 if inp.kv_format == "fp8" else decode
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    done = []
    t0 = time.perf_counter()
    passes = 0
    while True:
        for b in range(inp.batch):
            oracle_decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.scale,
                          inp.causal, requests=[b])
            done.append(b)
            if time.perf_counter() - t0 >= budget_s:
                break
        else:
            passes += 1
            continue
        break
    dt = time.perf_counter() - t0
    sl = [int(inp.seqlens[b]) for b in done]
    if inp.indices is not None:
        c = sparse_counts(inp.indices[done], sl, inp.s_q, inp.h_q, inp.causal, inp.kv_format)
    else:
        c = algorithmic_counts(sl, inp.s_q, inp.h_q, inp.kv_format)
    return {
        "value": round(c["bytes"] / dt / 1e9, 4),
        "unit": "GB/s",
        "tflops": round(c["flops"] / dt / 1e12, 6),
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{len(done)} requests ({passes} full passes over the {inp.batch}-request "
                  f"batch, {sum(sl)} keys) in {dt:.1f} s, fp64 numpy on {_cpu_model()}, "
                  f"{os.cpu_count()} logical CPUs",
    }


def splitkv_kernel_name(m_rows: int, kv: str = "bf16", sparse: bool = False) -> str:
    """HIP kernel that the decode launches for m_rows query rows per request
    (per item in the sparse mode)."""
    if m_rows % 128 == 0:
        if sparse:
            return "mla_rowwave_sparse_kernel" if kv == "bf16" else "mla_rowwave_f8_sparse_kernel"
        return "mla_rowwave_kernel" if kv == "bf16" else "mla_rowwave_f8_kernel"
    rt = 1 if m_rows <= 16 else 2 if m_rows <= 32 else 4
    f = lambda x: "true" if x else "false"
    return f"mla_splitkv_ws_kernel<{rt}, {f(kv == 'fp8')}, {f(sparse)}>"


def run_one(args, key: str, cpu_budget: float) -> dict:
    """Time one workload; returns its JSON line (a dict)."""
    import torch
    import mla_paged_kv_04_amd as mla
    from workloads import WORKLOADS, algorithmic_counts, make_inputs, sparse_counts

    w = WORKLOADS[key]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    fp8 = args.kv == "fp8"
    sparse = w.topk > 0
    if args.launch == "inline" and (sparse or args.graph):
        raise ValueError("--launch inline applies to the eager dense decode")
    if sparse and (args.with_append or args.graph):
        raise ValueError("the sparse workload runs eagerly, without the append")
    inp = make_inputs(key, kv_format=args.kv)
    g = inp.to(dev)
    if sparse:
        counts = sparse_counts(inp.indices, inp.seqlens, inp.s_q, inp.h_q, inp.causal, args.kv)
    else:
        counts = algorithmic_counts(inp.seqlens.tolist(), inp.s_q, inp.h_q, args.kv)
    decode_fn = mla.splitkv_fp8 if fp8 else mla.splitkv
    sparse_fn = mla.sparse_fwd_fp8 if fp8 else mla.sparse_fwd
    append_fn = mla.kv_append_fp8 if fp8 else mla.kv_append

    if sparse:   # (request, token) items of topk entries
        topk = int(inp.indices.shape[2])
        parts = args.parts or mla.num_parts(inp.batch * inp.s_q, 1, inp.h_q, 1,
                                            mla.device_num_cus(dev))
        ws_bytes = mla.sparse_workspace_bytes(inp.batch, inp.s_q, inp.h_q, topk, parts)
    else:
        parts = args.parts or mla.num_parts(inp.batch, inp.s_q, inp.h_q, 1,
                                            mla.device_num_cus(dev))
        ws_bytes = mla.workspace_bytes(inp.batch, inp.s_q, inp.h_q, parts)
    ws = torch.empty((max(256, ws_bytes),), dtype=torch.uint8, device=dev)
    out = torch.empty((inp.batch, inp.s_q, inp.h_q, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((inp.batch, inp.s_q, inp.h_q), dtype=torch.float32, device=dev)
    new_kv = (torch.randn((inp.batch, inp.s_q, 576), generator=torch.Generator().manual_seed(5))
              .to(torch.bfloat16).to(dev)) if args.with_append else None
    flush_buf = torch.ones((1 << 28,), dtype=torch.int32, device=dev)   # 1 GiB
    flush_sink = torch.empty((), dtype=torch.int32, device=dev)

    def flush():
        if args.flush == "read":
            torch.amax(flush_buf, dim=0, out=flush_sink)
        elif args.flush == "write":
            flush_buf.fill_(1)

    # --launch inline: the plan buffers the decode kernel writes (the combine
    # reads split_offsets from them).
    inline_meta = None
    if args.launch == "inline":
        inline_meta = mla.binding.Metadata(
            torch.empty((parts, mla.binding.TILE_META_INTS), dtype=torch.int32, device=dev),
            torch.empty((inp.batch + 1,), dtype=torch.int32, device=dev), parts, inp.s_q,
            inp.h_q)

    # evs: [step start, step end, decode kernel start, decode kernel end]; the
    # last two are recorded by the decode kernel's own launch, so the step's
    # stream carries no marker between its three kernels.
    def step(evs=None):
        if sparse:
            if evs is not None:
                evs[0].record()
            meta = mla.sparse_metadata(inp.batch, inp.s_q, inp.h_q, topk, dev, parts=parts)
            sparse_fn(g.q, g.kcache, g.block_table, g.seqlens, g.indices, inp.scale,
                      inp.causal, meta=meta, workspace=ws, out=out, lse=lse,
                      start_event=evs[2] if evs else None,
                      stop_event=evs[3] if evs else None)
            if evs is not None:
                evs[1].record()
            return
        if evs is not None:
            evs[0].record()
        if new_kv is not None:
            append_fn(new_kv, g.kcache, g.block_table, g.seqlens)
        if inline_meta is not None:
            mla.fwd_inline_plan(g.q, g.kcache, g.block_table, g.seqlens, inp.scale, inp.causal,
                                meta=inline_meta, workspace=ws, out=out, lse=lse,
                                start_event=evs[2] if evs else None,
                                stop_event=evs[3] if evs else None, fp8=fp8)
        else:
            meta = mla.metadata(g.seqlens, inp.s_q, inp.h_q, parts=parts)
            decode_fn(g.q, g.kcache, g.block_table, g.seqlens, inp.scale, inp.causal, meta, ws,
                      out, lse, start_event=evs[2] if evs else None,
                      stop_event=evs[3] if evs else None)
            mla.combine(g.seqlens, inp.s_q, inp.h_q, meta, ws, out, lse)
        if evs is not None:
            evs[1].record()

    # Per-kernel breakdown of the scheduler and the combine (marker events
    # between kernels), in a separate loop after the timed one.
    def step_breakdown(evs):
        if sparse:   # scheduler; resolve + decode + combine
            evs[0].record()
            meta = mla.sparse_metadata(inp.batch, inp.s_q, inp.h_q, topk, dev, parts=parts)
            evs[1].record()
            sparse_fn(g.q, g.kcache, g.block_table, g.seqlens, g.indices, inp.scale,
                      inp.causal, meta=meta, workspace=ws, out=out, lse=lse)
            evs[2].record()
            evs[3].record()
            return
        if new_kv is not None:
            append_fn(new_kv, g.kcache, g.block_table, g.seqlens)
        evs[0].record()
        if inline_meta is not None:   # no scheduler kernel; the merge timed on its own
            evs[1].record()
            mla.fwd_inline_plan(g.q, g.kcache, g.block_table, g.seqlens, inp.scale, inp.causal,
                                meta=inline_meta, workspace=ws, out=out, lse=lse, fp8=fp8)
            evs[2].record()
            mla.combine(g.seqlens, inp.s_q, inp.h_q, inline_meta, ws, out, lse)
            evs[3].record()
            return
        meta = mla.metadata(g.seqlens, inp.s_q, inp.h_q, parts=parts)
        evs[1].record()
        decode_fn(g.q, g.kcache, g.block_table, g.seqlens, inp.scale, inp.causal, meta, ws,
                  out, lse)
        evs[2].record()
        mla.combine(g.seqlens, inp.s_q, inp.h_q, meta, ws, out, lse)
        evs[3].record()

    for _ in range(args.warmup):
        flush()
        step()
    torch.cuda.synchronize(dev)

    # The step captured once as a HIP graph (metadata, decode, combine), as a
    # serving loop would launch it; replays reuse the same buffers.
    graph = None
    if args.graph:
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize(dev)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(args.warmup):
            flush()
            graph.replay()
        torch.cuda.synchronize(dev)

    if args.copy_calib_mib > 0:
        n = args.copy_calib_mib << 18
        src = torch.ones((n,), dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize(dev)
        torch.neg(src, out=dst)
        torch.cuda.synchronize(dev)
        del src, dst

    K = args.steps
    new_events = lambda: [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
                          for _ in range(K)]
    evs = new_events()
    for e in evs:             # create the kernel-timing events before the timed region
        e[2].record()
        e[3].record()
    torch.cuda.synchronize(dev)
    gevs = new_events()
    t_wall0 = time.perf_counter()
    if graph is not None:
        for k in range(K):
            flush()
            gevs[k][0].record()
            graph.replay()
            gevs[k][1].record()
    else:
        for k in range(K):
            flush()
            step(evs[k])
    torch.cuda.synchronize(dev)
    t_wall = time.perf_counter() - t_wall0
    if graph is not None:   # eager steps: the decode kernel's own duration
        for k in range(K):
            flush()
            step(evs[k])
        torch.cuda.synchronize(dev)

    bevs = new_events()
    for k in range(K):
        flush()
        step_breakdown(bevs[k])
    torch.cuda.synchronize(dev)

    eager_ms = [e[0].elapsed_time(e[1]) for e in evs]
    append_ms = None
    if new_kv is not None:
        aevs = new_events()
        for k in range(K):
            flush()
            aevs[k][0].record()
            append_fn(new_kv, g.kcache, g.block_table, g.seqlens)
            aevs[k][1].record()
        torch.cuda.synchronize(dev)
        append_ms = [e[0].elapsed_time(e[1]) for e in aevs]
    step_ms = [e[0].elapsed_time(e[1]) for e in gevs] if graph is not None else eager_ms
    dec_ms = [e[2].elapsed_time(e[3]) for e in evs]
    meta_ms = [e[0].elapsed_time(e[1]) for e in bevs]
    comb_ms = [e[2].elapsed_time(e[3]) for e in bevs]
    mean = lambda xs: sum(xs) / len(xs)
    med = lambda xs: sorted(xs)[len(xs) // 2]
    ms = mean(step_ms)
    gbs = counts["bytes"] / (ms * 1e-3) / 1e9
    tfl = counts["flops"] / (ms * 1e-3) / 1e12
    dec = mean(dec_ms)
    dec_gbs = counts["bytes"] / (dec * 1e-3) / 1e9
    dec_tfl = counts["flops"] / (dec * 1e-3) / 1e12

    # warm back-to-back rate (no flush), for reference only
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K):
        if graph is not None:
            graph.replay()
        else:
            step()
    e1.record()
    torch.cuda.synchronize(dev)
    warm_ms = e0.elapsed_time(e1) / K

    traffic = measured_traffic(key, args.kv)
    # The binding roof of the decode kernel: HBM below the ridge point
    # (peak flops / peak bytes = 312.5 flop/byte), the bf16 MFMA above it.
    mfma_bound = counts["flops"] / counts["bytes"] > PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    line = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": key, "desc": w.desc, "batch": inp.batch,
                   "s_q": inp.s_q, "h_q": inp.h_q, "h_kv": 1, "d_k": 576, "d_v": 512,
                   "block_size": 64, "total_keys": int(inp.seqlens.sum()),
                   "num_parts": parts, "cache_flush_between_steps": args.flush,
                   "step_launch": ("hip_graph" if graph is not None else
                                   "eager, in-kernel plan (decode + combine)"
                                   if inline_meta is not None else "eager"),
                   "kv_append_in_step": new_kv is not None,
                   "kv_cache": ("fp8_e4m3 latent codes, fp32 per-token scale, bf16 rope "
                                "(644 B/token)" if fp8 else "bf16 (1152 B/token)"),
                   "sparse_topk": w.topk or None,
                   "counted_entries": counts.get("counted")},
        "tflops": round(tfl, 2),
        "algorithmic_bytes": counts["bytes"],
        "algorithmic_flops": counts["flops"],
        "kernels_ms": {"metadata": None if inline_meta is not None else round(mean(meta_ms), 5),
                       "splitkv": round(dec, 5),
                       "combine": round(mean(comb_ms), 5),
                       "splitkv_median": round(med(dec_ms), 5),
                       "splitkv_p90": round(sorted(dec_ms)[int(0.9 * (len(dec_ms) - 1))], 5),
                       "step_median": round(med(step_ms), 5),
                       "eager_step": round(mean(eager_ms), 5),
                       "append": round(mean(append_ms), 5) if append_ms else None},
        "warm_ms_per_step": round(warm_ms, 5),
        "wall_s_timed_region": round(t_wall, 4),
        "roofline": {
            "kernel": splitkv_kernel_name(inp.h_q if sparse else inp.s_q * inp.h_q, args.kv,
                                          sparse),
            "bound": "mfma" if mfma_bound else "hbm",
            "achieved": round(dec_tfl if mfma_bound else dec_gbs, 2),
            "peak": PEAK_BF16_TFLOPS if mfma_bound else PEAK_HBM_GBS,
            "unit": "TFLOP/s" if mfma_bound else "GB/s",
            "frac": round(dec_tfl / PEAK_BF16_TFLOPS if mfma_bound else dec_gbs / PEAK_HBM_GBS, 4),
            "arith_intensity": round(counts["flops"] / counts["bytes"], 1),
            "hbm_gbs": round(dec_gbs, 2),
            "hbm_frac": round(dec_gbs / PEAK_HBM_GBS, 4),
            "traffic": (None if traffic is None
                        else traffic["fetch_bytes"] + traffic["write_bytes"]),
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                            "copy-calibrated)",
            "traffic_detail": traffic,
            "mfma_busy": (None if traffic is None else traffic.get("mfma_util")),
            "mfma_busy_source": "rocprofv3 MfmaUtil (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x 1024 SIMDs), profiles/",
            "mfma_tflops": round(dec_tfl, 2),
            "mfma_frac": round(dec_tfl / PEAK_BF16_TFLOPS, 4),
        },
    }
    if not args.no_cpu_baseline and cpu_budget > 0:
        line["cpu_baseline"] = cpu_baseline(inp, cpu_budget)
    del g, ws, out, lse, flush_buf
    torch.cuda.empty_cache()
    return line


# The five configurations of the metric, in order; the last is the headline
# of the default run (the largest single-GPU configuration by bytes).
SUITE = ["tiny", "membound", "ridge", "ragged", "long"]
HEADLINE = "long"


def summary(line: dict) -> dict:
    """The per-configuration figures of a workload's line."""
    r = line["roofline"]
    traffic = r.get("traffic")
    return {
        "ms_per_step": line["ms_per_step"],
        "decode_ms": line["kernels_ms"]["splitkv"],
        "kernels_ms": line["kernels_ms"],
        "step_gbs": line["value"],
        "step_tflops": line["tflops"],
        "decode_gbs": r["hbm_gbs"],
        "decode_tflops": r["mfma_tflops"],
        "hbm_frac": r["hbm_frac"],
        "mfma_frac": r["mfma_frac"],
        "bound": r["bound"],
        "frac": r["frac"],
        "mfma_busy": r.get("mfma_busy"),
        "traffic_ratio": (None if traffic is None
                          else round(traffic / line["algorithmic_bytes"], 4)),
        "algorithmic_bytes": line["algorithmic_bytes"],
        "algorithmic_flops": line["algorithmic_flops"],
        "cpu_baseline": line.get("cpu_baseline"),
        "desc": line["config"]["desc"],
    }


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None,
                    help="tiny | membound | ridge | ragged | long | draft | prefill | sparse; "
                         "default: the five configurations tiny, membound, ridge, ragged, "
                         "long in one run, the line headed by long with a per_config map")
    ap.add_argument("--parts", type=int, default=None, help="override split-KV part count")
    ap.add_argument("--kv", choices=["bf16", "fp8"], default="bf16",
                    help="KV cache format: bf16 rows, or FP8 pages (E4M3 latent codes with a "
                         "per-token fp32 scale, bf16 rope)")
    ap.add_argument("--flush", choices=["read", "write", "none"], default="read",
                    help="cache flush between timed steps (outside the timed events)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="run one plain elementwise copy of this many MiB (int32 -> int32) "
                         "after warmup, outside the timed region: the known-size kernel "
                         "that HBM byte counters are scaled against")
    ap.add_argument("--with-append", action="store_true",
                    help="include the paged-KV append of the step's new tokens "
                         "(mla_kv_append) in every step")
    ap.add_argument("--graph", action="store_true",
                    help="time HIP-graph replays of the step instead of eager launches "
                         "(slower on this stack: replays add ~4-14 us per step)")
    ap.add_argument("--launch", choices=["three", "inline"], default="three",
                    help="three: scheduler, decode and combine kernels; inline: the decode "
                         "kernel derives its split plan itself (mla_decode_fwd_inline_plan), "
                         "two launches per step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle time for the cpu_baseline of the reported workload")
    ap.add_argument("--cpu-budget-each", type=float, default=3.0,
                    help="seconds of oracle time for each other configuration of the default "
                         "run (its per_config cpu_baseline)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the benchmark runs on one GPU only; --gpus above 1 (or a "
              "multi-rank launch) is not supported.", file=sys.stderr)
        return 2
    try:
        if args.workload is not None:
            line = run_one(args, args.workload, args.cpu_budget)
        else:
            lines = {}
            for key in SUITE:
                budget = args.cpu_budget if key == HEADLINE else args.cpu_budget_each
                lines[key] = run_one(args, key, budget)
                print(f"bench.py: {key} done: step {lines[key]['ms_per_step']} ms, decode "
                      f"{lines[key]['kernels_ms']['splitkv']} ms", file=sys.stderr, flush=True)
            line = lines[HEADLINE]
            line["per_config"] = {k: summary(v) for k, v in lines.items()}
    except ValueError as e:
        print(f"bench.py: {e}", file=sys.stderr)
        return 2
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
