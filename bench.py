"""Decode-attention benchmark on one MI355X.

One step = one call of the fused decode attention for the whole batch: the
decode kernel (every K/V byte streamed once, split evenly over the workers)
then the split-merge kernel (log-sum-exp combine of the sequences that several
workers share), on synthetic inputs already resident in HBM.  The timed region
is K such calls back to back; a second pass of K calls with an event around
each kernel gives the decode kernel's own duration for the roofline.  Inputs are replicated
R = max(2, ceil(1 GiB / bytes)) times and the steps cycle through the
replicas, so the 256 MB Infinity Cache cannot serve a step from the previous
one.

Prints one JSON line:
  value      KV GB/s = algorithmic bytes (every K and V element, or every
             latent row, read once) / time per step
  roofline   the decode kernel against the 8 TB/s HBM peak; achieved = the
             same bytes / the kernel's average duration, from HIP events
             recorded around every launch on the launch stream (these include
             the launch's dispatch, about 2 us more than a kernel trace shows);
             traffic and mfma_busy come from the committed rocprofv3 counter
             record when it was taken on the current kernel sources
  cpu_baseline  the fp64 oracle on the host cores, on a bounded sample
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

HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["zl_device.h", "zl_split.h", "zl_tile.h", "zl_kernels.h", "decode_attn.hip",
                  "decode_mla.hip", "split_merge.hip"]


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "mla_attention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profile_record(workload: str) -> dict:
    """The committed rocprofv3 counter record for this workload (HBM bytes per
    launch, matrix-core busy share), if it was taken on the current kernel
    sources; else an empty dict."""
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != kernel_source_sha():
        return {}
    return rec


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5],
                    help="workload (default 2: batch 32, 32/8 heads, D 128, ragged 512..4096)")
    ap.add_argument("--workers", type=int, default=0, help="decode workers (0 = library default)")
    ap.add_argument("--q-len", type=int, default=1, metavar="N",
                    help="new query tokens per sequence (N > 1: draft tokens checked in one step, "
                         "causal among themselves, through the several-new-tokens entry points)")
    ap.add_argument("--codec", choices=["quantize", "dequantize", "reduce"], default=None,
                    help="instead: time the INT8 all-reduce payload codec kernel on --codec-mib of fp16 payload")
    ap.add_argument("--codec-mib", type=int, default=64)
    ap.add_argument("--prefill", type=int, default=0, metavar="LEN",
                    help="instead: time the prefill kernel on --prefill-batch whole prompts of LEN tokens "
                         "(heads, head dim and dtype of --config), causal")
    ap.add_argument("--prefill-batch", type=int, default=4)
    ap.add_argument("--codec-chunk", type=int, default=512)
    ap.add_argument("--paged", type=int, default=0, metavar="PAGE_SIZE",
                    help="read the caches from a shuffled page pool through a block table "
                         "(pages of PAGE_SIZE tokens; 0 = packed rows)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target host time of the oracle sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--profile-run", action="store_true",
                    help="a few launches only (for rocprofv3 counter passes); no JSON")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead: copy a MIB-sized buffer a few times with a plain device copy "
                         "(the reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return ap.parse_args()


def copy_calibration(mib: int, launches: int):
    import torch

    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(launches):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copy calibration: {launches} copies of {n} bytes", flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "bench.py measures one GPU: the decode kernel runs on one GPU's share of "
                                   "the batch (sharding across GPUs is a design note, not a code path)",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration, max(3, args.steps))
        return
    if args.codec:
        bench_codec(args)
        return
    if args.prefill:
        bench_prefill(args)
        return

    import numpy as np
    import torch

    import mla_attention_amd as zl
    import workloads

    spec = workloads.WORKLOADS[args.config]
    dev = torch.device("cuda:0")
    x = workloads.make_inputs(spec)
    kv_bytes = x.kv_bytes()
    reps = max(2, math.ceil((1 << 30) / kv_bytes))
    if args.profile_run:
        reps = 1
    vq = workloads.make_varlen_query(x, [args.q_len] * spec.batch, seed=args.config) if args.q_len > 1 else None
    cu = x.cu_seqlens.to(dev)
    q = vq.q.to(dev) if vq else x.q.to(dev)
    cu_q = vq.cu_q.to(dev) if vq else None
    paged = workloads.make_paged(x, args.paged) if args.paged else None
    table = paged.block_table.to(dev) if paged else None
    if paged:
        pools = (paged.kv_pages,) if spec.kind == "mla" else (paged.k_pages, paged.v_pages)
        caches = [tuple(t.to(dev) for t in pools) for _ in range(reps)]
    else:
        caches = [(x.latent.to(dev),) if spec.kind == "mla" else (x.k.to(dev), x.v.to(dev))
                  for _ in range(reps)]
    if spec.kind == "mla":
        ws_bytes = zl.zl_decode_attn_mla_workspace_size(spec.batch, spec.num_q_heads, 512, 64,
                                                        x.max_seqlen, spec.torch_dtype, args.workers)
    else:
        ws_bytes = zl.zl_decode_attn_workspace_size(spec.batch, spec.num_q_heads, spec.num_kv_heads,
                                                    spec.head_dim_k, x.max_seqlen, spec.torch_dtype,
                                                    args.workers)
    ws = zl.new_workspace(ws_bytes, dev)
    rows = q.shape[0]
    out = torch.empty(rows, spec.num_q_heads, spec.head_dim_v, dtype=spec.torch_dtype, device=dev)
    lse = torch.empty(rows, spec.num_q_heads, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i, phases=3):
        c = caches[i % reps]
        if vq is not None and paged and spec.kind == "mla":
            zl.zl_attn_varlen_mla_paged(q, c[0], table, cu_q, cu, x.max_seqlen, spec.scale, out=out, lse=lse,
                                        workspace=ws, num_workers=args.workers, stream=stream, phases=phases)
        elif vq is not None and paged:
            zl.zl_attn_varlen_gqa_paged(q, c[0], c[1], table, cu_q, cu, x.max_seqlen, spec.scale, out=out,
                                        lse=lse, workspace=ws, num_workers=args.workers, stream=stream,
                                        phases=phases)
        elif vq is not None and spec.kind == "mla":
            zl.zl_attn_varlen_mla(q, c[0], cu_q, cu, x.max_seqlen, spec.scale, out=out, lse=lse, workspace=ws,
                                  num_workers=args.workers, stream=stream, phases=phases)
        elif vq is not None:
            zl.zl_attn_varlen_gqa(q, c[0], c[1], cu_q, cu, x.max_seqlen, spec.scale, out=out, lse=lse,
                                  workspace=ws, num_workers=args.workers, stream=stream, phases=phases)
        elif paged and spec.kind == "mla":
            zl.zl_decode_attn_mla_paged(q, c[0], table, cu, x.max_seqlen, spec.scale, out=out, lse=lse,
                                        workspace=ws, num_workers=args.workers, stream=stream, phases=phases)
        elif paged:
            zl.zl_decode_attn_gqa_paged(q, c[0], c[1], table, cu, x.max_seqlen, spec.scale, out=out, lse=lse,
                                        workspace=ws, num_workers=args.workers, stream=stream, phases=phases)
        elif spec.kind == "mla":
            zl.zl_decode_attn_mla(q, c[0], cu, x.max_seqlen, spec.scale, out=out, lse=lse, workspace=ws,
                                  num_workers=args.workers, stream=stream, phases=phases)
        else:
            zl.zl_decode_attn_gqa(q, c[0], c[1], cu, x.max_seqlen, spec.scale, out=out, lse=lse,
                                  workspace=ws, num_workers=args.workers, stream=stream, phases=phases)

    if args.profile_run:
        for i in range(max(3, args.steps)):
            step(i)
        torch.cuda.synchronize()
        print(f"profile run: {spec.name}{' paged' if paged else ''}, {max(3, args.steps)} launches", flush=True)
        return

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: K whole calls (decode kernel + merge kernel), back to back
    # on the launch stream, events only at the two ends.
    K = args.steps
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(K):
        step(args.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ms_per_step = ev0.elapsed_time(ev1) / K
    value_gbs = kv_bytes / (ms_per_step * 1e-3) / 1e9

    # Per-kernel pass for the roofline: the same K steps with the two phases
    # of each call enqueued separately and an event around each launch.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        ev[i][0].record(stream)
        step(args.warmup + K + i, phases=1)
        ev[i][1].record(stream)
        step(args.warmup + K + i, phases=2)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    kern_ms = float(np.mean([ev[i][0].elapsed_time(ev[i][1]) for i in range(K)]))
    merge_ms = float(np.mean([ev[i][1].elapsed_time(ev[i][2]) for i in range(K)]))
    achieved_gbs = kv_bytes / (kern_ms * 1e-3) / 1e9

    # Per-call spread: K more whole calls, each between two events (the
    # events add a little to each interval; the headline is the span above).
    evc = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        evc[i][0].record(stream)
        step(args.warmup + 2 * K + i)
        evc[i][1].record(stream)
    torch.cuda.synchronize()
    per_call_us = np.array([a.elapsed_time(b) * 1e3 for a, b in evc])
    spread = {"p10": round(float(np.percentile(per_call_us, 10)), 2),
              "p50": round(float(np.percentile(per_call_us, 50)), 2),
              "p90": round(float(np.percentile(per_call_us, 90)), 2)}
    workload = spec.name + (f"+paged{args.paged}" if paged else "") + (f"+q{args.q_len}" if vq else "")
    prof = profile_record(workload)

    cpu = None
    if not args.no_cpu and vq is None:  # (the oracle baseline covers one new token per sequence)
        cpu = cpu_baseline(x, spec, args.cpu_seconds)

    # Useful matrix flops of one step: QK^T and PV, 2 flops per multiply-add.
    flops = 2.0 * x.total_tokens * spec.num_q_heads * (spec.head_dim_k + spec.head_dim_v) * args.q_len
    rec = {
        "metric": "decode-attn KV GB/s (algorithmic K+V bytes / step time) and us/step, % of MI355X HBM peak",
        "value": round(value_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "us_per_call_percentiles": spread,
        "hbm_peak_frac": round(value_gbs / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if spec.dtype == "f16" else "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V, ragged lengths; no dataset or weights)",
        "config": {
            "workload": workload,
            "batch": spec.batch,
            "num_q_heads": spec.num_q_heads,
            "num_kv_heads": spec.num_kv_heads,
            "head_dim_k": spec.head_dim_k,
            "head_dim_v": spec.head_dim_v,
            "ctx_lens": list(spec.lens) if not isinstance(spec.lens[0], str) else
            f"uniform[{spec.lens[1]},{spec.lens[2]}] seed {spec.seed}",
            "total_tokens": x.total_tokens,
            "kv_bytes_per_step": kv_bytes,
            "cold_cache_replicas": reps,
            "workers": args.workers or "default",
            "kv_layout": f"paged, {args.paged}-token pages in a shuffled pool" if paged else "packed rows",
            "new_tokens_per_seq": args.q_len,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "mla_decode_kernel" if spec.kind == "mla" else "decode_kernel",
            "achieved": round(achieved_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
            "traffic": prof.get("hbm_bytes_per_launch"),
            "avg_launch_us": round(kern_ms * 1e3, 2),
            "merge_launch_us": round(merge_ms * 1e3, 2),
            "mfma_busy": prof.get("mfma_busy_frac"),
            "math_tflops": round(flops / (kern_ms * 1e-3) / 1e12, 2),
        },
        "cpu_baseline": cpu,
        "wall_ms_timed_region": round(wall_ms, 2),
    }
    print(json.dumps(rec), flush=True)


MFMA_PEAK_TFLOPS = 2500.0  # dense fp16 / bf16


def bench_prefill(args):
    """Whole prompts through the prefill kernel.  Useful flops: QK^T and PV over
    the causal triangle, 2 * 2 * Hq * D * L (L + 1) / 2 per prompt."""
    import numpy as np
    import torch

    import mla_attention_amd as zl
    import workloads

    spec0 = workloads.WORKLOADS[args.config]
    L, B = args.prefill, args.prefill_batch
    spec = workloads.with_shape(spec0, batch=B, lens=tuple([L] * B))
    dev = torch.device("cuda:0")
    x = workloads.make_inputs(spec)
    vq = workloads.make_varlen_query(x, [L] * B, seed=args.config)
    q, k, v = vq.q.to(dev), x.k.to(dev), x.v.to(dev)
    cq, ck = vq.cu_q.to(dev), x.cu_seqlens.to(dev)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev)
    flops = 4.0 * spec.num_q_heads * spec.head_dim_k * B * L * (L + 1) / 2

    def step(i):
        zl.zl_attn_prefill_gqa(q, k, v, cq, ck, L, spec.scale, out=out, stream=stream)

    if args.profile_run:
        for i in range(max(3, args.steps)):
            step(i)
        torch.cuda.synchronize()
        print(f"profile run: prefill {B} x {L}, {max(3, args.steps)} launches", flush=True)
        return
    # The matrix units' clocks settle only after about 0.2 s of sustained
    # work (measured: 3 warm-up launches give 19% less than 300), so the
    # prefill timing warms up for at least 300 launches.
    W = max(args.warmup, 300)
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(K):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    tf = flops / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "prefill attention TFLOP/s (useful causal QK^T + PV flops / step time)",
        "value": round(tf, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16" if spec.dtype == "f16" else "bf16", "data": "synthetic (seeded N(0,1) Q/K/V)",
        "config": {"workload": f"prefill-b{B}-L{L}-h{spec.num_q_heads}kv{spec.num_kv_heads}-d{spec.head_dim_k}",
                   "batch": B, "prompt_len": L, "num_q_heads": spec.num_q_heads,
                   "num_kv_heads": spec.num_kv_heads, "head_dim": spec.head_dim_k, "causal": True},
        "roofline": {"bound": "mfma", "kernel": "prefill_kernel", "achieved": round(tf, 1),
                     "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / MFMA_PEAK_TFLOPS, 4),
                     "traffic": None},
        "cpu_baseline": None}), flush=True)


def bench_codec(args):
    """One codec kernel on a cold payload: the same K steps protocol; bytes are
    the arrays the kernel must read and write once (16-bit values, codes, one
    fp32 scale per chunk)."""
    import numpy as np
    import torch

    import mla_attention_amd as zl

    dev = torch.device("cuda:0")
    n = (args.codec_mib << 20) // 2
    C = args.codec_chunk
    nch = (n + C - 1) // C
    per_call = {"quantize": 3 * n + 4 * nch, "dequantize": 3 * n + 4 * nch, "reduce": 6 * n + 8 * nch}[args.codec]
    reps = max(2, math.ceil((1 << 30) / per_call))
    if args.profile_run:
        reps = 1
    g = torch.Generator(device="cpu").manual_seed(0)
    base = torch.randn(n, generator=g).to(torch.float16)
    xs = [base.to(dev) for _ in range(reps)]
    codes0, scales0 = zl.zl_int8_quantize(xs[0], chunk=C)
    codes = [codes0.clone() for _ in range(reps)]
    scales = [scales0.clone() for _ in range(reps)]
    outs = [torch.empty(n, dtype=torch.float16, device=dev) for _ in range(reps)]
    co = [torch.empty(n, dtype=torch.int8, device=dev) for _ in range(reps)]
    so = [torch.empty(nch, dtype=torch.float32, device=dev) for _ in range(reps)]
    stream = torch.cuda.current_stream(dev)

    def step(i):
        j = i % reps
        if args.codec == "quantize":
            zl.zl_int8_quantize(xs[j], chunk=C, codes=co[j], scales=so[j], stream=stream)
        elif args.codec == "dequantize":
            zl.zl_int8_dequantize(codes[j], scales[j], dtype=torch.float16, chunk=C, out=outs[j], stream=stream)
        else:
            zl.zl_int8_reduce_step(codes[j], scales[j], xs[j], chunk=C, codes_out=co[j], scales_out=so[j],
                                   sum_out=outs[j], stream=stream)

    if args.profile_run:
        for i in range(max(3, args.steps)):
            step(i)
        torch.cuda.synchronize()
        print(f"profile run: codec {args.codec}, {max(3, args.steps)} launches", flush=True)
        return
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(K):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    for i in range(K):
        ev[i][0].record(stream)
        step(args.warmup + K + i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    kern_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    gbs = per_call / (ms * 1e-3) / 1e9
    kgbs = per_call / (kern_ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": f"INT8 all-reduce payload codec ({args.codec}) GB/s of algorithmic bytes",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16->i8", "data": "synthetic (seeded N(0,1) fp16 payload)",
        "config": {"workload": f"codec-{args.codec}-{args.codec_mib}MiB-fp16-chunk{C}", "elements": n,
                   "bytes_per_call": per_call, "cold_cache_replicas": reps},
        "roofline": {"bound": "hbm", "kernel": "codec_kernel", "achieved": round(kgbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(kgbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "avg_launch_us": round(kern_ms * 1e3, 2)},
        "cpu_baseline": None}), flush=True)


def cpu_baseline(x, spec, target_s: float):
    """The fp64 oracle over whole sequences of the same batch, on all host
    cores (about target_s seconds of work), then on one core (a third of
    that); reported in the metric's unit (KV GB/s of the sample)."""
    import oracle

    rec = oracle_rate(x, spec, target_s, oracle.max_threads())
    one = oracle_rate(x, spec, target_s / 3, 1)
    rec["single_core"] = {"value": one["value"], "unit": one["unit"], "cores": 1, "sample": one["sample"]}
    return rec


def oracle_rate(x, spec, target_s: float, threads: int):
    import numpy as np

    import oracle

    cu = x.cu_seqlens.numpy()
    dt = oracle.F16 if spec.dtype == "f16" else oracle.BF16
    row_bytes = (spec.head_dim_k * 2 if spec.kind == "mla"
                 else 2 * spec.num_kv_heads * spec.head_dim_k * 2)
    q = x.bits("q")
    done_bytes, elapsed, nseq, passes = 0, 0.0, 0, 0
    order = list(range(spec.batch))
    while elapsed < target_s and passes < 100:
        for b in order:
            a, e = int(cu[b]), int(cu[b + 1])
            sub = np.array([0, e - a], dtype=np.int32)
            t = time.perf_counter()
            if spec.kind == "mla":
                oracle.mla_decode(q[b:b + 1], x.bits("latent")[a:e], sub, spec.scale, dt, threads=threads)
            else:
                oracle.gqa_decode(q[b:b + 1], x.bits("k")[a:e], x.bits("v")[a:e], sub, spec.num_kv_heads,
                                  spec.scale, dt, threads=threads)
            elapsed += time.perf_counter() - t
            done_bytes += (e - a) * row_bytes
            nseq += 1
            if elapsed >= target_s:
                break
        passes += 1
    return {
        "value": round(done_bytes / elapsed / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{nseq} whole sequences of this batch (all {spec.num_q_heads} query heads each, "
                  f"{done_bytes} KV bytes) through the fp64 C oracle, OpenMP over heads on {threads} "
                  f"thread{'s' if threads > 1 else ''}, {elapsed:.1f} s",
        "us_per_step_equiv": round(x.kv_bytes() / (done_bytes / elapsed) * 1e6, 1),
    }


if __name__ == "__main__":
    main()
