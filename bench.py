"""Decode-attention benchmark on one MI355X.

One step = one call of the fused decode attention for the whole batch: the
decode kernel (every K/V byte streamed once, split evenly over the workers)
then the split-merge kernel (log-sum-exp combine of the sequences that several
workers share), on synthetic inputs already resident in HBM.  Inputs are
replicated R = max(2, ceil(1 GiB / bytes)) times and the steps cycle through
the replicas, so the 256 MB Infinity Cache cannot serve a step from the
previous one.

The headline workload (--config, default 4: the largest that the workloads
name) is timed first; then, unless --single, every workload is timed the same
way in the same process and listed in `per_config`.  Per workload:
  us_per_step   K whole calls back to back, events only at the two ends
  kernel_us     K decode-kernel launches back to back (no merge), events at
                the ends: the kernel's duration plus the launch gap, the
                figure a kernel trace compares with
  kernel_us_bracketed  each decode launch between its own events (adds the
                event overhead), and merge_us_bracketed likewise
  read_ceiling_us  a plain streaming read of the same bytes at the decode
                kernel's launch shape and load instruction, with no arithmetic
                (zl_hbm_read_probe): what a read alone reaches at that size
  warm_us_per_step  K whole calls all on the first replica, so that the
                Infinity Cache may serve what fits (secondary, never the
                headline)
Fractions are algorithmic bytes (every K and V element, or every latent row,
read once) / time / 8 TB/s.

Warm-up: at least --warmup calls and at least 0.25 s of them (the clocks
settle only after a fraction of a second of work); `warmup` reports the
calls made.

Prints one JSON line:
  value      KV GB/s of the headline workload = algorithmic bytes / us_per_step
  roofline   the headline's decode kernel against the 8 TB/s HBM peak
             (achieved = bytes / kernel_us); traffic (L2-to-fabric bytes per
             launch, read + written, from request counts) and mfma_busy come
             from the committed rocprofv3 counter record
             (profiles/traffic_<workload>.json) when it was taken on the
             current kernel sources, else null
  cpu_baseline  the fp64 oracle on the host cores, on a bounded sample of the
             headline workload
  per_config every workload, as above
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
# The sources of each mode's kernels: a counter record is used only when it
# was taken on these exact sources.
KERNEL_SOURCES = {
    "decode": ["zl_device.h", "zl_split.h", "zl_tile.h", "zl_kernels.h", "decode_attn.hip", "decode_mla.hip",
               "split_merge.hip"],
    "prefill": ["zl_device.h", "zl_split.h", "zl_tile.h", "zl_kernels.h", "prefill_attn.hip"],
    "codec": ["zl_device.h", "zl_kernels.h", "int8_codec.hip"],
}


def code_only(text: str) -> str:
    """C++ source without its comments and with runs of whitespace collapsed,
    so that the hash below names the code that was measured, not its prose.
    (String literals in these sources hold no comment markers.)"""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_sha(kind: str = "decode", read=None) -> str:
    """Hash of the code of one mode's kernel sources.  read(name) -> text
    (default: the files in mla_attention_amd/csrc)."""
    if read is None:
        def read(name):
            with open(os.path.join(ROOT, "mla_attention_amd", "csrc", name)) as f:
                return f.read()
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        h.update(code_only(read(name)).encode())
    return h.hexdigest()[:16]


def profile_record(workload: str, kind: str = "decode") -> dict:
    """The committed rocprofv3 counter record for this workload (HBM bytes per
    launch, matrix-core busy share), if it was taken on the current kernel
    sources; else an empty dict."""
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != kernel_source_sha(kind):
        return {}
    return rec


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=4, choices=[1, 2, 3, 4, 5],
                    help="headline workload (default 4, the largest: batch 8, 32/8 heads, D 128, every "
                         "sequence 32768 tokens, bf16)")
    ap.add_argument("--single", action="store_true",
                    help="time the headline workload only (default: also every other workload, in per_config)")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the plain-read ceiling beside each workload")
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
    ap.add_argument("--prefill-lens", type=str, default="", metavar="L1,L2,...",
                    help="instead of --prefill / --prefill-batch: whole prompts of these lengths (a ragged batch)")
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
    if args.prefill or args.prefill_lens:
        bench_prefill(args)
        return

    if args.profile_run:
        decode_profile_run(args)
        return

    head = bench_decode(args.config, args)
    spec = head["spec"]
    cpu = None
    if not args.no_cpu and args.q_len == 1:  # (the oracle baseline covers one new token per sequence)
        cpu = cpu_baseline(head["inputs"], spec, args.cpu_seconds)
    per_config = []
    if not args.single:
        for c in sorted(WORKLOAD_IDS):
            per_config.append(head["summary"] if c == args.config else bench_decode(c, args)["summary"])
    workload = head["summary"]["workload"]
    prof = profile_record(workload)
    x = head["inputs"]
    rec = {
        "metric": "decode-attn KV GB/s (algorithmic K+V bytes / step time) and us/step, % of MI355X HBM peak",
        "value": round(head["value_gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": head["summary"]["warmup_calls"],
        "ms_per_step": round(head["ms_per_step"], 5),
        "us_per_step": round(head["ms_per_step"] * 1e3, 2),
        "us_per_call_percentiles": head["spread"],
        "hbm_peak_frac": round(head["value_gbs"] / HBM_PEAK_GBS, 4),
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
            "kv_bytes_per_step": x.kv_bytes(),
            "cold_cache_replicas": head["reps"],
            "workers": args.workers or "default",
            "kv_layout": f"paged, {args.paged}-token pages in a shuffled pool" if args.paged else "packed rows",
            "new_tokens_per_seq": args.q_len,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "mla_decode_kernel" if spec.kind == "mla" else "decode_kernel",
            "achieved": round(head["kernel_gbs"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(head["kernel_gbs"] / HBM_PEAK_GBS, 4),
            "traffic": prof.get("hbm_bytes_per_launch"),
            "avg_launch_us": round(head["kernel_ms"] * 1e3, 2),
            "avg_launch_us_bracketed": round(head["kernel_ms_bracketed"] * 1e3, 2),
            "merge_launch_us": round(head["merge_ms"] * 1e3, 2),
            "mfma_busy": prof.get("mfma_busy_frac"),
            "math_tflops": round(head["flops"] / (head["kernel_ms"] * 1e-3) / 1e12, 2),
            "read_ceiling_us": head["summary"].get("read_ceiling_us"),
        },
        "cpu_baseline": cpu,
        "per_config": per_config,
        "wall_ms_timed_region": round(head["wall_ms"], 2),
    }
    print(json.dumps(rec), flush=True)


WORKLOAD_IDS = (1, 2, 3, 4, 5)


class DecodeRig:
    """Inputs of one workload resident in HBM (R cold-cache replicas of the
    caches), its output and workspace, and one step = one library call."""

    def __init__(self, cfg, args, reps_override=None):
        import torch

        import mla_attention_amd as zl
        import workloads

        self.zl = zl
        self.args = args
        spec = self.spec = workloads.WORKLOADS[cfg]
        dev = self.dev = torch.device("cuda:0")
        x = self.x = workloads.make_inputs(spec)
        self.kv_bytes = x.kv_bytes()
        self.reps = reps_override or max(2, math.ceil((1 << 30) / self.kv_bytes))
        q_len = args.q_len
        self.vq = vq = workloads.make_varlen_query(x, [q_len] * spec.batch, seed=cfg) if q_len > 1 else None
        self.cu = x.cu_seqlens.to(dev)
        self.q = vq.q.to(dev) if vq else x.q.to(dev)
        self.cu_q = vq.cu_q.to(dev) if vq else None
        paged = self.paged = workloads.make_paged(x, args.paged) if args.paged else None
        self.table = paged.block_table.to(dev) if paged else None
        if paged:
            pools = (paged.kv_pages,) if spec.kind == "mla" else (paged.k_pages, paged.v_pages)
            self.caches = [tuple(t.to(dev) for t in pools) for _ in range(self.reps)]
        else:
            self.caches = [(x.latent.to(dev),) if spec.kind == "mla" else (x.k.to(dev), x.v.to(dev))
                           for _ in range(self.reps)]
        if spec.kind == "mla":
            ws_bytes = zl.zl_decode_attn_mla_workspace_size(spec.batch, spec.num_q_heads, 512, 64, x.max_seqlen,
                                                            spec.torch_dtype, args.workers)
        else:
            ws_bytes = zl.zl_decode_attn_workspace_size(spec.batch, spec.num_q_heads, spec.num_kv_heads,
                                                        spec.head_dim_k, x.max_seqlen, spec.torch_dtype,
                                                        args.workers)
        self.ws = zl.new_workspace(ws_bytes, dev)
        rows = self.q.shape[0]
        self.out = torch.empty(rows, spec.num_q_heads, spec.head_dim_v, dtype=spec.torch_dtype, device=dev)
        self.lse = torch.empty(rows, spec.num_q_heads, dtype=torch.float32, device=dev)
        self.stream = torch.cuda.current_stream(dev)
        self.name = spec.name + (f"+paged{args.paged}" if paged else "") + (f"+q{q_len}" if vq else "")

    def step(self, i, phases=3):
        zl, spec, x, a = self.zl, self.spec, self.x, self.args
        c = self.caches[i % self.reps]
        kw = dict(out=self.out, lse=self.lse, workspace=self.ws, num_workers=a.workers, stream=self.stream,
                  phases=phases)
        mla = spec.kind == "mla"
        if self.vq is not None and self.paged is not None:
            if mla:
                zl.zl_attn_varlen_mla_paged(self.q, c[0], self.table, self.cu_q, self.cu, x.max_seqlen, spec.scale,
                                            **kw)
            else:
                zl.zl_attn_varlen_gqa_paged(self.q, c[0], c[1], self.table, self.cu_q, self.cu, x.max_seqlen,
                                            spec.scale, **kw)
        elif self.vq is not None:
            if mla:
                zl.zl_attn_varlen_mla(self.q, c[0], self.cu_q, self.cu, x.max_seqlen, spec.scale, **kw)
            else:
                zl.zl_attn_varlen_gqa(self.q, c[0], c[1], self.cu_q, self.cu, x.max_seqlen, spec.scale, **kw)
        elif self.paged is not None:
            if mla:
                zl.zl_decode_attn_mla_paged(self.q, c[0], self.table, self.cu, x.max_seqlen, spec.scale, **kw)
            else:
                zl.zl_decode_attn_gqa_paged(self.q, c[0], c[1], self.table, self.cu, x.max_seqlen, spec.scale, **kw)
        elif mla:
            zl.zl_decode_attn_mla(self.q, c[0], self.cu, x.max_seqlen, spec.scale, **kw)
        else:
            zl.zl_decode_attn_gqa(self.q, c[0], c[1], self.cu, x.max_seqlen, spec.scale, **kw)


def decode_profile_run(args):
    """A few whole calls only, for rocprofv3 counter passes (no JSON)."""
    import torch

    rig = DecodeRig(args.config, args, reps_override=1)
    n = max(3, args.steps)
    for i in range(n):
        rig.step(i)
    torch.cuda.synchronize()
    print(f"profile run: {rig.name}, {n} launches", flush=True)


# The clocks reach their sustained level only after a fraction of a second of
# work (the prefill measurements below show it for the matrix units; decode
# steps measured right after a few warm-up calls read up to 8% slow).
MIN_WARMUP_S = 0.25


def warm_up(step, W):
    """Run step(i) at least W times and for at least MIN_WARMUP_S seconds;
    returns the number of warm-up calls made."""
    import torch

    t0 = time.perf_counter()
    i = 0
    while i < W or time.perf_counter() - t0 < MIN_WARMUP_S:
        step(i)
        i += 1
        if i >= W and i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return i


def timed_span(stream, fn, K):
    """Milliseconds per call of K back-to-back fn(i) on `stream`, with events
    only at the two ends."""
    import torch

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(K):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / K


def bench_decode(cfg, args):
    """Time one workload: whole calls back to back (the headline), the decode
    kernel alone back to back (its duration for the roofline), each launch
    between its own events, per-call spread, and the read ceiling."""
    import numpy as np
    import torch

    rig = DecodeRig(cfg, args)
    spec, x, stream = rig.spec, rig.x, rig.stream
    K = args.steps
    W = warm_up(rig.step, args.warmup)

    # Timed region: K whole calls (decode kernel + merge kernel), back to back
    # on the launch stream, events only at the two ends.
    t0 = time.perf_counter()
    ms_per_step = timed_span(stream, lambda i: rig.step(W + i), K)
    wall_ms = (time.perf_counter() - t0) * 1e3

    # The decode kernel alone: K launches back to back (each leaves its
    # partials in the workspace; the next overwrites them), events at the
    # ends: its average duration plus the gap between launches, as close to a
    # kernel trace as events on the launch stream get.
    kernel_ms = timed_span(stream, lambda i: rig.step(W + K + i, phases=1), K)

    # Each launch between its own events (these add the event overhead).
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        ev[i][0].record(stream)
        rig.step(W + 2 * K + i, phases=1)
        ev[i][1].record(stream)
        rig.step(W + 2 * K + i, phases=2)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    kern_br = float(np.mean([ev[i][0].elapsed_time(ev[i][1]) for i in range(K)]))
    merge_ms = float(np.mean([ev[i][1].elapsed_time(ev[i][2]) for i in range(K)]))

    # Per-call spread: K more whole calls, each between two events.
    evc = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        evc[i][0].record(stream)
        rig.step(W + 3 * K + i)
        evc[i][1].record(stream)
    torch.cuda.synchronize()
    per_call_us = np.array([a.elapsed_time(b) * 1e3 for a, b in evc])
    spread = {"p10": round(float(np.percentile(per_call_us, 10)), 2),
              "p50": round(float(np.percentile(per_call_us, 50)), 2),
              "p90": round(float(np.percentile(per_call_us, 90)), 2)}

    # Secondary, warm: K more whole calls all on the first replica, so that
    # the 256 MB MALL may serve what fits of it (never the headline).
    warm_ms = timed_span(stream, lambda i: rig.step(0), K)

    kv = rig.kv_bytes
    summary = {
        "config": cfg,
        "workload": rig.name,
        "dtype": spec.dtype,
        "kv_bytes": kv,
        "us_per_step": round(ms_per_step * 1e3, 2),
        "step_frac": round(kv / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "kernel_us": round(kernel_ms * 1e3, 2),
        "kernel_frac": round(kv / (kernel_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "kernel_us_bracketed": round(kern_br * 1e3, 2),
        "kernel_frac_bracketed": round(kv / (kern_br * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "merge_us_bracketed": round(merge_ms * 1e3, 2),
        "warm_us_per_step": round(warm_ms * 1e3, 2),
        "warmup_calls": W,
    }
    if not args.no_read_ceiling and rig.paged is None and rig.vq is None:
        summary.update(read_ceiling(rig, K, W))
    del rig.caches
    torch.cuda.empty_cache()
    flops = 2.0 * x.total_tokens * spec.num_q_heads * (spec.head_dim_k + spec.head_dim_v) * args.q_len
    return {"spec": spec, "inputs": x, "reps": rig.reps, "ms_per_step": ms_per_step, "wall_ms": wall_ms,
            "value_gbs": kv / (ms_per_step * 1e-3) / 1e9, "kernel_ms": kernel_ms, "kernel_ms_bracketed": kern_br,
            "kernel_gbs": kv / (kernel_ms * 1e-3) / 1e9, "merge_ms": merge_ms, "spread": spread,
            "flops": flops, "summary": summary}


def read_ceiling(rig, K, W):
    """A plain streaming read of the same byte count at the decode kernel's
    launch shape (zl_hbm_read_probe: its load instruction and ring, no
    arithmetic), cold-cache replicas as for the decode steps."""
    import torch

    zl, spec = rig.zl, rig.spec
    nbytes = rig.kv_bytes // 1024 * 1024
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device=rig.dev) for _ in range(rig.reps)]
    for b in bufs:
        b.fill_(1)
    wg = rig.args.workers or {64: 1536, 128: 768, 576: 256}[spec.head_dim_k]
    sink = torch.empty(wg, dtype=torch.int32, device=rig.dev)

    def rd(i):
        zl.zl_hbm_read_probe(bufs[i % rig.reps], spec.head_dim_k, workgroups=rig.args.workers, sink=sink,
                             stream=rig.stream)
    for i in range(W):
        rd(i)
    ms = timed_span(rig.stream, lambda i: rd(W + i), K)
    del bufs
    return {"read_ceiling_us": round(ms * 1e3, 2),
            "read_ceiling_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "read_ceiling_workgroups": wg}


MFMA_PEAK_TFLOPS = 2500.0  # dense fp16 / bf16


def bench_prefill(args):
    """Whole prompts through the prefill kernel.  Useful flops: QK^T and PV over
    the causal triangle, 2 * 2 * Hq * D * L (L + 1) / 2 per prompt."""
    import numpy as np
    import torch

    import mla_attention_amd as zl
    import workloads

    spec0 = workloads.WORKLOADS[args.config]
    lens = [int(t) for t in args.prefill_lens.split(",")] if args.prefill_lens else [args.prefill] * args.prefill_batch
    B, L = len(lens), max(lens)
    spec = workloads.with_shape(spec0, batch=B, lens=tuple(lens))
    dev = torch.device("cuda:0")
    x = workloads.make_inputs(spec)
    vq = workloads.make_varlen_query(x, lens, seed=args.config)
    q = vq.q.to(dev)
    cq, ck = vq.cu_q.to(dev), x.cu_seqlens.to(dev)
    if args.paged:
        px = workloads.make_paged(x, args.paged)
        k, v, table = px.k_pages.to(dev), px.v_pages.to(dev), px.block_table.to(dev)
    else:
        k, v = x.k.to(dev), x.v.to(dev)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev)
    flops = sum(4.0 * spec.num_q_heads * spec.head_dim_k * n * (n + 1) / 2 for n in lens)
    ragged = len(set(lens)) > 1

    def step(i):
        if args.paged:
            zl.zl_attn_prefill_gqa_paged(q, k, v, table, cq, ck, L, spec.scale, out=out, stream=stream)
        else:
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
    workload = ((f"prefill-ragged-b{B}-Lmax{L}" if ragged else f"prefill-b{B}-L{L}") +
                f"-h{spec.num_q_heads}kv{spec.num_kv_heads}-d{spec.head_dim_k}-{spec.dtype}" +
                (f"+paged{args.paged}" if args.paged else ""))
    prof = profile_record(workload, "prefill")
    cpu = None if args.no_cpu else cpu_baseline_prefill(x, vq, spec, flops, args.cpu_seconds)
    print(json.dumps({
        "metric": "prefill attention TFLOP/s (useful causal QK^T + PV flops / step time)",
        "value": round(tf, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16" if spec.dtype == "f16" else "bf16", "data": "synthetic (seeded N(0,1) Q/K/V)",
        "config": {"workload": workload,
                   "batch": B, "prompt_len": lens if ragged else L, "num_q_heads": spec.num_q_heads,
                   "num_kv_heads": spec.num_kv_heads, "head_dim": spec.head_dim_k, "causal": True},
        "roofline": {"bound": "mfma", "kernel": "prefill_kernel", "achieved": round(tf, 1),
                     "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / MFMA_PEAK_TFLOPS, 4),
                     "traffic": prof.get("hbm_bytes_per_launch"), "mfma_busy": prof.get("mfma_busy_frac")},
        "cpu_baseline": cpu}), flush=True)


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
    workload = f"codec-{args.codec}-{args.codec_mib}MiB-fp16-chunk{C}"
    prof = profile_record(workload, "codec")
    cpu = None if args.no_cpu else cpu_baseline_codec(args.codec, base, C, per_call / n, args.cpu_seconds)
    print(json.dumps({
        "metric": f"INT8 all-reduce payload codec ({args.codec}) GB/s of algorithmic bytes",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16->i8", "data": "synthetic (seeded N(0,1) fp16 payload)",
        "config": {"workload": workload, "elements": n,
                   "bytes_per_call": per_call, "cold_cache_replicas": reps},
        "roofline": {"bound": "hbm", "kernel": "codec_kernel", "achieved": round(kgbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(kgbs / HBM_PEAK_GBS, 4),
                     "traffic": prof.get("hbm_bytes_per_launch"),
                     "avg_launch_us": round(kern_ms * 1e3, 2)},
        "cpu_baseline": cpu}), flush=True)


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


def cpu_baseline_prefill(x, vq, spec, flops_per_step: float, target_s: float):
    """The fp64 oracle on a bounded sample of the prefill's query rows: every
    (new token, head) pair of a strided grid (about 256 tokens by 8 heads),
    repeated for about target_s seconds on all host cores; reported in the
    metric's unit (useful causal flops of the sample per second)."""
    import numpy as np
    import torch

    import oracle

    threads = oracle.max_threads()
    dt = oracle.F16 if spec.dtype == "f16" else oracle.BF16
    cq, ck = vq.cu_q.numpy(), x.cu_seqlens.numpy()
    Tq, Hq, D = vq.total_q, spec.num_q_heads, spec.head_dim_k
    rows = [(t, h) for t in range(0, Tq, max(1, Tq // 256)) for h in range(0, Hq, max(1, Hq // 8))]
    seq = np.searchsorted(cq, np.arange(Tq), side="right") - 1
    flops = 0.0
    for t, _ in rows:  # keys seen by new token i of nq over a cache of lk rows: lk - nq + i + 1
        b = seq[t]
        nq, lk = int(cq[b + 1] - cq[b]), int(ck[b + 1] - ck[b])
        flops += 4.0 * D * max(0, lk - nq + (t - int(cq[b])) + 1)
    qb = vq.q.contiguous().view(torch.int16).numpy().view(np.uint16)
    kb, vb = x.bits("k"), x.bits("v")
    elapsed, calls = 0.0, 0
    while elapsed < target_s or calls == 0:
        t0 = time.perf_counter()
        oracle.gqa_varlen(qb, kb, vb, cq, ck, spec.num_kv_heads, spec.scale, dt, causal=True, rows=rows,
                          threads=threads)
        elapsed += time.perf_counter() - t0
        calls += 1
    rate = flops * calls / elapsed
    return {
        "value": round(rate / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{len(rows)} (new token, head) rows of this prefill on a strided grid, {flops:.4g} useful "
                  f"flops, through the fp64 C oracle {calls} times on {threads} threads, {elapsed:.1f} s",
        "us_per_step_equiv": round(flops_per_step / rate * 1e6, 1),
    }


def cpu_baseline_codec(mode: str, base, chunk: int, bytes_per_elem: float, target_s: float):
    """The numpy codec oracle (one core) on the first 4 Mi elements of the same
    payload, repeated for about target_s seconds; reported in the metric's
    unit (algorithmic bytes per second)."""
    import numpy as np
    import torch

    import oracle
    from oracle import codec

    n = min(base.numel(), 1 << 22)
    n -= n % chunk
    bits = base[:n].contiguous().view(torch.int16).numpy().view(np.uint16)
    codes, scales = codec.quantize(bits, oracle.F16, chunk)
    elapsed, calls = 0.0, 0
    while elapsed < target_s or calls == 0:
        t0 = time.perf_counter()
        if mode == "quantize":
            codec.quantize(bits, oracle.F16, chunk)
        elif mode == "dequantize":
            codec.dequantize(codes, scales, chunk, oracle.F16)
        else:
            codec.reduce_step(codes, scales, bits, oracle.F16, chunk)
        elapsed += time.perf_counter() - t0
        calls += 1
    return {
        "value": round(bytes_per_elem * n * calls / elapsed / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"the codec oracle (numpy) on the payload's first {n} fp16 values, {calls} calls, {elapsed:.1f} s",
    }


if __name__ == "__main__":
    main()
