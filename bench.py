#!/usr/bin/env python3
"""Benchmark of the paged-attention path on one MI355X.

Headline (one JSON line on stdout): decode tokens/s and KV GB/s (fraction of
the 8 TB/s HBM peak) for batched GQA decode, B=64, sq=1, Hq=32, Hkv=8, D=128,
page_size=16, seq_lens uniform in [512, 8192]; plus the sq=16 query block's
MFMA utilisation (B=32, sq=16, seq_lens uniform in [1024, 32768]).

A step is one paged_attn_run call (partial pass + Split-KV combine when the
library splits) on inputs already resident in HBM.  The dominant kernel (the
attention partial pass) is also timed alone, in the same launch
configuration, with HIP events on the launch stream; its algorithmic bytes
per launch are the visible K/V bytes: sum_b L'_b * Hkv * 2 * D * 2.

The "kv_write" entry times paged_kv_write (new K/V rows scattered into the
page cache, bf16 and fp8) for a 65536-token prefill chunk and a 64-token
decode step; its bytes are the rows read plus the slot rows written.

Every other configuration (the tiny decode, the windowed and causal sq=16 blocks, the
fp8-query block, long-context Split-KV in bf16 and fp8, the DASH segments fused and
two-stage) is timed after the headline in the same run, each with the fp64 oracle
timed beside it on the host over a bounded sample ("workloads" in the JSON line).

    python bench.py [--steps K] [--warmup W] [--headline-only] [--no-cpu-baseline]
                    [--no-kv-write] [--cpu-seconds S] [--cpu-seconds-other S]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode tokens/s and KV GB/s (% of HBM peak) at B=64,Hkv=8,D=128; sq=16 MFMA %"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
BF16_DENSE_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
KERNEL_SOURCES = ["pa_attention.hip", "pa_device.h", "pa_plan.h", "pa_kernels.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "segmented_attention_paged_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_counters(workload: str):
    """HBM traffic per launch recorded by rocprofv3 --pmc runs for this kernel source, or None."""
    path = os.path.join(ROOT, "profiles", f"attn_kernel_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for ln in open(path):
        if "=" in ln and not ln.startswith("#"):
            k, v = ln.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_src_sha256") != kernel_sha():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def time_events(fn, steps: int, warmup: int, flush=None, rounds: int = 1):
    """ms per call on the current stream (HIP events); optional cache flush between calls.

    Back to back: the average over `steps` calls, and with rounds > 1 the median of
    `rounds` such averages.  With a flush each call is timed alone between its own
    events and the median call is returned (rounds is then ignored).  Medians keep a
    stall of the launching host thread out of a kernel's figure."""
    import statistics

    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    if flush is None:
        avgs, walls = [], []
        for _ in range(rounds):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            s.record()
            for _ in range(steps):
                fn()
            e.record()
            torch.cuda.synchronize()
            walls.append((time.perf_counter() - t0) * 1e3 / steps)
            avgs.append(s.elapsed_time(e) / steps)
        return statistics.median(avgs), statistics.median(walls)
    per_call = []
    t0 = time.perf_counter()
    for _ in range(steps):
        flush()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        torch.cuda.synchronize()
        per_call.append(s.elapsed_time(e))
    return statistics.median(per_call), (time.perf_counter() - t0) * 1e3 / steps


_FLUSH = {}


def mall_flush(nbytes: int, force: bool = False):
    """A 512 MB read run between timed calls when a call touches less than 1 GiB (or
    always, with force), so its data is not served from the 256 MB Infinity Cache; None
    otherwise.  A read, not a fill: a fill leaves dirty lines whose write-back the timed
    call would pay for."""
    import torch

    if nbytes >= (1 << 30) and not force:
        return None
    if "buf" not in _FLUSH:
        _FLUSH["buf"] = torch.ones(1 << 26, dtype=torch.int64, device="cuda")
        _FLUSH["sum"] = torch.empty((), dtype=torch.int64, device="cuda")
    buf, acc = _FLUSH["buf"], _FLUSH["sum"]
    return lambda: torch.sum(buf, dim=0, out=acc)


class PagedBench:
    """Preallocated buffers and closures for one paged workload."""

    def __init__(self, name: str, num_splits=None, causal: bool = False):
        import torch

        import segmented_attention_paged_amd as sap
        from workloads import paged_config

        self.sap = sap
        self.inp = inp = paged_config(name, device="cuda")
        self.name = name
        self.causal = causal
        self.k, self.v = sap.kv_halves(inp.cache, inp.D)
        self.num_splits = inp.num_splits if num_splits is None else num_splits
        W = inp.block_table.shape[1]
        self.plan = sap.plan(inp.B, inp.sq, inp.Hq, inp.Hkv, inp.D, inp.P, W, inp.window,
                             self.num_splits)
        self.out = torch.empty((inp.B, inp.sq, inp.Hq, inp.D), dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty((inp.B, inp.sq, inp.Hq), dtype=torch.float32, device="cuda")
        ws = sap.workspace_size(inp.B, inp.sq, inp.Hq, inp.Hkv, inp.D, inp.P, W, inp.window,
                                self.num_splits)
        self.ws = sap.new_workspace(ws, "cuda")
        S = self.plan["splits"]
        self.part_o = torch.empty((S, inp.B * inp.sq, inp.Hq, inp.D), dtype=torch.float32,
                                  device="cuda")
        self.part_lse = torch.empty((S, inp.B * inp.sq, inp.Hq), dtype=torch.float32, device="cuda")
        lens, _, _ = sap.paged_attn_describe_host(
            inp.block_table.cpu(), inp.seq_lens.cpu(), query_len=inp.sq, Hq=inp.Hq, Hkv=inp.Hkv,
            D=inp.D, page_size=inp.P, window=inp.window, num_splits=1)
        self.visible_lens = [int(x) for x in lens.tolist()]
        self.visible = sum(self.visible_lens)
        elem = 1 if inp.kv_dtype == "fp8_e4m3" else 2
        self.kv_bytes = self.visible * inp.Hkv * 2 * inp.D * elem
        self.flops = 4 * inp.sq * inp.Hq * inp.D * self.visible

    def step(self):
        i = self.inp
        self.sap.paged_attn_run(i.q, self.k, self.v, i.block_table, i.seq_lens,
                                scale=i.scale * i.q_scale,
                                window=i.window, num_splits=self.num_splits, k_scale=i.k_scale,
                                v_scale=i.v_scale, out=self.out, lse=self.lse, workspace=self.ws,
                                causal=self.causal)

    def kernel(self):
        i = self.inp
        self.sap.paged_attn_partial(i.q, self.k, self.v, i.block_table, i.seq_lens,
                                    scale=i.scale * i.q_scale,
                                    num_splits=self.plan["partial_num_splits"], window=i.window,
                                    k_scale=i.k_scale, v_scale=i.v_scale, part_o=self.part_o,
                                    part_lse=self.part_lse)


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info

        return int(max([d.get("num_threads", 1) for d in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(pb: PagedBench, seconds: float):
    """The fp64 oracle on the host over the same workload: requests in order,
    wrapping around for further passes, until `seconds` of oracle time (at least
    one request).  Each request is evaluated from host copies of its own pages."""
    import numpy as np
    import torch

    import oracle
    from oracle.attention import kv_halves
    from workloads import to_numpy_bits

    inp = pb.inp
    bt = inp.block_table.cpu()
    lens = inp.seq_lens.cpu()
    q = to_numpy_bits(inp.q.cpu())
    q_dtype = {torch.bfloat16: "bf16", torch.float16: "fp16", torch.uint8: "fp8_e4m3"}[inp.q.dtype]
    elem = 1 if inp.kv_dtype == "fp8_e4m3" else 2
    host = {}  # request -> (k, v, table): host copies of exactly its pages
    done, toks, t_used = 0, 0, 0.0
    while t_used < seconds or done == 0:
        b = done % inp.B
        if b not in host:
            if len(host) > 4:
                host.clear()
            n = -(-int(lens[b]) // inp.P)
            pages = bt[b, :n].to(torch.long)
            cache = to_numpy_bits(inp.cache.index_select(0, pages.to(inp.cache.device)).cpu())
            table = np.zeros((inp.B, max(n, 1)), dtype=np.int64)
            table[b, :n] = np.arange(n)
            k, v = kv_halves(cache, inp.D)
            host[b] = (k, v, table)
        k, v, table = host[b]
        t0 = time.perf_counter()
        oracle.paged_attention(q, q_dtype, k, v, inp.kv_dtype, table, lens.numpy(),
                               scale=inp.scale, q_scale=inp.q_scale, window=inp.window,
                               k_scale=inp.k_scale, v_scale=inp.v_scale, requests=[b],
                               causal=pb.causal)
        t_used += time.perf_counter() - t0
        done += 1
        toks += int(pb.visible_lens[b])
    return {
        "value": done * inp.sq / t_used,
        "unit": "tokens/s",
        "cores": _blas_threads(),
        "kind": "oracle",
        "sample": f"{done} request evaluations of {pb.name}{' (causal)' if pb.causal else ''} "
                  f"({done / inp.B:.2f} passes over its {inp.B} requests, all {inp.Hkv} kv heads, "
                  f"{toks} visible keys), fp64 numpy, {t_used:.1f} s",
        "host_cpus": len(os.sched_getaffinity(0)),
        "kv_gbps_equiv": toks * inp.Hkv * 2 * inp.D * elem / t_used / 1e9,
    }


def cpu_baseline_segments(s, seconds: float):
    """The fp64 oracle (two-stage form) on the host, one DASH query at a time (each
    query's own rows of K/V), until `seconds` of oracle time."""
    import oracle
    from workloads import to_numpy_bits

    q = to_numpy_bits(s.q.cpu())
    k = to_numpy_bits(s.k.cpu())
    v = to_numpy_bits(s.v.cpu())
    used = s.used.cpu().numpy()
    bias = s.bias.cpu().numpy()
    per = s.topk * s.bs + s.local
    done, toks, t_used = 0, 0, 0.0
    while t_used < seconds or done == 0:
        n = done % s.N
        rows = slice(n * per, (n + 1) * per)
        t0 = time.perf_counter()
        oracle.segment_attention(q[n:n + 1], k[rows], v[rows], used[n:n + 1], bias[n:n + 1],
                                 topk=s.topk, bs=s.bs, local=s.local, scale=s.scale)
        t_used += time.perf_counter() - t0
        done += 1
        toks += int(used[n].sum())
    return {
        "value": done / t_used,
        "unit": "queries/s",
        "cores": _blas_threads(),
        "kind": "oracle",
        "sample": f"{done} of the {s.N} DASH queries (all {s.topk + 1} segments and {s.Hkv} kv "
                  f"heads each, {toks} valid rows), fp64 numpy two-stage form, {t_used:.1f} s",
        "host_cpus": len(os.sched_getaffinity(0)),
        "kv_gbps_equiv": toks * s.Hkv * 2 * s.D * 2 / t_used / 1e9,
    }


def calibrate_copy(n_bytes: int = 1 << 30, reps: int = 3):
    """A plain device copy of known size, for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE."""
    import torch

    src = torch.empty(n_bytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"calibration copy: {reps} x {n_bytes} bytes read and written")


def measure_paged(name: str, causal: bool, steps: int, warmup: int, cpu_seconds: float,
                  pb: PagedBench = None):
    """Step time (paged_attn_run, combine included), the attention kernel alone (the
    partial pass in the same launch configuration; dense blocks only, the partial entry
    point has no causal form) and the oracle beside it, for one paged workload."""
    import torch

    pb = pb or PagedBench(name, causal=causal)
    inp = pb.inp
    flush = mall_flush(pb.kv_bytes)
    step_ms, _ = time_events(pb.step, steps, warmup, flush, rounds=3)
    res = {
        "workload": name, "causal": causal, "B": inp.B, "query_len": inp.sq, "Hq": inp.Hq,
        "Hkv": inp.Hkv, "head_dim": inp.D, "kv_dtype": inp.kv_dtype,
        "q_dtype": str(inp.q.dtype).replace("torch.", ""), "window": inp.window,
        "splits": pb.plan["splits"], "grid": pb.plan["grid"], "visible_keys": pb.visible,
        "kv_bytes": pb.kv_bytes, "mall_flush": flush is not None,
        "step_us": step_ms * 1e3, "tokens_per_s": inp.B * inp.sq / (step_ms / 1e3),
        "kv_gbps": pb.kv_bytes / step_ms / 1e6, "hbm_frac": pb.kv_bytes / step_ms / 1e6 / HBM_PEAK_GBPS,
    }
    if not causal:
        kern_ms, _ = time_events(pb.kernel, steps, warmup, flush, rounds=3)
        res.update(kernel_us=kern_ms * 1e3, kernel_gbps=pb.kv_bytes / kern_ms / 1e6,
                   kernel_hbm_frac=pb.kv_bytes / kern_ms / 1e6 / HBM_PEAK_GBPS)
    if inp.sq >= 16:
        res.update(mfma_tflops=pb.flops / step_ms / 1e9,
                   mfma_frac_of_bf16_peak=pb.flops / step_ms / 1e9 / BF16_DENSE_TFLOPS)
    log(f"{name}{' causal' if causal else ''}: step {step_ms * 1e3:.1f} us "
        f"({res['kv_gbps']:.0f} GB/s)" + (f", kernel {res['kernel_us']:.1f} us" if not causal else ""))
    if cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(pb, cpu_seconds)
    del pb
    torch.cuda.empty_cache()
    return res


def run_segments(steps, warmup, cpu_seconds):
    """C5: the fused kernel (one launch) and the two-stage form (partials + combine)."""
    import torch

    import segmented_attention_paged_amd as sap
    from workloads import segment_config

    s = segment_config("c5_dash_segments", device="cuda")
    out = torch.empty((s.N, s.Hq, s.D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(sap.segment_attn_workspace_size(s.N, s.topk, s.Hq, s.D), dtype=torch.uint8,
                     device="cuda")
    kv_bytes = int(s.used.to(torch.int64).sum()) * s.Hkv * 2 * s.D * 2
    res = {"workload": "c5_dash_segments", "N": s.N, "Hq": s.Hq, "Hkv": s.Hkv, "head_dim": s.D,
           "topk": s.topk, "bs": s.bs, "local": s.local, "kv_bytes": kv_bytes, "mall_flush": True}
    for fused in (True, False):
        fn = lambda: sap.segment_attn_run(s.q, s.k, s.v, s.used, s.bias, bs=s.bs, local=s.local,
                                          fused=fused, out=out, workspace=ws)
        ms, _ = time_events(fn, steps, warmup, mall_flush(kv_bytes))
        res["fused" if fused else "two_stage"] = {
            "step_us": ms * 1e3, "queries_per_s": s.N / (ms / 1e3), "kv_gbps": kv_bytes / ms / 1e6,
            "hbm_frac": kv_bytes / ms / 1e6 / HBM_PEAK_GBPS}
        log(f"c5_dash_segments {'fused' if fused else 'two-stage'}: {ms * 1e3:.1f} us "
            f"({kv_bytes / ms / 1e6:.0f} GB/s)")
    if cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline_segments(s, cpu_seconds)
    del s, out, ws
    torch.cuda.empty_cache()
    return res


def run_kv_write(steps, warmup):
    """paged_kv_write of a prefill chunk (65536 tokens x 8 kv heads x D=128, scattered
    over a pool of twice as many 16-token slots) and of one decode step (64 tokens)."""
    import torch

    import segmented_attention_paged_amd as sap
    from workloads import make_kv_write

    res = {}
    for cache_dtype in ("bf16", "fp8_e4m3"):
        for label, T, pages in (("prefill_chunk", 65536, 8192), ("decode_step", 64, 8192)):
            w = make_kv_write(T=T, Hkv=8, D=128, P=16, pages=pages, seed=50, cache_dtype=cache_dtype,
                              device="cuda")
            k, v = sap.kv_halves(w.cache, w.D)
            fn = lambda: sap.paged_kv_write(w.key, w.value, w.slot_mapping, k, v, k_scale=w.k_scale,
                                            v_scale=w.v_scale)
            eb = 1 if cache_dtype == "fp8_e4m3" else 2
            nbytes = T * w.Hkv * w.D * 2 * 2 + T * w.Hkv * 2 * w.D * eb + T * 8  # read, write, slots
            ms, _ = time_events(fn, steps, warmup, mall_flush(nbytes))
            res[f"{label}_{cache_dtype}"] = {
                "tokens": T, "us": ms * 1e3, "gbps": nbytes / ms / 1e6,
                "hbm_frac": nbytes / ms / 1e6 / HBM_PEAK_GBPS, "algorithmic_bytes": nbytes}
            log(f"kv write {label} {cache_dtype}: {ms * 1e3:.1f} us, {nbytes / ms / 1e6:.0f} GB/s")
            del w, k, v
            torch.cuda.empty_cache()
    return res


# Every other configuration, measured in the default run after the headline:
# (workload, causal).  C3 (dense) is measured with the headline's sq=16 block.
OTHER_PAGED = [
    ("c1_tiny", False), ("c3w_query_block_window", False), ("c3_query_block", True),
    ("c3w_query_block_window", True), ("c3f_query_block_fp8", False), ("c4_split_kv", False),
    ("c4f_split_kv_fp8", False),
]


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c2_gqa_decode")
    ap.add_argument("--num-splits", type=int, default=None,
                    help="override the split policy (0 auto, S > 0, -c chunks of c pages)")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the headline workload (no sq=16 block, other configs or cache write)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kv-write", action="store_true", help="skip the cache-write measurement")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="oracle seconds for the headline workload's CPU baseline")
    ap.add_argument("--cpu-seconds-other", type=float, default=2.0,
                    help="oracle seconds for each other configuration's CPU baseline")
    ap.add_argument("--calibrate-copy", action="store_true")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path, so --gpus > 1 "
              "is not supported.", file=sys.stderr)
        return 2

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    import segmented_attention_paged_amd as sap

    sap.load()
    if args.calibrate_copy:
        calibrate_copy()
    cpu_s = 0.0 if args.no_cpu_baseline else args.cpu_seconds
    cpu_o = 0.0 if args.no_cpu_baseline else args.cpu_seconds_other
    sub_steps, sub_warm = max(10, args.steps // 2), max(3, args.warmup // 2)

    pb = PagedBench(args.workload, args.num_splits)
    inp = pb.inp
    log(f"{args.workload}: B={inp.B} sq={inp.sq} Hq={inp.Hq} Hkv={inp.Hkv} D={inp.D} P={inp.P} "
        f"visible keys={pb.visible} KV bytes={pb.kv_bytes / 1e9:.3f} GB plan={pb.plan}")
    step_ms, step_wall = time_events(pb.step, args.steps, args.warmup)
    kern_ms, _ = time_events(pb.kernel, args.steps, args.warmup)
    log(f"step {step_ms * 1e3:.1f} us (wall {step_wall * 1e3:.1f} us), attention kernel "
        f"{kern_ms * 1e3:.1f} us")
    # the same step with a 512 MB read between calls: what the Infinity Cache holds of
    # the last call does not count
    flushed_ms, _ = time_events(pb.step, sub_steps, sub_warm, mall_flush(pb.kv_bytes, force=True))
    log(f"step after a 512 MB read flush: {flushed_ms * 1e3:.1f} us")
    tok_s = inp.B * inp.sq / (step_ms / 1e3)
    kv_gbps = pb.kv_bytes / step_ms / 1e6
    kern_gbps = pb.kv_bytes / kern_ms / 1e6
    traffic = read_counters(args.workload)
    headline_cfg = {
        "workload": args.workload, "B": inp.B, "query_len": inp.sq, "Hq": inp.Hq,
        "Hkv": inp.Hkv, "head_dim": inp.D, "page_size": inp.P, "window": inp.window,
        "visible_keys": pb.visible, "splits": pb.plan["splits"],
        "chunk_pages": pb.plan["chunk_pages"], "grid": pb.plan["grid"],
    }
    result = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if inp.kv_dtype == "bf16" else "fp8_e4m3 kv, bf16 q",
        "data": "synthetic",
        "config": headline_cfg,
        "kv_gbps": kv_gbps,
        "hbm_frac": kv_gbps / HBM_PEAK_GBPS,
        "step_us_after_mall_flush": flushed_ms * 1e3,
        "roofline": {
            "kernel": "attn_kernel (paged partial pass)",
            "bound": "hbm",
            "achieved": kern_gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": kern_gbps / HBM_PEAK_GBPS,
            "traffic": traffic,
            "kernel_us": kern_ms * 1e3,
            "algorithmic_bytes_per_launch": pb.kv_bytes,
        },
    }
    workloads = {args.workload: dict(headline_cfg, step_us=step_ms * 1e3, tokens_per_s=tok_s,
                                     kv_gbps=kv_gbps, hbm_frac=kv_gbps / HBM_PEAK_GBPS,
                                     kernel_us=kern_ms * 1e3, kernel_gbps=kern_gbps,
                                     kernel_hbm_frac=kern_gbps / HBM_PEAK_GBPS,
                                     step_us_after_mall_flush=flushed_ms * 1e3)}
    if cpu_s > 0:
        result["cpu_baseline"] = cpu_baseline(pb, cpu_s)
        workloads[args.workload]["cpu_baseline"] = result["cpu_baseline"]
    del pb
    torch.cuda.empty_cache()

    if not args.headline_only:
        c3 = measure_paged("c3_query_block", False, sub_steps, sub_warm, cpu_o)
        workloads["c3_query_block"] = c3
        result["sq16_block"] = {
            "workload": "c3_query_block", "us": c3["step_us"], "tokens_per_s": c3["tokens_per_s"],
            "kv_gbps": c3["kv_gbps"], "hbm_frac": c3["hbm_frac"], "mfma_tflops": c3["mfma_tflops"],
            "mfma_frac_of_bf16_peak": c3["mfma_frac_of_bf16_peak"], "splits": c3["splits"],
            "kernel_us": c3["kernel_us"], "kernel_hbm_frac": c3["kernel_hbm_frac"],
        }
        for name, causal in OTHER_PAGED:
            key = name + ("_causal" if causal else "")
            workloads[key] = measure_paged(name, causal, sub_steps, sub_warm, cpu_o)
        workloads["c5_dash_segments"] = run_segments(sub_steps, sub_warm, cpu_o)
        if not args.no_kv_write:
            result["kv_write"] = run_kv_write(sub_steps, sub_warm)
    result["workloads"] = workloads

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
