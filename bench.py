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

    python bench.py [--steps K] [--warmup W] [--all] [--no-cpu-baseline] [--no-kv-write]
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


def time_events(fn, steps: int, warmup: int, flush=None):
    """Average ms per call on the current stream (HIP events); optional cache flush between calls."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    if flush is None:
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        s.record()
        for _ in range(steps):
            fn()
        e.record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / steps
        return s.elapsed_time(e) / steps, wall
    total = 0.0
    t0 = time.perf_counter()
    for _ in range(steps):
        flush()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        torch.cuda.synchronize()
        total += s.elapsed_time(e)
    return total / steps, (time.perf_counter() - t0) * 1e3 / steps


_FLUSH = {}


def mall_flush(nbytes: int):
    """A 512 MB read run between timed calls when a call touches less than 1 GiB, so its
    data is not served from the 256 MB Infinity Cache; None otherwise.  A read, not a
    fill: a fill leaves dirty lines whose write-back the timed call would pay for."""
    import torch

    if nbytes >= (1 << 30):
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
        self.visible = int(lens.to(torch.int64).sum())
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


def cpu_baseline(pb: PagedBench, seconds: float):
    """The fp64 oracle on the host over the same workload: requests in order,
    wrapping around for further passes, until `seconds` of oracle time."""
    import numpy as np
    import torch

    import oracle
    from oracle.attention import kv_halves
    from workloads import to_numpy_bits

    inp = pb.inp
    bt = inp.block_table.cpu()
    lens = inp.seq_lens.cpu()
    q = to_numpy_bits(inp.q.cpu())
    try:
        from threadpoolctl import threadpool_info

        blas_threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    host = {}  # request -> (k, v, table): host copies of exactly its pages
    done, toks, t_used = 0, 0, 0.0
    while t_used < seconds:
        b = done % inp.B
        if b not in host:
            n = -(-int(lens[b]) // inp.P)
            pages = bt[b, :n].to(torch.long)
            cache = to_numpy_bits(inp.cache.index_select(0, pages.to(inp.cache.device)).cpu())
            table = np.zeros((inp.B, max(n, 1)), dtype=np.int64)
            table[b, :n] = np.arange(n)
            k, v = kv_halves(cache, inp.D)
            host[b] = (k, v, table)
        k, v, table = host[b]
        t0 = time.perf_counter()
        oracle.paged_attention(q, "bf16", k, v, inp.kv_dtype, table, lens.numpy(), scale=inp.scale,
                               window=inp.window, k_scale=inp.k_scale, v_scale=inp.v_scale,
                               requests=[b])
        t_used += time.perf_counter() - t0
        done += 1
        toks += int(lens[b])
    return {
        "value": done * inp.sq / t_used,
        "unit": "tokens/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"{done} request evaluations of {pb.name} ({done / inp.B:.1f} passes over its "
                  f"{inp.B} requests, all {inp.Hkv} kv heads, {toks} keys), fp64 numpy, "
                  f"{t_used:.1f} s",
        "host_cpus": len(os.sched_getaffinity(0)),
        "kv_gbps_equiv": toks * inp.Hkv * 2 * inp.D * 2 / t_used / 1e9,
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


def run_segments(steps, warmup):
    import torch

    import segmented_attention_paged_amd as sap
    from workloads import segment_config

    s = segment_config("c5_dash_segments", device="cuda")
    out = torch.empty((s.N, s.Hq, s.D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(sap.segment_attn_workspace_size(s.N, s.topk, s.Hq, s.D), dtype=torch.uint8,
                     device="cuda")
    kv_bytes = int(s.used.to(torch.int64).sum()) * s.Hkv * 2 * s.D * 2
    res = {}
    for fused in (True, False):
        fn = lambda: sap.segment_attn_run(s.q, s.k, s.v, s.used, s.bias, bs=s.bs, local=s.local,
                                          fused=fused, out=out, workspace=ws)
        ms, _ = time_events(fn, steps, warmup, mall_flush(kv_bytes))
        res["fused" if fused else "two_stage"] = {
            "us": ms * 1e3, "kv_gbps": kv_bytes / ms / 1e6,
            "hbm_frac": kv_bytes / ms / 1e6 / HBM_PEAK_GBPS}
    res["kv_bytes"] = kv_bytes
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


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c2_gqa_decode")
    ap.add_argument("--num-splits", type=int, default=None,
                    help="override the split policy (0 auto, S > 0, -c chunks of c pages)")
    ap.add_argument("--all", action="store_true", help="also time every other workload")
    ap.add_argument("--no-block", action="store_true", help="skip the sq=16 MFMA measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kv-write", action="store_true", help="skip the cache-write measurement")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
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

    pb = PagedBench(args.workload, args.num_splits)
    inp = pb.inp
    log(f"{args.workload}: B={inp.B} sq={inp.sq} Hq={inp.Hq} Hkv={inp.Hkv} D={inp.D} P={inp.P} "
        f"visible keys={pb.visible} KV bytes={pb.kv_bytes / 1e9:.3f} GB plan={pb.plan}")
    step_ms, step_wall = time_events(pb.step, args.steps, args.warmup)
    kern_ms, _ = time_events(pb.kernel, args.steps, args.warmup)
    log(f"step {step_ms * 1e3:.1f} us (wall {step_wall * 1e3:.1f} us), attention kernel "
        f"{kern_ms * 1e3:.1f} us")
    tok_s = inp.B * inp.sq / (step_ms / 1e3)
    kv_gbps = pb.kv_bytes / step_ms / 1e6
    kern_gbps = pb.kv_bytes / kern_ms / 1e6
    traffic = read_counters(args.workload)

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
        "config": {
            "workload": args.workload, "B": inp.B, "query_len": inp.sq, "Hq": inp.Hq,
            "Hkv": inp.Hkv, "head_dim": inp.D, "page_size": inp.P, "window": inp.window,
            "visible_keys": pb.visible, "splits": pb.plan["splits"],
            "chunk_pages": pb.plan["chunk_pages"], "grid": pb.plan["grid"],
        },
        "kv_gbps": kv_gbps,
        "hbm_frac": kv_gbps / HBM_PEAK_GBPS,
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
    del pb
    torch.cuda.empty_cache()

    if not args.no_block:
        bb = PagedBench("c3_query_block")
        ms, _ = time_events(bb.step, max(10, args.steps // 2), max(3, args.warmup // 2))
        result["sq16_block"] = {
            "workload": "c3_query_block", "us": ms * 1e3,
            "tokens_per_s": bb.inp.B * bb.inp.sq / (ms / 1e3),
            "kv_gbps": bb.kv_bytes / ms / 1e6, "hbm_frac": bb.kv_bytes / ms / 1e6 / HBM_PEAK_GBPS,
            "mfma_tflops": bb.flops / ms / 1e9,
            "mfma_frac_of_bf16_peak": bb.flops / ms / 1e9 / BF16_DENSE_TFLOPS,
            "splits": bb.plan["splits"],
        }
        log(f"c3_query_block: {ms * 1e3:.1f} us, MFMA {bb.flops / ms / 1e9:.1f} TFLOP/s")
        del bb
        torch.cuda.empty_cache()
        # the same blocks with the causal mask (exact per-token window for C3w); the
        # pages read are the same as the dense block's, so the byte count is too
        causal = {}
        for name in ("c3_query_block", "c3w_query_block_window"):
            bb = PagedBench(name, causal=True)
            ms, _ = time_events(bb.step, max(10, args.steps // 2), max(3, args.warmup // 2),
                                mall_flush(bb.kv_bytes))
            causal[name] = {"us": ms * 1e3, "tokens_per_s": bb.inp.B * bb.inp.sq / (ms / 1e3),
                            "kv_gbps": bb.kv_bytes / ms / 1e6,
                            "hbm_frac": bb.kv_bytes / ms / 1e6 / HBM_PEAK_GBPS,
                            "splits": bb.plan["splits"]}
            log(f"{name} causal: {ms * 1e3:.1f} us")
            del bb
            torch.cuda.empty_cache()
        result["sq16_block"]["causal"] = causal
        # fp8 query against an fp8 cache (q.k on fp8 MFMA, P.V in bf16)
        bb = PagedBench("c3f_query_block_fp8")
        ms, _ = time_events(bb.step, max(10, args.steps // 2), max(3, args.warmup // 2))
        result["sq16_block"]["fp8_query"] = {
            "workload": "c3f_query_block_fp8", "us": ms * 1e3,
            "tokens_per_s": bb.inp.B * bb.inp.sq / (ms / 1e3), "kv_gbps": bb.kv_bytes / ms / 1e6,
            "hbm_frac": bb.kv_bytes / ms / 1e6 / HBM_PEAK_GBPS, "splits": bb.plan["splits"]}
        log(f"c3f_query_block_fp8: {ms * 1e3:.1f} us, {bb.kv_bytes / ms / 1e6:.0f} GB/s")
        del bb
        torch.cuda.empty_cache()

    if not args.no_kv_write:
        result["kv_write"] = run_kv_write(max(10, args.steps // 2), max(3, args.warmup // 2))

    if args.all:
        extra = {}
        for name in ["c1_tiny", "c3w_query_block_window", "c4_split_kv", "c4f_split_kv_fp8"]:
            bb = PagedBench(name)
            flush = mall_flush(bb.kv_bytes)
            ms, _ = time_events(bb.step, max(10, args.steps // 2), max(3, args.warmup // 2), flush)
            extra[name] = {"us": ms * 1e3, "tokens_per_s": bb.inp.B * bb.inp.sq / (ms / 1e3),
                           "kv_gbps": bb.kv_bytes / ms / 1e6,
                           "hbm_frac": bb.kv_bytes / ms / 1e6 / HBM_PEAK_GBPS,
                           "splits": bb.plan["splits"]}
            log(f"{name}: {ms * 1e3:.1f} us, {bb.kv_bytes / ms / 1e6:.0f} GB/s")
            del bb
            torch.cuda.empty_cache()
        extra["c5_dash_segments"] = run_segments(max(10, args.steps // 2), max(3, args.warmup // 2))
        result["other_workloads"] = extra

    if not args.no_cpu_baseline:
        pb2 = PagedBench(args.workload, args.num_splits)
        result["cpu_baseline"] = cpu_baseline(pb2, args.cpu_seconds)
        del pb2

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
