#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

One step = one decode-attention call of the hot path: decode_attn_run (the
split kernel: bounds, mask program, address translation, K/V streaming,
scores, online softmax, PV, state write) followed by decode_attn_combine (the
log-sum-exp reduction), on the workload

    B=8, S_q=1, H_q=32, H_kv=8 (4 query heads per K/V head), d_h=128,
    S_k=4096 for every sequence, bf16 q/k/v ~ N(0,1), contiguous
    [B, T, H_kv, d_h] cache, fp32 output (a Llama-3-8B-shaped layer).

Inputs are resident in HBM before timing.  Several disjoint input sets
(> 512 MiB in total) are rotated so the 256 MB last-level cache cannot serve
repeated K/V.  The printed JSON line reports algorithmic GB/s per call as
`value`, the per-call time, the split kernel's roofline against the 8 TB/s
HBM peak (its duration measured with HIP events on the launch stream), HBM
traffic from the committed profiler counters when they were taken on the
current kernel sources, and the CPU oracle's throughput on the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0
WORKLOAD = dict(batch=8, num_q_heads=32, num_kv_heads=8, head_dim=128, seq_len=4096)
LONG = dict(batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128, seq_len=131072)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "split_kernel_llama3_8b_layer_traffic.json")
KERNEL_SOURCES = ["kv_cache_amd/csrc/split_kernel_mfma.hpp", "kv_cache_amd/csrc/split_common.hpp",
                  "kv_cache_amd/csrc/device_common.hpp", "kv_cache_amd/csrc/decode_attn.hip"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(B, Hq, Hkv, D, T, S):
    kv = 2 * B * T * Hkv * D * 2                      # visible K and V rows, once per K/V head
    q = B * Hq * D * 2
    ws = B * Hq * S * (D + 2) * 4                      # (m, l, u) states
    out = B * Hq * D * 4 + B * Hq * 4                  # O and LSE
    meta = B * 4                                       # seq_lens
    split = kv + q + ws + meta                         # split kernel: reads K/V/q, writes states
    combine = ws + out                                 # combine kernel: reads states, writes O, LSE
    return kv, split, split + combine


class Case:
    """Device buffers and a plan for one contiguous bf16 decode shape."""

    def __init__(self, torch, ka, shape, num_splits, min_bytes, seed):
        self.torch, self.ka = torch, ka
        B, Hq, Hkv, D, T = (shape[k] for k in ("batch", "num_q_heads", "num_kv_heads", "head_dim",
                                                "seq_len"))
        self.shape = (B, Hq, Hkv, D, T)
        import synth
        prob = synth.Problem(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, q_dtype="bf16",
                             kv_format="bf16", layout="contig", kv_capacity=T, max_seq_len=T,
                             num_splits=num_splits)
        _, self.plan, self.ws_bytes, _ = ka.decode_attn_plan(ka.problem_from(prob))
        per_set = 2 * B * T * Hkv * D * 2
        self.nsets = max(2, -(-min_bytes // per_set))
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        self.sets = []
        for _ in range(self.nsets):
            k = torch.randn((B, T, Hkv, D), device="cuda", dtype=torch.bfloat16, generator=g)
            v = torch.randn((B, T, Hkv, D), device="cuda", dtype=torch.bfloat16, generator=g)
            q = torch.randn((B, Hq, D), device="cuda", dtype=torch.bfloat16, generator=g)
            self.sets.append((q, k, v))
        self.seq_lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        self.out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
        self.lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        self.args = [ka.make_args(q, k, v, self.seq_lens, self.ws, self.ws_bytes)
                     for (q, k, v) in self.sets]
        self.stream = torch.cuda.current_stream().cuda_stream

    def run(self, i):
        self.ka.decode_attn_run(self.plan, self.args[i % self.nsets], self.stream)

    def call(self, i):
        self.ka.decode_attn_run(self.plan, self.args[i % self.nsets], self.stream)
        self.ka.decode_attn_combine(self.plan, self.ws, self.ws_bytes, self.out, self.lse, self.stream)

    def time(self, fn, steps, warmup):
        torch = self.torch
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            fn(warmup + i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps      # ms per launch sequence

    def samples(self, fn, n, warmup):
        """Per-call event pairs (each call's own interval) for the sample log."""
        torch = self.torch
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for i, (a, b) in enumerate(evs):
            a.record()
            fn(warmup + i)
            b.record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1000.0 for a, b in evs]


def hbm_probe(torch, nbytes=512 << 20):
    """Practical read ceiling of the box: a plain streaming-read kernel."""
    import ctypes
    path = os.path.join(ROOT, "kv_cache_amd", "libhbm_probe.so")
    L = ctypes.CDLL(path)
    L.hbm_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int,
                                 ctypes.c_void_p]
    L.hbm_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int,
                                 ctypes.c_void_p]
    st = torch.cuda.current_stream().cuda_stream
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    sink = torch.empty(4096, dtype=torch.int32, device="cuda")
    for i in range(3):
        L.hbm_probe_read(bufs[i % 2].data_ptr(), nbytes, sink.data_ptr(), 2048, st)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 20
    e0.record()
    for i in range(n):
        L.hbm_probe_read(bufs[i % 2].data_ptr(), nbytes, sink.data_ptr(), 2048, st)
    e1.record()
    torch.cuda.synchronize()
    read_gbs = nbytes / (e0.elapsed_time(e1) / n * 1e-3) / 1e9
    # one copy of known size: the reference for the profiler's byte counters
    L.hbm_probe_copy(bufs[0].data_ptr(), bufs[1].data_ptr(), 256 << 20, 2048, st)
    torch.cuda.synchronize()
    del bufs
    return read_gbs


def cpu_baseline(seconds: float = 10.0):
    """The fp64 NumPy oracle on the same workload shape and seeded data,
    repeated until about `seconds` of wall clock have passed."""
    import numpy as np  # noqa: F401
    import oracle
    import synth
    w = synth.make_contiguous(0, WORKLOAD["batch"], WORKLOAD["num_q_heads"], WORKLOAD["num_kv_heads"],
                              WORKLOAD["head_dim"], [WORKLOAD["seq_len"]] * WORKLOAD["batch"])
    calls = 0
    t0 = time.perf_counter()
    while True:
        oracle.attend(w.problem, w.buffers)
        calls += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    B, Hq, Hkv, D, T = (WORKLOAD[k] for k in ("batch", "num_q_heads", "num_kv_heads", "head_dim", "seq_len"))
    _, _, alg = algorithmic_bytes(B, Hq, Hkv, D, T, 1)
    threads = 1
    try:
        import threadpoolctl
        threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] or [1])
    except Exception:
        pass
    return {"value": round(alg * calls / dt / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "s_per_call": round(dt / calls, 4),
            "sample": f"{calls} full calls of the workload (fp64 NumPy oracle, seed 0), {dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long", action="store_true", help="skip the 128k-context figure")
    ap.add_argument("--samples-out", default=None, help="write raw per-call samples (JSON)")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode path has no multi-GPU mode "
              "(it shards by request and K/V head with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import kv_cache_amd as ka
    ka.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    ceiling = hbm_probe(torch)
    case = Case(torch, ka, WORKLOAD, a.num_splits, 600 << 20, seed=0)
    B, Hq, Hkv, D, T = case.shape
    S = case.plan.num_splits
    kv_bytes, split_bytes, call_bytes = algorithmic_bytes(B, Hq, Hkv, D, T, S)

    torch.cuda.synchronize()
    ms_call = case.time(case.call, a.steps, a.warmup)     # timed region: K steps
    ms_split = case.time(case.run, a.steps, a.warmup)      # split kernel alone, same stream
    samples = case.samples(case.call, 100, 10)
    us_call = ms_call * 1000.0
    value = call_bytes / (ms_call * 1e-3) / 1e9

    achieved = split_bytes / (ms_split * 1e-3) / 1e9
    traffic = None
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_source_hash") == kernel_source_hash() and tr.get("num_splits") == S:
            traffic = tr.get("hbm_bytes_per_launch")
    except (OSError, ValueError):
        traffic = None

    extra = {}
    if not a.no_long:
        long_case = Case(torch, ka, LONG, 0, 600 << 20, seed=1)
        ms_long = long_case.time(long_case.call, 30, 5)
        _, _, long_bytes = algorithmic_bytes(*long_case.shape, long_case.plan.num_splits)
        extra["long_context_128k"] = {
            "config": "B=1 H_q=32 H_kv=8 d=128 T=131072 bf16 contiguous causal",
            "num_splits": long_case.plan.num_splits, "us_per_call": round(ms_long * 1000, 2),
            "GBs": round(long_bytes / (ms_long * 1e-3) / 1e9, 1),
            "pct_of_peak": round(100 * long_bytes / (ms_long * 1e-3) / 1e9 / PEAK_GBS, 1)}
        del long_case

    samples.sort()
    line = {
        "metric": "decode-attn us/call + achieved HBM GB/s (% of peak), GQA 32q/8kv d128",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_call, 5),
        "us_per_call": round(us_call, 2),
        "pct_of_peak": round(100 * value / PEAK_GBS, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, rotated input sets > 512 MiB)",
        "config": {"workload": "llama3-8b-layer decode: B=8 H_q=32 H_kv=8 d=128 S_k=4096 bf16 "
                               "contiguous causal, fp32 out",
                   "num_splits": S, "chunk": case.plan.chunk, "input_sets": case.nsets},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "split_kernel_mfma", "us_per_launch": round(ms_split * 1000, 2),
                     "algorithmic_bytes_per_launch": split_bytes},
        "samples_us": {"count": len(samples), "min": round(samples[0], 2),
                       "median": round(samples[len(samples) // 2], 2),
                       "p95": round(samples[int(len(samples) * 0.95)], 2), "max": round(samples[-1], 2)},
        "hbm_read_probe_GBs": round(ceiling, 1),
        "kernel_source_hash": kernel_source_hash(),
    }
    line.update(extra)
    if a.samples_out:
        with open(a.samples_out, "w") as f:
            json.dump({"per_call_us": samples}, f)
    del case
    torch.cuda.synchronize()
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
