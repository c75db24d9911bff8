#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

One step = one decode-attention call of the hot path: decode_attn_run (the
split kernel: bounds, mask program, address translation, K/V streaming,
scores, online softmax, PV, state write) followed by decode_attn_combine (the
log-sum-exp reduction).  The headline workload is

    B=8, S_q=1, H_q=32, H_kv=8 (4 query heads per K/V head), d_h=128,
    S_k=4096 for every sequence, bf16 q/k/v ~ N(0,1), contiguous
    [B, T, H_kv, d_h] cache, fp32 output (a Llama-3-8B-shaped layer).

Inputs are resident in HBM before timing.  Several disjoint input sets
(> 512 MiB in total) are rotated so the 256 MB last-level cache cannot serve
repeated K/V.  The JSON line reports algorithmic GB/s per call as `value`,
the per-call time, the split kernel's roofline against the 8 TB/s HBM peak
(its duration measured with HIP events on the launch stream), HBM traffic
from the committed profiler counters when they were taken on the current
kernel sources, the other decode workloads (128k context, paged ragged batch,
int8 cache with sink+window mask, tiny fp32), and the CPU oracle's
throughput on the headline workload.
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
SETTLE_S = 0.25          # untimed calls before every timed region (GPU clock ramp)
PROFILES = os.path.join(ROOT, "profiles")
# every source that decides what the timed kernels do (the split count too)
KERNEL_SOURCES = ["kv_cache_amd/csrc/split_kernel_mfma.hpp", "kv_cache_amd/csrc/split_kernel_mfma_i8.hpp",
                  "kv_cache_amd/csrc/split_kernel.hpp", "kv_cache_amd/csrc/split_common.hpp",
                  "kv_cache_amd/csrc/combine_kernel.hpp", "kv_cache_amd/csrc/device_common.hpp",
                  "kv_cache_amd/csrc/decode_attn.hip", "kv_cache_amd/csrc/plan.cpp"]
# the kernel that moves the call's bytes, per workload (substring of its name)
DOMINANT = {"llama3_8b_layer": "split_kernel_mfma<4, false, 4, true, false, false, 0>",
            "long_context_128k": "split_kernel_mfma<4, false, 4, false, false, false, 0>",
            "int8_sink_window": "split_kernel_mfma_i8<4, 4, true, 0, false, true>",
            "paged_ragged": "split_kernel_mfma<4, true, 4, false, false, true, 0>"}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profile_record(workload):
    """The machine-readable block of profiles/<workload>_kernel_trace.md (written
    by ``bench.py --summarize``), or None."""
    path = os.path.join(PROFILES, f"{workload}_kernel_trace.md")
    try:
        with open(path) as f:
            text = f.read()
    except OSError:
        return None
    tag = "<!-- bench-data "
    i = text.find(tag)
    if i < 0:
        return None
    try:
        return json.loads(text[i + len(tag):text.index(" -->", i)])
    except ValueError:
        return None


def profiled_roofline(workload, call_bytes, num_splits):
    """Roofline of the workload's dominant kernel from its committed rocprofv3
    summary: its average duration and counter traffic, only when the summary
    was taken on the current kernel sources and split count."""
    rec = profile_record(workload)
    if not rec:
        return None, "no profile summary"
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None, f"profile taken on other kernel sources ({rec.get('kernel_source_hash')})"
    if rec.get("num_splits") != num_splits:
        return None, f"profile taken at {rec.get('num_splits')} splits"
    k = rec["kernels"].get(rec["dominant"])
    if not k:
        return None, "dominant kernel missing from the profile"
    us = k["avg_ns"] / 1000.0
    ach = call_bytes / (us * 1e-6) / 1e9
    out = {"kernel": rec["dominant"], "us_per_launch": round(us, 2), "calls": k["calls"],
           "achieved": round(ach, 1), "frac": round(ach / PEAK_GBS, 4),
           "source_hash": rec["kernel_source_hash"], "file": f"profiles/{workload}_kernel_trace.md"}
    tr = rec.get("traffic")
    if tr:
        out["traffic"] = tr["hbm_bytes_per_launch"]
    return out, None


def visible(T, mask):
    """Visible positions of a request of length T (plain set arithmetic)."""
    if mask is None:
        return range(T)
    ns, W = mask
    return sorted(set(range(min(ns, T))) | set(range(max(0, T - W), T)))


def algorithmic_bytes(kind, B, Hq, Hkv, D, lens, S, eb=2, mask=None, hidden=None, C=1, residual=128,
                      k_group=128, page_size=16):
    """Bytes the method must move once per call: every visible K/V row once per
    K/V head (int8: codes, the row's V scale, each touched K scale row once,
    bf16 residual rows), q, the split states written and read back, O and LSE,
    and the metadata (lengths, block-table entries, FlashMask summaries).
    Returns (K/V bytes, split-kernel bytes, whole-call bytes)."""
    kvb = 0
    meta = B * 4
    for bi, t in enumerate(lens):
        vis = visible(t, mask)
        if hidden is not None:          # FlashMask: the visible keys, plus the block summaries
            vis = [p for p in vis if not hidden[bi][p]]
            meta += ((t + 15) // 16) * 2 * 16
        if kind == "i8":
            n_q = t - min(t, residual)
            quant = [p for p in vis if p < n_q]
            kvb += Hkv * (len(quant) * (2 * D + 2) + (len(vis) - len(quant)) * 2 * D * 2
                          + len({p // k_group for p in quant}) * D * 2)
        else:
            kvb += Hkv * len(vis) * 2 * D * eb
        if kind == "paged":
            meta += ((t + page_size - 1) // page_size) * 4
    q = B * C * Hq * D * eb
    ws = B * C * Hq * S * (D + 2) * 4
    out = B * C * Hq * (D + 1) * 4
    split = kvb + q + ws + meta
    return kvb, split, split + ws + out


def sample_stats(samples):
    """count, min, median, p95 and max of sorted per-call samples (µs)."""
    n = len(samples)
    return {"count": n, "min": round(samples[0], 2), "median": round(samples[n // 2], 2),
            "p95": round(samples[int(n * 0.95)], 2), "max": round(samples[-1], 2)}


class GpuWorkload:
    """Device buffers, a plan and the algorithmic byte count of one workload.

    kinds: "contig" (bf16 or fp32), "paged" (bf16, P=16, ragged), "i8"
    (int8 codes + fp16 scales + bf16 residual, sink+window mask).  Contiguous
    options: C query rows per request (bottom-right causal), the HND layout,
    and FlashMask column intervals (seeded document/scatter runs)."""

    def __init__(self, torch, ka, kind, B, Hq, Hkv, D, lens, num_splits=0, min_bytes=0, seed=0,
                 dtype="bf16", mask=None, page_size=16, k_group=128, residual=128, C=1, hnd=False,
                 flashmask=False):
        import numpy as np
        import synth
        self.torch, self.ka, self.kind = torch, ka, kind
        self.B, self.Hq, self.Hkv, self.D = B, Hq, Hkv, D
        self.lens = [int(t) for t in lens]
        T = max(self.lens)
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        eb = 4 if dtype == "f32" else 2
        tdt = torch.float32 if dtype == "f32" else torch.bfloat16
        mk = dict(mask_kind="sink_window", n_sink=mask[0], window=mask[1]) if mask else {}
        if flashmask:
            mk = dict(mask_kind="flashmask")
        if kind == "contig":
            prob = synth.Problem(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, q_dtype=dtype,
                                 kv_format=dtype, kv_capacity=T, max_seq_len=T, num_splits=num_splits,
                                 num_queries=C, layout="contig_hnd" if hnd else "contig", **mk)
            per_set = 2 * B * T * Hkv * D * eb
        elif kind == "paged":
            pages = [(t + page_size - 1) // page_size for t in self.lens]
            n_pages = int(sum(pages) * 1.1) + 1
            maxp = max(pages)
            prob = synth.Problem(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, layout="paged",
                                 page_size=page_size, max_pages_per_seq=maxp, num_pages=n_pages,
                                 max_seq_len=T, num_splits=num_splits, **mk)
            per_set = 2 * n_pages * page_size * Hkv * D * 2
        elif kind == "i8":
            prob = synth.Problem(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, kv_format="i8",
                                 kv_capacity=T, max_seq_len=T, num_splits=num_splits, k_group=k_group,
                                 residual_len=residual, **mk)
            per_set = 2 * B * T * Hkv * D
        else:
            raise ValueError(kind)
        self.prob = prob
        _, self.plan, self.ws_bytes, _ = ka.decode_attn_plan(ka.problem_from(prob))
        self.S = self.plan.num_splits
        self.nsets = max(1, -(-min_bytes // per_set)) if min_bytes else 1
        self.seq_lens = torch.tensor(self.lens, dtype=torch.int32, device="cuda")
        self.mask_iv = self.mask_sum = None
        hidden = None
        if flashmask:
            iv = synth.flashmask_intervals(seed, self.lens, T)
            self.mask_iv = torch.from_numpy(np.ascontiguousarray(iv.astype(np.int32))).to("cuda")
            nblk = (T + 15) // 16
            self.mask_sum = torch.empty((B, nblk, 2, 4), dtype=torch.int32, device="cuda")
            ka.decode_attn_flashmask_summarize(self.plan, self.mask_iv, self.mask_sum,
                                               torch.cuda.current_stream().cuda_stream)
            # keys the decode row q = T_b - 1 cannot see: q in [UTS, UTE) or [LTS, LTE)
            hidden = [((iv[b, :t, 0] <= t - 1) & (t - 1 < iv[b, :t, 1])) |
                      ((iv[b, :t, 2] <= t - 1) & (t - 1 < iv[b, :t, 3])) for b, t in enumerate(self.lens)]
        qshape = (B, C, Hq, D) if C > 1 else (B, Hq, D)
        self.sets = []
        for _ in range(self.nsets):
            d = {"q": torch.randn(qshape, device="cuda", dtype=tdt, generator=g)}
            if kind == "contig":
                kvshape = (B, Hkv, T, D) if hnd else (B, T, Hkv, D)
                d["k"] = torch.randn(kvshape, device="cuda", dtype=tdt, generator=g)
                d["v"] = torch.randn(kvshape, device="cuda", dtype=tdt, generator=g)
            elif kind == "paged":
                d["k"] = torch.randn((n_pages, page_size, Hkv, D), device="cuda", dtype=tdt, generator=g)
                d["v"] = torch.randn((n_pages, page_size, Hkv, D), device="cuda", dtype=tdt, generator=g)
                perm = torch.randperm(n_pages, device="cuda", generator=g).to(torch.int32)
                table = torch.full((B, maxp), -1, dtype=torch.int32, device="cuda")
                cur = 0
                for b, n in enumerate(pages):
                    table[b, :n] = perm[cur:cur + n]
                    cur += n
                d["block_table"] = table
            else:
                n_groups = (T + k_group - 1) // k_group
                d["k"] = torch.randint(-127, 128, (B, T, Hkv, D), device="cuda", dtype=torch.int8, generator=g)
                d["v"] = torch.randint(-127, 128, (B, T, Hkv, D), device="cuda", dtype=torch.int8, generator=g)
                d["k_scale"] = (torch.rand((B, n_groups, Hkv, D), device="cuda", generator=g) * 0.04 + 0.005).half()
                d["v_scale"] = (torch.rand((B, T, Hkv), device="cuda", generator=g) * 0.04 + 0.005).half()
                d["k_resid"] = torch.randn((B, residual, Hkv, D), device="cuda", dtype=tdt, generator=g)
                d["v_resid"] = torch.randn((B, residual, Hkv, D), device="cuda", dtype=tdt, generator=g)
            self.sets.append(d)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        self.out = torch.empty(qshape, dtype=torch.float32, device="cuda")
        self.lse = torch.empty(qshape[:-1], dtype=torch.float32, device="cuda")
        self.order = None
        self.make_all_args()
        self.stream = torch.cuda.current_stream().cuda_stream
        ka.decode_attn_workspace_init(self.plan, self.ws, self.ws_bytes, self.stream)
        # ---- algorithmic bytes: what the method must move once ----
        self.kv_bytes, self.split_bytes, self.call_bytes = algorithmic_bytes(
            kind, B, Hq, Hkv, D, self.lens, self.S, eb=eb, mask=mask, hidden=hidden, C=C,
            residual=residual, k_group=k_group, page_size=page_size)

    def replan(self, num_splits):
        """Plan the same buffers for another split count (fresh workspace,
        arguments and byte count)."""
        ka, torch = self.ka, self.torch
        self.prob.num_splits = num_splits
        _, self.plan, self.ws_bytes, _ = ka.decode_attn_plan(ka.problem_from(self.prob))
        S_old, self.S = self.S, self.plan.num_splits
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        self.make_all_args()
        ka.decode_attn_workspace_init(self.plan, self.ws, self.ws_bytes, self.stream)
        d_ws = self.B * self.prob.num_queries * self.Hq * (self.S - S_old) * (self.D + 2) * 4
        self.split_bytes += d_ws
        self.call_bytes += 2 * d_ws
        return self

    def sweep(self, splits, steps=30, warmup=5):
        """Per-call time of decode_attn_forward for each split count (0:
        the planner's choice), restoring the original plan afterwards."""
        S0 = self.prob.num_splits
        out = []
        for S in splits:
            self.replan(S)
            ms = self.time(self.fwd, steps, warmup)
            gbs = self.call_bytes / (ms * 1e-3) / 1e9
            out.append({"requested": S, "num_splits": self.S, "chunk": self.plan.chunk,
                        "us_per_call": round(ms * 1000, 2), "GBs": round(gbs, 1),
                        "pct_of_peak": round(100 * gbs / PEAK_GBS, 1)})
        self.replan(S0)
        return out

    def host_buffers(self):
        """Input set 0 copied to host arrays in the oracle's storage formats
        (bf16 as uint16 bit patterns, fp16 scales as float16)."""
        import numpy as np
        torch = self.torch
        out = {"seq_lens": self.seq_lens.cpu().numpy()}
        for k, t in self.sets[0].items():
            if t.dtype == torch.bfloat16:
                out[k] = t.view(torch.int16).cpu().numpy().view(np.uint16)
            else:
                out[k] = t.cpu().numpy()
        return out

    def make_all_args(self):
        ka = self.ka
        self.args = [ka.make_args(d["q"], d["k"], d["v"], self.seq_lens, self.ws, self.ws_bytes,
                                  k_scale=d.get("k_scale"), v_scale=d.get("v_scale"),
                                  k_resid=d.get("k_resid"), v_resid=d.get("v_resid"),
                                  block_table=d.get("block_table"), work_order=self.order,
                                  mask_intervals=self.mask_iv, mask_summary=self.mask_sum,
                                  partition=getattr(self, "part", None),
                                  partition_items=getattr(self, "part_items", 0))
                     for d in self.sets]

    def use_schedule(self, on=True):
        """Largest-first work order from the host lengths (decode_attn_schedule)."""
        torch = self.torch
        self.order = (torch.from_numpy(self.ka.decode_attn_schedule(self.plan, self.lens)).to("cuda")
                      if on else None)
        self.make_all_args()

    def use_partition(self, items_per_head=0):
        """Balanced partition of the batch from the host lengths (decode_attn_partition)."""
        torch = self.torch
        part, items = self.ka.decode_attn_partition(self.plan, self.lens, items_per_head)
        self.part, self.part_items = torch.from_numpy(part).to("cuda"), items
        self.make_all_args()
        # the states a partitioned run writes (and the combine reads): one per
        # request piece and query head, instead of B*H_q*S
        B, L = self.B, int(part[1])
        P = [int(x) for x in part[4:5 + B]]
        pieces = sum((P[b + 1] - 1) // L - P[b] // L + 1 for b in range(B) if P[b + 1] > P[b])
        ws_old = B * self.Hq * self.S * (self.D + 2) * 4
        ws_new = pieces * self.Hq * (self.D + 2) * 4
        self.split_bytes += ws_new - ws_old
        self.call_bytes += 2 * (ws_new - ws_old)
        return self

    def run(self, i):
        self.ka.decode_attn_run(self.plan, self.args[i % self.nsets], self.stream)

    def call(self, i):
        """Two launches: split kernel, then combine kernel."""
        self.ka.decode_attn_run(self.plan, self.args[i % self.nsets], self.stream)
        self.ka.decode_attn_combine(self.plan, self.ws, self.ws_bytes, self.out, self.lse, self.stream)

    def fwd(self, i):
        """One launch: split kernel with the fused last-arrival reduction."""
        self.ka.decode_attn_forward(self.plan, self.args[i % self.nsets], self.out, self.lse,
                                    self.stream)

    def settle(self, fn, seconds=SETTLE_S):
        """Untimed calls for `seconds` of wall time.  After the GPU has idled
        (allocation, host work, the oracle) its clocks need several
        milliseconds of work to come back up: the first 200 calls of the
        headline workload run about 6 % slower than the next 200.  Every timed
        region therefore starts from steady state."""
        torch = self.torch
        t0 = time.perf_counter()
        i = 0
        while time.perf_counter() - t0 < seconds:
            for _ in range(50):
                fn(i)
                i += 1
            torch.cuda.synchronize()

    def time(self, fn, steps, warmup):
        torch = self.torch
        self.settle(fn)
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
        """Per-call event pairs for the sample statistics."""
        torch = self.torch
        self.settle(fn)
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
        return sorted(a.elapsed_time(b) * 1000.0 for a, b in evs)

    def _launch(self, fused, i, st):
        if fused:
            self.ka.decode_attn_forward(self.plan, self.args[i % self.nsets], self.out, self.lse, st)
        else:
            self.ka.decode_attn_run(self.plan, self.args[i % self.nsets], st)
            self.ka.decode_attn_combine(self.plan, self.ws, self.ws_bytes, self.out, self.lse, st)

    def graph_time(self, fused, calls_per_graph=20, replays=10):
        """Declared hipGraph replay of `calls_per_graph` calls (rotating input
        sets): the GPU-side time per call without host launch costs."""
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            st = torch.cuda.current_stream().cuda_stream
            for i in range(3):
                self._launch(fused, i, st)
            side.synchronize()
            with torch.cuda.graph(graph, stream=side):
                st = torch.cuda.current_stream().cuda_stream
                for i in range(calls_per_graph):
                    self._launch(fused, i, st)
        torch.cuda.current_stream().wait_stream(side)
        graph.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (replays * calls_per_graph)

    def report(self, name, config, steps=30, warmup=5):
        ms = self.time(self.fwd, steps, warmup)
        ms2 = self.time(self.call, steps, warmup)
        gbs = self.call_bytes / (ms * 1e-3) / 1e9
        return {"config": config, "num_splits": self.S, "us_per_call": round(ms * 1000, 2),
                "GBs": round(gbs, 1), "pct_of_peak": round(100 * gbs / PEAK_GBS, 1),
                "two_launch_us_per_call": round(ms2 * 1000, 2),
                "algorithmic_bytes": self.call_bytes,
                "samples_us": sample_stats(self.samples(self.fwd, 100, 10))}


def oracle_timing(w, us_gpu, runs, single_thread=False):
    """The fp64 NumPy oracle on input set 0 of a timed workload: wall clock
    per call (median of `runs`), its algorithmic GB/s and the GPU speedup;
    with `single_thread` also the same with the BLAS pool limited to one
    thread."""
    import oracle
    buf = w.host_buffers()

    def med():
        ts = []
        for _ in range(runs):
            t0 = time.perf_counter()
            oracle.attend(w.prob, buf)
            ts.append(time.perf_counter() - t0)
        return sorted(ts)[len(ts) // 2]

    t = med()
    r = {"runs": runs, "s_per_call": round(t, 6), "GBs": round(w.call_bytes / t / 1e9, 3),
         "gpu_speedup": round(t / (us_gpu * 1e-6), 1)}
    if single_thread:
        try:
            import threadpoolctl
            with threadpoolctl.threadpool_limits(1):
                t1 = med()
            r["single_thread_s_per_call"] = round(t1, 6)
            r["single_thread_gpu_speedup"] = round(t1 / (us_gpu * 1e-6), 1)
        except ImportError:
            pass
    return r


# oracle runs per workload when the CPU leg is on: median of 3 for the small
# and int8 workloads, one call for the two largest
ORACLE_RUNS = {"tiny_fp32": 3, "int8_sink_window": 3, "long_context_128k": 1, "paged_ragged": 1}


def _with_oracle(w, r, oracle_runs, single_thread=False):
    if oracle_runs:
        r["oracle"] = oracle_timing(w, r["us_per_call"], oracle_runs, single_thread)
    return r


def other_workload(torch, ka, name, steps=30, warmup=5, oracle_runs=0):
    """Timing report of one of the non-headline workloads; with `oracle_runs`
    the report also carries the oracle's time on input set 0 ("oracle")."""
    import synth
    if name == "long_context_128k":
        w = GpuWorkload(torch, ka, "contig", 1, 32, 8, 128, [131072], min_bytes=600 << 20, seed=1)
        return _with_oracle(w, w.report("long", "B=1 H_q=32 H_kv=8 d=128 T=131072 bf16 contiguous causal, "
                                                "auto splits", steps, warmup), oracle_runs)
    if name == "paged_ragged":
        lens = synth.ragged_lengths(0, 32).tolist()
        w = GpuWorkload(torch, ka, "paged", 32, 32, 8, 128, lens, seed=2)
        fixed = w.time(w.fwd, steps, warmup)
        w.use_schedule()
        scheduled = w.time(w.fwd, steps, warmup)
        w.use_schedule(False)
        w.use_partition()
        r = w.report("paged", "B=32 H_q=32 H_kv=8 d=128 bf16 P=16 T~U[1,32768] (seed 0), permuted pool, "
                              "balanced partition from decode_attn_partition (equal visible rows per "
                              "workgroup)", steps, warmup)
        r["partition_items_per_head"] = w.part_items
        r["fixed_splits_us_per_call"] = round(fixed * 1000, 2)
        r["fixed_splits_largest_first_us_per_call"] = round(scheduled * 1000, 2)
        return _with_oracle(w, r, oracle_runs)
    if name == "int8_sink_window":
        w = GpuWorkload(torch, ka, "i8", 16, 32, 8, 128, [16384] * 16, min_bytes=600 << 20, seed=3,
                        mask=(4, 4096))
        r = w.report("int8", "B=16 H_q=32 H_kv=8 d=128 T=16384 int8 K/V + bf16 residual "
                             "128, 4 sinks + window 4096", steps, warmup)
        r["code_pattern_probe"] = i8_pattern_probe(torch, w, 4096)
        return _with_oracle(w, r, oracle_runs)
    if name == "int8_ragged":
        lens = synth.ragged_lengths(4, 32, 1, 16384).tolist()
        w = GpuWorkload(torch, ka, "i8", 32, 32, 8, 128, lens, min_bytes=600 << 20, seed=9)
        fixed = w.time(w.fwd, steps, warmup)
        w.use_partition()
        r = w.report("int8r", "B=32 H_q=32 H_kv=8 d=128 int8 K/V + bf16 residual 128, causal, "
                              "T~U[1,16384] (seed 4), balanced partition from decode_attn_partition",
                     steps, warmup)
        r["partition_items_per_head"] = w.part_items
        r["fixed_splits_us_per_call"] = round(fixed * 1000, 2)
        return r
    layer = "B=8 H_q=32 H_kv=8 d=128 S_k=4096 bf16"
    if name == "few_query_c2":
        w = GpuWorkload(torch, ka, "contig", 8, 32, 8, 128, [4096] * 8, min_bytes=600 << 20, seed=6, C=2)
        return w.report("fewq", layer + " contiguous, C=2 query rows per request (bottom-right causal)",
                        steps, warmup)
    if name == "hnd_layout":
        w = GpuWorkload(torch, ka, "contig", 8, 32, 8, 128, [4096] * 8, min_bytes=600 << 20, seed=7, hnd=True)
        return w.report("hnd", layer + " contiguous HND [B, H_kv, T, d], causal", steps, warmup)
    if name == "flashmask":
        w = GpuWorkload(torch, ka, "contig", 8, 32, 8, 128, [4096] * 8, min_bytes=600 << 20, seed=8,
                        flashmask=True)
        r = w.report("fm", layer + " contiguous, FlashMask column intervals (seeded runs of closed "
                             "documents, visible blocks and scattered hidden keys)", steps, warmup)
        r["visible_kv_bytes"] = w.kv_bytes
        r["nonskip_tile_kv_bytes"] = flashmask_loaded_bytes(w)
        return r
    if name == "tiny_fp32":
        w = GpuWorkload(torch, ka, "contig", 1, 4, 4, 64, [256], num_splits=4, seed=4, dtype="f32")
        return _with_oracle(w, w.report("tiny", "B=1 H_q=H_kv=4 d=64 T=256 fp32 contiguous, S=4", steps,
                                        warmup), oracle_runs, single_thread=True)
    raise ValueError(name)


def i8_pattern_probe(torch, w, window, steps=100, warmup=10):
    """The int8 split kernel's code loads without its arithmetic
    (hbm_probe.hip i8_pattern_kernel) over the window's K and V codes of the
    workload's input sets, with its grid: the read ceiling of that access
    pattern (the sinks, residual rows and scales, a few percent of the bytes,
    left out)."""
    import ctypes
    L = ctypes.CDLL(os.path.join(ROOT, "kv_cache_amd", "libhbm_probe.so"))
    L.hbm_probe_i8_pattern.argtypes = [ctypes.c_void_p, ctypes.c_void_p] + [ctypes.c_int] * 6 + \
        [ctypes.c_void_p, ctypes.c_void_p]
    T = max(w.lens)
    S = w.S
    chunk = -(-window // S)
    sink = torch.empty(w.B * w.Hkv * S, dtype=torch.int32, device="cuda")

    def call(i):
        d = w.sets[i % w.nsets]
        assert L.hbm_probe_i8_pattern(d["k"].data_ptr(), d["v"].data_ptr(), w.B, T, w.Hkv, S, chunk, window,
                                      sink.data_ptr(), w.stream) == 0
    ms = w.time(call, steps, warmup)
    nbytes = 2 * w.B * w.Hkv * window * w.D
    return {"us_per_launch": round(ms * 1000, 2), "GBs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "code_bytes": nbytes, "grid": w.B * w.Hkv * S, "chunk": chunk}


def flashmask_loaded_bytes(w):
    """K and V bytes of the rows the kernel loads under FlashMask: the rows
    (< T_b) of every 16-key tile its block summary does not mark SKIP for the
    decode row q = T_b - 1 (all columns hidden by one interval family: q at or
    past the family's largest start and before its smallest end)."""
    import numpy as np
    sm = w.mask_sum.cpu().numpy()          # [B, nblk, 2, 4]: per family (start min, max, end min, max)
    rows = 0
    for b, T in enumerate(w.lens):
        q = T - 1
        for j in range((T + 15) // 16):
            skip = any(q >= sm[b, j, f, 1] and q + 1 <= sm[b, j, f, 2] for f in range(2))
            if not skip:
                rows += min(16, T - 16 * j)
    return rows * w.Hkv * w.D * 2 * 2


def append_timing(torch, ka, B=16, Hkv=8, D=128, T=16384, G=128, R=128, steps=50):
    """decode_attn_append on the int8 cache shape of the sink+window workload
    (group-closing residual of R rows, K groups of G): one call where no
    request closes a group and one where every request closes one (its
    oldest G residual rows; the other R - G move down)."""
    import synth
    assert (T - R) % G == 0 and G > 28
    cap = T + R
    prob = synth.Problem(batch=B, num_q_heads=4 * Hkv, num_kv_heads=Hkv, head_dim=D, kv_format="i8",
                         kv_capacity=cap, max_seq_len=cap, k_group=G, residual_len=R,
                         residual_policy="groups")
    _, plan, _, _ = ka.decode_attn_plan(ka.problem_from(prob))
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    k = torch.randint(-127, 128, (B, cap, Hkv, D), device="cuda", dtype=torch.int8, generator=g)
    v = torch.randint(-127, 128, (B, cap, Hkv, D), device="cuda", dtype=torch.int8, generator=g)
    ks = (torch.rand((B, cap // G + 1, Hkv, D), device="cuda", generator=g) * 0.04 + 0.005).half()
    vs = (torch.rand((B, cap, Hkv), device="cuda", generator=g) * 0.04 + 0.005).half()
    kr = torch.randn((B, R, Hkv, D), device="cuda", generator=g).bfloat16()
    vr = torch.randn((B, R, Hkv, D), device="cuda", generator=g).bfloat16()
    kn = torch.randn((B, Hkv, D), device="cuda", generator=g).bfloat16()
    vn = torch.randn((B, Hkv, D), device="cuda", generator=g).bfloat16()
    status = torch.zeros(B, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    out = {}
    # lengths before the append: residual R - 28 rows (no closure) / R rows (closure)
    for name, t in (("no_closure", T - 28), ("closure", T)):
        sl = torch.full((B,), t, dtype=torch.int32, device="cuda")
        call = lambda: ka.decode_attn_append(plan, kn, vn, k, v, ks, vs, kr, vr, sl, status, st)
        for _ in range(5):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            call()
        e1.record()
        torch.cuda.synchronize()
        out[name + "_us"] = round(e0.elapsed_time(e1) / steps * 1000, 2)
    assert int(status.max()) == 0
    out["config"] = (f"B={B} H_kv={Hkv} d={D} int8 cache T={T}, G={G}, R={R}; closure = quantize "
                     f"the oldest {G} residual rows per (b, h_kv) (K per channel, V per row)"
                     + (f" and move the other {R - G} down" if R > G else ""))
    return out


def hbm_probe(torch, nbytes=512 << 20):
    """Practical read ceiling of the box: a plain streaming-read kernel; then
    one copy of known size, the reference for the profiler's byte counters."""
    import ctypes
    L = ctypes.CDLL(os.path.join(ROOT, "kv_cache_amd", "libhbm_probe.so"))
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
    L.hbm_probe_copy(bufs[0].data_ptr(), bufs[1].data_ptr(), 256 << 20, 2048, st)
    torch.cuda.synchronize()
    del bufs
    return read_gbs


def pattern_probe(torch, w, steps=100, warmup=10, stamp_calls=20):
    """The split kernel's read pattern without its arithmetic (hbm_probe.hip
    pattern_kernel) on the headline workload's input sets, same grid and
    split length: the read ceiling of that access pattern on this machine, and
    its per-XCD completion (the median over calls of each XCD's last
    workgroup end, counted from the earliest workgroup end).  Then the same
    bytes read in address order (hbm_probe.hip read2_kernel): the ceiling of
    one launch that reads them, whatever its pattern."""
    import ctypes
    import numpy as np
    L = ctypes.CDLL(os.path.join(ROOT, "kv_cache_amd", "libhbm_probe.so"))
    L.hbm_probe_pattern.argtypes = [ctypes.c_void_p, ctypes.c_void_p] + [ctypes.c_int] * 5 + \
        [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    T = max(w.lens)
    grid = w.B * w.Hkv * w.S
    sink = torch.empty(grid, dtype=torch.int32, device="cuda")
    st = torch.zeros((grid, 2), dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def call(i, stamps=None):
        d = w.sets[i % w.nsets]
        rc = L.hbm_probe_pattern(d["k"].data_ptr(), d["v"].data_ptr(), w.B, T, w.Hkv, w.S, w.plan.chunk,
                                 sink.data_ptr(), stamps, stream)
        assert rc == 0
    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        call(i)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / steps * 1000
    ends = []
    for i in range(stamp_calls):
        call(i, st.data_ptr())
        torch.cuda.synchronize()
        a = st.cpu().numpy().view(np.uint64)
        e = (a[:, 0] - a[:, 0].min()).astype(np.float64) / 100.0      # 100 MHz counter -> us
        x = a[:, 1].astype(int)
        ends.append([float(e[x == k].max()) if (x == k).any() else 0.0 for k in range(8)])
    kv = 2 * w.B * T * w.Hkv * w.D * 2
    # the same K and V bytes read in address order (grid-stride, 1024 workgroups)
    L.hbm_probe_read2.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                  ctypes.c_int, ctypes.c_void_p]
    sink2 = torch.empty(1024, dtype=torch.int32, device="cuda")

    def call2(i):
        d = w.sets[i % w.nsets]
        assert L.hbm_probe_read2(d["k"].data_ptr(), d["v"].data_ptr(), kv // 2, sink2.data_ptr(), 1024,
                                 stream) == 0
    for i in range(warmup):
        call2(i)
    e0.record()
    for i in range(steps):
        call2(i)
    e1.record()
    torch.cuda.synchronize()
    us2 = e0.elapsed_time(e1) / steps * 1000
    return {"us_per_launch": round(us, 2), "GBs": round(kv / (us * 1e-6) / 1e9, 1), "bytes": kv,
            "grid": grid, "chunk": w.plan.chunk,
            "xcd_last_end_spread_us_median": [round(float(np.median([c[k] for c in ends])), 2) for k in range(8)],
            "contiguous_read": {"us_per_launch": round(us2, 2), "GBs": round(kv / (us2 * 1e-6) / 1e9, 1),
                                "grid": 1024}}


def host_info():
    """Core counts and CPU model of the host the oracle ran on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)), "model": model}


def cpu_baseline(call_bytes, seconds: float = 10.0):
    """The fp64 NumPy oracle on the headline workload shape (seeded synth
    data), repeated until about `seconds` of wall clock have passed."""
    import oracle
    import synth
    w = synth.make_contiguous(0, 8, 32, 8, 128, [4096] * 8)
    calls = 0
    t0 = time.perf_counter()
    while True:
        oracle.attend(w.problem, w.buffers)
        calls += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    threads = 1
    try:
        import threadpoolctl
        threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] or [1])
    except Exception:
        pass
    return {"value": round(call_bytes * calls / dt / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "s_per_call": round(dt / calls, 4),
            "sample": f"{calls} full calls of the headline workload (fp64 NumPy oracle, seed 0), "
                      f"{dt:.1f} s wall"}


def headline(torch, ka, num_splits=0):
    """The Llama-3-8B-shaped layer: B=8, H_q=32, H_kv=8, d=128, S_k=4096, bf16."""
    return GpuWorkload(torch, ka, "contig", 8, 32, 8, 128, [4096] * 8, num_splits=num_splits,
                       min_bytes=600 << 20, seed=0)


def make_workload(torch, ka, name):
    """Device workload of one of the named timed workloads (for --stamps)."""
    import synth
    if name == "llama3_8b_layer":
        return headline(torch, ka)
    if name == "long_context_128k":
        return GpuWorkload(torch, ka, "contig", 1, 32, 8, 128, [131072], min_bytes=600 << 20, seed=1)
    if name == "int8_sink_window":
        return GpuWorkload(torch, ka, "i8", 16, 32, 8, 128, [16384] * 16, min_bytes=600 << 20, seed=3,
                           mask=(4, 4096))
    if name == "paged_ragged":
        return GpuWorkload(torch, ka, "paged", 32, 32, 8, 128, synth.ragged_lengths(0, 32).tolist(), seed=2)
    raise ValueError(name)


def stamps_summary(torch, ka, name, calls=20, warmup=5):
    """Per-workgroup timestamps of decode_attn_forward's launches
    (decode_attn_timestamps) over `calls` calls: when workgroups start and
    store their states, how the 8 XCDs finish, and how long the folds take."""
    import numpy as np
    w = make_workload(torch, ka, name)
    grid = w.B * w.Hkv * w.S
    st = torch.zeros((grid, 4), dtype=torch.int64, device="cuda")
    rows = []
    hz = 0
    for i in range(warmup + calls):
        _, hz = ka.decode_attn_timestamps(w.plan, w.args[i % w.nsets], w.out, w.lse, st, w.stream)
        torch.cuda.synchronize()
        if i >= warmup:
            rows.append(st.cpu().numpy().view(np.uint64).copy())
    us = 1e6 / hz
    res = {"workload": name, "num_splits": w.S, "workgroups": grid, "clock_hz": hz, "calls": calls}
    per = []
    for a in rows:
        t0 = a[:, 0].min()
        start, stored, end = ((a[:, k] - t0) * us for k in range(3))
        xcc = (a[:, 3] & 0xF).astype(int)
        hw = ((a[:, 3] >> 8) & 0xFFFFFFFF).astype(np.int64)
        folded = (a[:, 3] >> 63).astype(bool)
        # (XCC, SE_ID, SH_ID, CU_ID) from HW_ID: CU_ID bits 8..11, SH_ID 12, SE_ID 13..15
        cu = ((hw >> 8) & 0x1F) | (((hw >> 13) & 0x7) << 5) | (xcc.astype(np.int64) << 8)
        per.append({"span": float(end.max()), "last_start": float(start.max()),
                    "stored_median": float(np.median(stored)), "stored_max": float(stored.max()),
                    "xcd_last_store": [float(stored[xcc == x].max()) if (xcc == x).any() else 0.0
                                       for x in range(8)],
                    "xcd_wgs": [int((xcc == x).sum()) for x in range(8)],
                    "cu_last_store_p10_p90": [float(np.percentile([stored[cu == c].max() for c in np.unique(cu)], q))
                                              for q in (10, 90)],
                    "fold_us_median": float(np.median((end - stored)[folded])) if folded.any() else None,
                    "fold_us_max": float((end - stored)[folded].max()) if folded.any() else None,
                    # the workgroups that did not fold: store wait + arrival atomic only
                    "arrival_us_median": float(np.median((end - stored)[~folded])) if (~folded).any() else None,
                    # the first fold on each XCD (the fold code's first run there)
                    "first_fold_us": float(np.median([(end - stored)[m][np.argmin(stored[m])] for m in
                                                      (folded & (xcc == x) for x in range(8)) if m.any()]))
                    if folded.any() else None,
                    "end_after_last_store": float(end.max() - stored.max()),
                    "cus": int(len(np.unique(cu)))})
    med = lambda k: round(float(np.median([p[k] for p in per])), 2)
    res.update({k: med(k) for k in ("span", "last_start", "stored_median", "stored_max",
                                    "end_after_last_store", "cus")})
    res["xcd_last_store_median"] = [round(float(np.median([p["xcd_last_store"][x] for p in per])), 2)
                                    for x in range(8)]
    res["xcd_workgroups"] = per[0]["xcd_wgs"]
    res["cu_last_store_p10_p90_median"] = [round(float(np.median([p["cu_last_store_p10_p90"][j] for p in per])), 2)
                                           for j in range(2)]
    if per[0]["fold_us_median"] is not None:
        res["fold_us_median"] = med("fold_us_median")
        res["fold_us_max_median"] = med("fold_us_max")
        res["first_fold_on_xcd_us_median"] = med("first_fold_us")
    if per[0]["arrival_us_median"] is not None and per[0]["fold_us_median"] is not None:
        res["arrival_us_median"] = med("arrival_us_median")
    return res


def summarize(a):
    """Write profiles/<workload>_kernel_trace.md from a rocprofv3 --stats
    kernel summary (and, when given, FETCH_SIZE / WRITE_SIZE counter passes
    calibrated by the probe's 256 MiB copy), with a machine-readable block
    that the bench line reads back."""
    import csv
    import re
    import statistics

    def short(n):
        n = n.replace("(anonymous namespace)::", "").replace("void ", "")
        return re.sub(r"\bda::", "", re.sub(r"\(.*", "", n))

    def one(d, suffix):
        for root, _, files in os.walk(d):
            for f in files:
                if f.endswith(suffix):
                    return os.path.join(root, f)
        raise FileNotFoundError(f"{suffix} under {d}")
    def ours(name):       # this library's kernels and the probe's (not torch's input generation)
        return bool(re.search(r"\bda::", name)) or any(
            k in name for k in ("read_kernel", "copy_kernel", "pattern_kernel", "zero_words"))
    stats = [r for r in csv.DictReader(open(one(a.trace, "kernel_stats.csv"))) if ours(r["Name"])]
    kernels = {short(r["Name"]): {"calls": int(r["Calls"]), "avg_ns": float(r["AverageNs"]),
                                  "min_ns": float(r["MinNs"]), "max_ns": float(r["MaxNs"]),
                                  "std_ns": float(r["StdDev"])} for r in stats}
    dom = DOMINANT[a.summarize]
    dominant = [k for k in kernels if k.startswith(dom)]
    line = None
    if a.bench_log:
        for ln in open(a.bench_log):
            if ln.startswith("{"):
                line = json.loads(ln)
    rec = {"workload": a.summarize, "kernel_source_hash": a.source_hash or kernel_source_hash(),
           "dominant": dominant[0] if dominant else dom, "kernels": kernels,
           "num_splits": a.num_splits}
    traffic_txt = ""
    if a.fetch and a.write:
        def counters(d):
            g = {}
            for r in csv.DictReader(open(one(d, "counter_collection.csv"))):
                g.setdefault(short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
            return g
        fetch, write = counters(a.fetch), counters(a.write)
        copy_kib = 256 * 1024
        rf = copy_kib / statistics.median(fetch["copy_kernel"])
        wf = copy_kib / statistics.median(write["copy_kernel"])
        fk = statistics.median(fetch[rec["dominant"]])
        wk = statistics.median(write[rec["dominant"]])
        hbm = int(round((fk * rf + wk * wf) * 1024))
        rec["traffic"] = {"fetch_kib": fk, "write_kib": wk, "fetch_factor": round(rf, 4),
                          "write_factor": round(wf, 4), "hbm_bytes_per_launch": hbm,
                          "commands": a.pmc_command}
        traffic_txt = (f"\nCounters (FETCH_SIZE, WRITE_SIZE; KiB per dispatch, medians) of `{rec['dominant']}`: "
                       f"{fk:.1f} / {wk:.1f}.  Calibration: the probe's copy of 256 MiB reads "
                       f"{statistics.median(fetch['copy_kernel']):.0f} / writes {statistics.median(write['copy_kernel']):.0f} KiB "
                       f"-> factors {rf:.3f} / {wf:.3f}.  HBM bytes per launch: {hbm}.\n\nCounter commands:\n\n"
                       + "".join(f"    {c}\n" for c in a.pmc_command))
    out = os.path.join(PROFILES, f"{a.summarize}_kernel_trace.md")
    with open(out, "w") as f:
        f.write(f"# Kernel trace: {a.title}\n\nCommand:\n\n    {a.trace_command}\n\n")
        f.write("rocprofv3 --kernel-trace --stats summary (durations in ns):\n\n"
                "| kernel | calls | average | min | max | stddev |\n|---|---|---|---|---|---|\n")
        for k, v in kernels.items():
            f.write(f"| `{k}` | {v['calls']} | {v['avg_ns']:.0f} | {v['min_ns']:.0f} | {v['max_ns']:.0f} | "
                    f"{v['std_ns']:.0f} |\n")
        f.write(f"\nDominant kernel: `{rec['dominant']}`; kernel sources hash {rec['kernel_source_hash']}; "
                f"{a.num_splits} splits.\n")
        if line:
            f.write(f"\nbench.py line of the same run: {json.dumps(line.get(a.summarize, line))[:600]}\n")
        f.write(traffic_txt)
        if a.variant_trace:
            vst = [r for r in csv.DictReader(open(one(a.variant_trace, "kernel_stats.csv"))) if ours(r["Name"])]
            f.write(f"\n## Variant: {a.variant_label}\n\nCommand:\n\n    {a.variant_command}\n\n"
                    "| kernel | calls | average | min | max | stddev |\n|---|---|---|---|---|---|\n")
            for r in vst:
                f.write(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                        f"{float(r['MinNs']):.0f} | {float(r['MaxNs']):.0f} | {float(r['StdDev']):.0f} |\n")
        f.write(f"\n<!-- bench-data {json.dumps(rec)} -->\n")
    print(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-sweep", action="store_true", help="skip the split-count sweeps")
    names = ["llama3_8b_layer", "long_context_128k", "paged_ragged", "int8_sink_window", "tiny_fp32",
             "few_query_c2", "hnd_layout", "flashmask", "int8_ragged"]
    ap.add_argument("--only", default=None, choices=names,
                    help="time one workload alone and print its report (for profiling)")
    ap.add_argument("--stamps", default=None, choices=list(DOMINANT),
                    help="per-workgroup timestamps of one workload's forward launches (JSON)")
    ap.add_argument("--samples-out", default=None, help="write raw per-call samples (JSON)")
    ap.add_argument("--summarize", default=None, choices=list(DOMINANT),
                    help="write profiles/<workload>_kernel_trace.md from rocprofv3 output (no GPU)")
    ap.add_argument("--trace", help="--summarize: directory of the --kernel-trace --stats run")
    ap.add_argument("--fetch", help="--summarize: directory of the FETCH_SIZE counter run")
    ap.add_argument("--write", help="--summarize: directory of the WRITE_SIZE counter run")
    ap.add_argument("--bench-log", help="--summarize: log holding the profiled run's JSON line")
    ap.add_argument("--title", default="", help="--summarize: title")
    ap.add_argument("--trace-command", default="", help="--summarize: the profiled command")
    ap.add_argument("--pmc-command", action="append", default=[], help="--summarize: counter commands")
    ap.add_argument("--source-hash", default=None,
                    help="--summarize: kernel sources hash of the profiled run (default: the tree's)")
    ap.add_argument("--variant-trace", help="--summarize: kernel-trace directory of a library variant")
    ap.add_argument("--variant-label", default="", help="--summarize: what the variant changes")
    ap.add_argument("--variant-command", default="", help="--summarize: the variant's commands")
    a = ap.parse_args()
    if a.summarize:
        a.num_splits = a.num_splits or 0
        summarize(a)
        return
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode path has no multi-GPU mode "
              "(it shards by request and K/V head with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import kv_cache_amd as ka
    ka.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if a.stamps:
        print(json.dumps({"stamps": stamps_summary(torch, ka, a.stamps)}), flush=True)
        return
    if a.only == "llama3_8b_layer":
        hbm_probe(torch)      # the copy of known size that calibrates the byte counters
        w = headline(torch, ka, a.num_splits)
        print(json.dumps({a.only: w.report("llama", "headline", a.steps, a.warmup)}), flush=True)
        return
    if a.only:
        if a.only in ("long_context_128k", "int8_sink_window", "paged_ragged"):
            hbm_probe(torch)
        print(json.dumps({a.only: other_workload(torch, ka, a.only, a.steps, a.warmup)}), flush=True)
        return

    ceiling = hbm_probe(torch)
    w = headline(torch, ka, a.num_splits)
    torch.cuda.synchronize()
    ms_call = w.time(w.fwd, a.steps, a.warmup)         # timed region: K steps
    ms_two = w.time(w.call, a.steps, a.warmup)          # run + combine, same stream
    ms_split = w.time(w.run, a.steps, a.warmup)         # split kernel alone, same stream
    samples = w.samples(w.fwd, 100, 10)
    ms_graph = w.graph_time(True)
    ms_graph_two = w.graph_time(False)
    value = w.call_bytes / (ms_call * 1e-3) / 1e9
    # The dominant kernel is the forward launch itself: one kernel moves every
    # algorithmic byte of the call.  Its roofline is reported from the HIP
    # events of the timed region and from the committed rocprofv3 summary of
    # the same kernel (when taken on these sources); the headline is the lower.
    event = {"us_per_launch": round(ms_call * 1000, 2), "achieved": round(value, 1),
             "frac": round(value / PEAK_GBS, 4)}
    prof, why = profiled_roofline("llama3_8b_layer", w.call_bytes, w.S)
    achieved = min(value, prof["achieved"]) if prof else value

    line = {
        "metric": "decode-attn us/call + achieved HBM GB/s (% of peak), GQA 32q/8kv d128",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_call, 5),
        "us_per_call": round(ms_call * 1000, 2),
        "pct_of_peak": round(100 * value / PEAK_GBS, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, rotated input sets > 512 MiB)",
        "config": {"workload": "llama3-8b-layer decode: B=8 H_q=32 H_kv=8 d=128 S_k=4096 bf16 "
                               "contiguous causal, fp32 out",
                   "num_splits": w.S, "chunk": w.plan.chunk, "input_sets": w.nsets,
                   "algorithmic_bytes_per_call": w.call_bytes},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBS, 4),
                     "traffic": prof.get("traffic") if prof else None,
                     "kernel": DOMINANT["llama3_8b_layer"],
                     "algorithmic_bytes_per_launch": w.call_bytes,
                     "event": event, "profiled": prof if prof else {"unavailable": why}},
        "samples_us": sample_stats(samples),
        "samples_raw_us": [round(x, 2) for x in samples],
        "graph_replay_us_per_call": round(ms_graph * 1000, 2),
        "two_launch": {"us_per_call": round(ms_two * 1000, 2),
                       "split_kernel_us": round(ms_split * 1000, 2),
                       "split_kernel_GBs": round(w.split_bytes / (ms_split * 1e-3) / 1e9, 1),
                       "graph_replay_us_per_call": round(ms_graph_two * 1000, 2)},
        "hbm_read_probe_GBs": round(ceiling, 1),
        "pattern_probe": pattern_probe(torch, w),
        "kernel_source_hash": kernel_source_hash(),
    }
    if a.samples_out:
        with open(a.samples_out, "w") as f:
            json.dump({"per_call_us": samples}, f)
    if not a.no_sweep:
        sweep = {"llama3_8b_layer": w.sweep([1, 2, 4, 8, 12, 16, 24, 32, 0])}
    call_bytes = w.call_bytes
    cpu = not a.no_cpu_baseline
    per_config = {}
    if cpu:
        per_config["llama3_8b_layer"] = oracle_timing(w, ms_call * 1000, 3, single_thread=True)
    del w
    if not a.no_sweep:
        wl = make_workload(torch, ka, "long_context_128k")
        sweep["long_context_128k"] = wl.sweep([1, 8, 32, 128, 0], steps=10, warmup=3)
        del wl
        w8 = make_workload(torch, ka, "int8_sink_window")
        sweep["int8_sink_window"] = w8.sweep([2, 3, 4, 6, 8, 12, 16, 0], steps=50, warmup=5)
        del w8
        line["split_sweep"] = sweep
    if not a.no_long:
        others = {name: other_workload(torch, ka, name, oracle_runs=ORACLE_RUNS[name] if cpu else 0)
                  for name in ("long_context_128k", "paged_ragged", "int8_sink_window")}
        others["int8_append"] = append_timing(torch, ka)
        others["int8_append_g32_r128"] = append_timing(torch, ka, G=32, R=128)
        others["tiny_fp32"] = other_workload(torch, ka, "tiny_fp32",
                                             oracle_runs=ORACLE_RUNS["tiny_fp32"] if cpu else 0)
        for name in ("int8_ragged", "few_query_c2", "hnd_layout", "flashmask"):
            others[name] = other_workload(torch, ka, name)
        fmr = others["flashmask"]
        # the loaded tiles' bytes at the causal headline's achieved rate: what
        # the masked call would take if SKIP tiles cost nothing
        fmr["us_at_headline_rate"] = round(fmr["nonskip_tile_kv_bytes"] / (value * 1e3), 2)
        for name, r in others.items():
            if "oracle" in r:
                per_config[name] = r.pop("oracle")
        line["other_workloads"] = others
    torch.cuda.synchronize()
    if cpu:
        line["cpu_baseline"] = cpu_baseline(call_bytes)
        line["cpu_baseline"]["per_config"] = per_config
        line["cpu_baseline"]["host"] = host_info()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
