"""Moves synthetic workloads to the GPU and calls the library through the C
ABI (kv_cache_amd binding).  Torch provides device memory and the stream."""
from __future__ import annotations

import sys

import numpy as np

import kv_cache_amd as ka


def torch():
    import torch as _t
    return _t


def to_dev(arr: np.ndarray):
    t = torch()
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16 or a.dtype == np.float16:
        a = a.view(np.int16)
    return t.from_numpy(a).to("cuda")


def announce(*what):
    print("[gpu-case]", *what, file=sys.stderr, flush=True)


class DeviceWorkload:
    """Device copies of a synth.Workload's buffers (and an optional work order)."""

    def __init__(self, w):
        self.w = w
        self.dev = {k: to_dev(v) for k, v in w.buffers.items()}
        self.order = None

    def summarize_mask(self, plan):
        """FlashMask block summaries of the device intervals, by the library."""
        t = torch()
        p = self.w.problem
        nblk = (p.max_seq_len + 15) // 16
        self.dev["mask_summary"] = t.zeros((p.batch, nblk, 8), dtype=t.int32, device="cuda")
        ka.decode_attn_flashmask_summarize(plan, self.dev["mask_intervals"], self.dev["mask_summary"],
                                           t.cuda.current_stream().cuda_stream)
        t.cuda.synchronize()
        return self.dev["mask_summary"].cpu().numpy()

    def schedule(self, plan):
        """Use the library's largest-first work order for this plan."""
        lens = self.w.buffers["seq_lens"]
        self.order = to_dev(ka.decode_attn_schedule(plan, lens))

    def partition(self, plan, items_per_head=0):
        """Use the library's balanced partition of this batch for this plan."""
        lens = self.w.buffers["seq_lens"]
        part, items = ka.decode_attn_partition(plan, lens, items_per_head)
        self.part, self.part_items = to_dev(part), items
        return part, items

    def args(self, ws, ws_bytes):
        d = self.dev
        return ka.make_args(d["q"], d["k"], d["v"], d["seq_lens"], ws, ws_bytes,
                            k_scale=d.get("k_scale"), v_scale=d.get("v_scale"),
                            k_resid=d.get("k_resid"), v_resid=d.get("v_resid"),
                            block_table=d.get("block_table"), work_order=self.order,
                            indptr=d.get("indptr"), cache_batch_idx=d.get("cache_batch_idx"),
                            mask_intervals=d.get("mask_intervals"), mask_summary=d.get("mask_summary"),
                            partition=getattr(self, "part", None),
                            partition_items=getattr(self, "part_items", 0))


def _outputs(w):
    """NaN-filled O and LSE, [B, H_q, D] / [B, H_q] or with a query-row axis
    after B when the problem has C > 1 query rows."""
    t = torch()
    p = w.problem
    C = getattr(p, "num_queries", 1)
    lead = (p.batch,) if C == 1 else (p.batch, C)
    out = t.full(lead + (p.num_q_heads, p.head_dim), float("nan"), dtype=t.float32, device="cuda")
    lse = t.full(lead + (p.num_q_heads,), float("nan"), dtype=t.float32, device="cuda")
    return out, lse


def plan_for(w, num_splits=None, num_cus=0):
    """num_cus > 0 plans for that many CUs instead of the device's (the launch
    picks the int8 kernel's instance by workgroups per CU of the plan)."""
    p = w.problem
    if num_splits is not None:
        p.num_splits = num_splits
    _, plan, ws, _ = ka.decode_attn_plan(ka.problem_from(p, num_cus=num_cus))
    return plan, ws


def run(w, num_splits=None, dw=None, poison_ws=True, want_ws=False, stream=None, partition=None,
        num_cus=0):
    """Plan, run, combine.  Returns (O, LSE, plan[, workspace numpy]).
    partition: None (fixed splits) or a target item count per K/V head for the
    balanced partition (0: the library's default)."""
    t = torch()
    dw = dw or DeviceWorkload(w)
    plan, ws_bytes = plan_for(w, num_splits, num_cus)
    if partition is not None:
        dw.partition(plan, partition)
    elif getattr(dw, "part", None) is not None:
        dw.part, dw.part_items = None, 0
    ws = t.empty(max(ws_bytes, 16), dtype=t.uint8, device="cuda")
    if poison_ws:
        ws.fill_(0xFF)                  # NaN everywhere: unwritten slots would show
    out, lse = _outputs(w)
    s = stream if stream is not None else t.cuda.current_stream().cuda_stream
    ka.decode_attn_run(plan, dw.args(ws, ws_bytes), s)
    ka.decode_attn_combine(plan, ws, ws_bytes, out, lse, s)
    t.cuda.synchronize()
    res = (out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), plan)
    if want_ws:
        res = res + (ws.cpu().numpy(),)
    return res


def states_bytes(plan):
    p = plan.problem
    raw = p.batch * p.num_queries * p.num_q_heads * plan.num_splits * (p.head_dim_v + 2) * 4
    return (raw + 255) // 256 * 256


def forward(w, num_splits=None, dw=None, ws=None, want_ws=False, init=True, num_cus=0):
    """Plan and run the single-launch path (split kernel with the fused
    reduction).  A fresh workspace is filled with 0xFF (NaN states, counters
    garbage) and then initialised through decode_attn_workspace_init."""
    t = torch()
    dw = dw or DeviceWorkload(w)
    plan, ws_bytes = plan_for(w, num_splits, num_cus)
    if ws is None:
        ws = t.empty(max(ws_bytes, 16), dtype=t.uint8, device="cuda")
        ws.fill_(0xFF)
    out, lse = _outputs(w)
    s = t.cuda.current_stream().cuda_stream
    if init:
        ka.decode_attn_workspace_init(plan, ws, ws_bytes, s)
    ka.decode_attn_forward(plan, dw.args(ws, ws_bytes), out, lse, s)
    t.cuda.synchronize()
    res = (out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), plan)
    if want_ws:
        res = res + (ws,)
    return res


def counters(ws, plan):
    p = plan.problem
    off = states_bytes(plan)
    n = p.batch * p.num_kv_heads
    return ws[off: off + 4 * n].cpu().numpy().view(np.uint32)


def split_workspace(ws_bytes: np.ndarray, plan):
    p = plan.problem
    n = p.batch * p.num_q_heads * plan.num_splits
    f = ws_bytes[: n * (p.head_dim_v + 2) * 4].view(np.float32)
    u = f[: n * p.head_dim_v].reshape(p.batch, p.num_q_heads, plan.num_splits, p.head_dim_v)
    m = f[n * p.head_dim_v: n * p.head_dim_v + n].reshape(p.batch, p.num_q_heads, plan.num_splits)
    l = f[n * p.head_dim_v + n:].reshape(p.batch, p.num_q_heads, plan.num_splits)
    return u, m, l


def trace(w, num_splits=None, dw=None, forward=False, partition=None, num_cus=0):
    """Runs the trace instance of the timed kernels: decode_attn_run's (then
    the combine), or with ``forward`` decode_attn_forward's; ``partition`` as
    in run().  Returns (trace dict of [B, H_kv, max_visible] arrays, plan, O,
    LSE)."""
    t = torch()
    dw = dw or DeviceWorkload(w)
    plan, ws_bytes = plan_for(w, num_splits, num_cus)
    if partition is not None:
        dw.partition(plan, partition)
    elif getattr(dw, "part", None) is not None:
        dw.part, dw.part_items = None, 0
    ws = t.empty(max(ws_bytes, 16), dtype=t.uint8, device="cuda")
    ws.fill_(0xFF)
    s = t.cuda.current_stream().cuda_stream
    if forward:
        ka.decode_attn_workspace_init(plan, ws, ws_bytes, s)
    p = w.problem
    n = max(p.batch * p.num_kv_heads * plan.max_visible, 1)
    arr = dict(k_offset=t.full((n,), -1, dtype=t.int64, device="cuda"),
               v_offset=t.full((n,), -1, dtype=t.int64, device="cuda"),
               position=t.full((n,), -1, dtype=t.int32, device="cuda"),
               count=t.zeros((n,), dtype=t.int32, device="cuda"),
               k_scale_offset=t.full((n,), -1, dtype=t.int64, device="cuda"),
               v_scale_offset=t.full((n,), -1, dtype=t.int64, device="cuda"))
    out, lse = _outputs(w)
    if forward:
        ka.decode_attn_trace_indices(plan, dw.args(ws, ws_bytes), **arr, out=out, lse=lse, stream=s)
    else:
        ka.decode_attn_trace_indices(plan, dw.args(ws, ws_bytes), **arr, stream=s)
        ka.decode_attn_combine(plan, ws, ws_bytes, out, lse, s)
    t.cuda.synchronize()
    shape = (p.batch, p.num_kv_heads, plan.max_visible)
    m = p.batch * p.num_kv_heads * plan.max_visible
    res = {k: v.cpu().numpy()[:m].reshape(shape) for k, v in arr.items()}
    return res, plan, out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


ONCE = 1 + (1 << 16)     # one K row load and one V row load


def check_trace(w, tr, fm_partial=None, ref=None):
    """The rows the timed kernel loaded are exactly the oracle's visible rows,
    each once as K and once as V, at the oracle's offsets (element offsets in
    the buffer each row comes from; int8: also the K scale row and the V
    scale), in the slot of their visible ordinal.  FlashMask (slots are
    positions): hidden rows may be loaded only inside tiles the classifier
    calls PARTIAL; ``fm_partial(b, pos) -> bool`` says which.  ``ref``: the
    oracle's trace, if already computed."""
    if ref is None:
        _, _, ref = oracle_attend_trace(w)
    i8 = w.problem.kv_format == "i8"
    for (b, h), r in ref.items():
        pos = r["positions"]
        cnt = tr["count"][b, h]
        slots = pos if fm_partial is not None else np.arange(pos.size)
        assert np.all(cnt[slots] == ONCE), (b, h, "a visible row not loaded exactly once")
        other = np.ones(cnt.size, bool)
        other[slots] = False
        if fm_partial is None:
            assert not cnt[other].any(), (b, h, "a row outside the visible set was loaded")
        else:
            extra = np.nonzero(other & (cnt != 0))[0]
            assert np.all(cnt[extra] == ONCE)
            assert all(fm_partial(b, int(x)) for x in extra), (b, h, "hidden row outside PARTIAL tiles")
        assert np.array_equal(tr["position"][b, h][slots], pos), (b, h)
        assert np.array_equal(tr["k_offset"][b, h][slots], r["offsets"]), (b, h)
        assert np.array_equal(tr["v_offset"][b, h][slots], r["offsets"]), (b, h)
        if i8:
            assert np.array_equal(tr["k_scale_offset"][b, h][slots], r["k_scale_offsets"]), (b, h)
            assert np.array_equal(tr["v_scale_offset"][b, h][slots], r["v_scale_offsets"]), (b, h)
    return sum(r["positions"].size for r in ref.values())


def oracle_attend_trace(w):
    import oracle
    return oracle.attend(w.problem, w.buffers, with_trace=True)


def errors(O, L, Or, Lr):
    """(max|O - O_ref|, max|LSE - LSE_ref| over rows with a finite reference)."""
    fin = np.isfinite(Lr)
    lerr = float(np.max(np.abs(L[fin] - Lr[fin]))) if fin.any() else 0.0
    return max_abs(O, Or), lerr


def max_abs(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def check_rows(O, L, Or, Lr, atol, rtol=0.0, rows=None, lse_atol=None):
    """Field-aware comparison ("M4.5 ...", section 0x07G): same finite/all-
    masked policy, max|O - O_ref| <= atol + rtol * max|O_ref|, LSE exact for
    -inf and within tolerance otherwise.  The LSE tolerance is atol when an
    absolute output tolerance is given, else 1e-3: an LSE error d changes the
    normalizer by a factor e^d ~ 1 + d, a tenth of a 1e-2 relative budget."""
    if lse_atol is None:
        lse_atol = atol if atol > 0 else 1e-3
    if rows is not None:
        O = np.stack([O[b, h] for b, h in rows])
        Or = np.stack([Or[b, h] for b, h in rows])
        L = np.array([L[b, h] for b, h in rows])
        Lr = np.array([Lr[b, h] for b, h in rows])
    assert O.shape == Or.shape
    masked = np.isneginf(Lr)
    assert np.array_equal(np.isneginf(L), masked), "all-masked policy differs"
    if masked.any():
        assert np.all(O[masked] == 0) and not np.signbit(O[masked]).any()
    assert np.all(np.isfinite(O)), "non-finite output"
    bound = atol + rtol * float(np.max(np.abs(Or))) if Or.size else atol
    err = max_abs(O, Or)
    assert err <= bound, f"max|dO| = {err:.3e} > {bound:.3e}"
    fin = ~masked
    if fin.any():
        lerr = float(np.max(np.abs(L[fin] - Lr[fin])))
        assert lerr <= max(lse_atol, 1e-6 * float(np.max(np.abs(Lr[fin])))), f"max|dLSE| = {lerr:.3e}"
    return err
