"""Thin ctypes binding of libdecode_attn.so (MI355X decode attention).

Argument marshalling only: every computation happens in the library's HIP
kernels.  Tensors are passed as device pointers (``tensor.data_ptr()``) and
the stream as ``torch.cuda.current_stream().cuda_stream``; PyTorch is used by
callers only for device memory and streams.  Importing this module does not
need a GPU; loading the library needs the built ``libdecode_attn.so`` and
fails loudly when it is missing.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "DA_OK", "DA_ERR_INVALID", "DA_ERR_UNSUPPORTED", "DA_ERR_WORKSPACE",
    "DA_ERR_PLAN_MISMATCH", "DA_ERR_HIP", "DecodeAttnError", "Problem", "Plan",
    "Args", "Trace", "lib", "library_path", "problem_from", "decode_attn_plan",
    "decode_attn_schedule", "decode_attn_append", "decode_attn_flashmask_summarize", "AppendArgs", "decode_attn_run", "decode_attn_combine", "decode_attn_forward",
    "decode_attn_workspace_init", "decode_attn_trace_indices", "decode_attn_forward_static", "decode_attn_timestamps",
    "STATIC_WORKSPACE_BYTES",
    "decode_attn_reason", "decode_attn_status_string", "reason_names",
]

DA_OK, DA_ERR_INVALID, DA_ERR_UNSUPPORTED = 0, -1, -2
DA_ERR_WORKSPACE, DA_ERR_PLAN_MISMATCH, DA_ERR_HIP = -3, -4, -5

DTYPES = {"f32": 0, "bf16": 1, "f16": 2}
KV_FORMATS = {"f32": 0, "bf16": 1, "i8": 2}
LAYOUTS = {"contig": 0, "paged": 1, "contig_hnd": 2, "paged_hnd": 3, "ragged": 4, "ring": 5}
PAGE_TABLES = {"dense": 0, "csr": 1}
MASKS = {"causal": 0, "sink_window": 1, "flashmask": 2}
RESIDUAL_POLICIES = {"window": 0, "groups": 1}
NUM_REASONS = 13
STATIC_WORKSPACE_BYTES = 32 << 20


class Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "num_q_heads", "num_kv_heads", "head_dim_qk", "head_dim_v", "q_dtype",
        "out_dtype", "kv_format", "layout", "kv_capacity", "page_size", "max_pages_per_seq",
        "num_pages", "max_seq_len", "mask_kind", "n_sink", "window")] + [
        ("softmax_scale", ctypes.c_float)] + [(n, ctypes.c_int32) for n in (
            "num_splits", "k_group", "residual_len", "num_cus", "residual_policy", "num_queries",
            "page_table", "cache_rows", "num_page_entries", "reserved1")]


class Plan(ctypes.Structure):
    _fields_ = [("key", ctypes.c_uint64), ("problem", Problem), ("num_splits", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("max_visible", ctypes.c_int32),
                ("num_cus", ctypes.c_int32), ("workspace_bytes", ctypes.c_uint64),
                ("reserved", ctypes.c_uint64 * 2)]


class Args(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "q", "k", "v", "k_scale", "v_scale", "k_resid", "v_resid", "block_table", "seq_lens",
        "workspace")] + [("workspace_bytes", ctypes.c_uint64), ("work_order", ctypes.c_void_p),
                         ("indptr", ctypes.c_void_p), ("cache_batch_idx", ctypes.c_void_p),
                         ("mask_intervals", ctypes.c_void_p), ("mask_summary", ctypes.c_void_p),
                         ("partition", ctypes.c_void_p), ("partition_items", ctypes.c_int32),
                         ("reserved0", ctypes.c_int32)]


class Trace(ctypes.Structure):
    """da_trace: device arrays of B * H_kv * plan.max_visible entries."""
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "k_offset", "v_offset", "position", "count", "k_scale_offset", "v_scale_offset")]


class AppendArgs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "k_new", "v_new", "k", "v", "k_scale", "v_scale", "k_resid", "v_resid", "seq_lens",
        "status")]


DA_APPEND_NO_ROOM, DA_APPEND_BAD_SCALE = 1, 2


class DecodeAttnError(RuntimeError):
    def __init__(self, status: int, what: str, reasons: int = 0):
        self.status = status
        self.reasons = reasons
        text = decode_attn_status_string(status)
        if reasons:
            text += ": " + "; ".join(reason_names(reasons))
        super().__init__(f"{what}: {text} (status {status}, reasons 0x{reasons:x})")


def library_path() -> str:
    """The in-tree library, or the variant named by KV_CACHE_AMD_LIB (a build
    of the same sources with other compile-time switches, for comparisons)."""
    return os.environ.get("KV_CACHE_AMD_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                               "libdecode_attn.so")


_LIB = None


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
        # One HIP runtime per process: torch ships its own libamdhip64 with the
        # same soname as ROCm's, and whichever loads first serves both.  Load
        # torch's first (the caller's tensors and streams live there); torch
        # then fails to initialise if this library's runtime came first.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(path)
        L.decode_attn_plan.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(Plan),
                                       ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_uint64)]
        L.decode_attn_plan.restype = ctypes.c_int32
        L.decode_attn_schedule.argtypes = [ctypes.POINTER(Plan), ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_uint64]
        L.decode_attn_schedule.restype = ctypes.c_int32
        L.decode_attn_partition.argtypes = [ctypes.POINTER(Plan), ctypes.c_void_p, ctypes.c_int32,
                                            ctypes.c_void_p, ctypes.c_uint64,
                                            ctypes.POINTER(ctypes.c_int32)]
        L.decode_attn_partition.restype = ctypes.c_int32
        L.decode_attn_append.argtypes = [ctypes.POINTER(Plan), ctypes.POINTER(AppendArgs),
                                         ctypes.c_void_p]
        L.decode_attn_append.restype = ctypes.c_int32
        L.decode_attn_flashmask_summarize.argtypes = [ctypes.POINTER(Plan), ctypes.c_void_p,
                                                      ctypes.c_void_p, ctypes.c_void_p]
        L.decode_attn_flashmask_summarize.restype = ctypes.c_int32
        L.decode_attn_run.argtypes = [ctypes.POINTER(Plan), ctypes.POINTER(Args), ctypes.c_void_p]
        L.decode_attn_run.restype = ctypes.c_int32
        L.decode_attn_combine.argtypes = [ctypes.POINTER(Plan), ctypes.c_void_p, ctypes.c_uint64,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.decode_attn_combine.restype = ctypes.c_int32
        L.decode_attn_forward.argtypes = [ctypes.POINTER(Plan), ctypes.POINTER(Args),
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.decode_attn_forward.restype = ctypes.c_int32
        L.decode_attn_forward_static.argtypes = [ctypes.POINTER(Plan), ctypes.POINTER(Args),
                                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.decode_attn_forward_static.restype = ctypes.c_int32
        L.decode_attn_workspace_init.argtypes = [ctypes.POINTER(Plan), ctypes.c_void_p,
                                                 ctypes.c_uint64, ctypes.c_void_p]
        L.decode_attn_workspace_init.restype = ctypes.c_int32
        L.decode_attn_trace_indices.argtypes = [ctypes.POINTER(Plan), ctypes.POINTER(Args),
                                                ctypes.POINTER(Trace), ctypes.c_void_p, ctypes.c_void_p,
                                                ctypes.c_void_p]
        L.decode_attn_trace_indices.restype = ctypes.c_int32
        L.decode_attn_timestamps.argtypes = [ctypes.POINTER(Plan), ctypes.POINTER(Args), ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.POINTER(ctypes.c_uint64), ctypes.c_void_p]
        L.decode_attn_timestamps.restype = ctypes.c_int32
        L.decode_attn_reason.argtypes = [ctypes.c_int]
        L.decode_attn_reason.restype = ctypes.c_char_p
        L.decode_attn_status_string.argtypes = [ctypes.c_int32]
        L.decode_attn_status_string.restype = ctypes.c_char_p
        _LIB = L
    return _LIB


def decode_attn_reason(bit: int) -> str:
    return lib().decode_attn_reason(bit).decode()


def decode_attn_status_string(status: int) -> str:
    return lib().decode_attn_status_string(status).decode()


def reason_names(reasons: int):
    return [decode_attn_reason(i) for i in range(NUM_REASONS) if reasons >> i & 1]


def problem_from(p, num_cus: int = 0) -> Problem:
    """Build the C struct from any object with the field names of
    ``da_problem`` (strings allowed for the enum fields)."""
    def enum(v, table):
        return table[v] if isinstance(v, str) else int(v)
    d = getattr(p, "head_dim", None)
    return Problem(
        batch=p.batch, num_q_heads=p.num_q_heads, num_kv_heads=p.num_kv_heads,
        head_dim_qk=getattr(p, "head_dim_qk", d), head_dim_v=getattr(p, "head_dim_v", d),
        q_dtype=enum(p.q_dtype, DTYPES), out_dtype=enum(getattr(p, "out_dtype", "f32"), DTYPES),
        kv_format=enum(p.kv_format, KV_FORMATS), layout=enum(p.layout, LAYOUTS),
        kv_capacity=p.kv_capacity if enum(p.layout, LAYOUTS) in (0, 2, 5) else 0,
        page_size=p.page_size, max_pages_per_seq=p.max_pages_per_seq, num_pages=p.num_pages,
        max_seq_len=p.max_seq_len, mask_kind=enum(p.mask_kind, MASKS), n_sink=p.n_sink,
        window=p.window, softmax_scale=p.softmax_scale, num_splits=p.num_splits,
        k_group=p.k_group, residual_len=p.residual_len, num_cus=num_cus,
        residual_policy=enum(getattr(p, "residual_policy", 0), RESIDUAL_POLICIES),
        num_queries=int(getattr(p, "num_queries", 1) or 1),
        page_table=enum(getattr(p, "page_table", 0), PAGE_TABLES),
        cache_rows=int(getattr(p, "cache_rows", 0)),
        num_page_entries=int(getattr(p, "num_page_entries", 0)))


def decode_attn_plan(problem: Problem, check: bool = True):
    """Returns ``(status, plan, workspace_bytes, reasons)``; raises
    DecodeAttnError on failure when ``check``."""
    plan = Plan()
    ws = ctypes.c_uint64(0)
    rs = ctypes.c_uint64(0)
    st = lib().decode_attn_plan(ctypes.byref(problem), ctypes.byref(plan), ctypes.byref(ws),
                                ctypes.byref(rs))
    if check and st != DA_OK:
        raise DecodeAttnError(st, "decode_attn_plan", rs.value)
    return st, plan, ws.value, rs.value


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def make_args(q, k, v, seq_lens, workspace, workspace_bytes, k_scale=None, v_scale=None,
              k_resid=None, v_resid=None, block_table=None, work_order=None, indptr=None,
              cache_batch_idx=None, mask_intervals=None, mask_summary=None, partition=None,
              partition_items=0) -> Args:
    return Args(q=_ptr(q), k=_ptr(k), v=_ptr(v), k_scale=_ptr(k_scale), v_scale=_ptr(v_scale),
                k_resid=_ptr(k_resid), v_resid=_ptr(v_resid), block_table=_ptr(block_table),
                seq_lens=_ptr(seq_lens), workspace=_ptr(workspace),
                workspace_bytes=int(workspace_bytes), work_order=_ptr(work_order),
                indptr=_ptr(indptr), cache_batch_idx=_ptr(cache_batch_idx),
                mask_intervals=_ptr(mask_intervals), mask_summary=_ptr(mask_summary),
                partition=_ptr(partition), partition_items=int(partition_items), reserved0=0)


def decode_attn_partition(plan: Plan, seq_lens_host, items_per_head: int = 0, check: bool = True):
    """Balanced partition of the batch from host lengths; returns (descriptor
    int32 NumPy array, W).  Copy the descriptor to the device and pass both to
    make_args(partition=..., partition_items=W)."""
    import numpy as np
    lens = np.ascontiguousarray(np.asarray(seq_lens_host, dtype=np.int32))
    p = plan.problem
    target = items_per_head or max(1, (3 * plan.num_cus) // max(p.num_kv_heads, 1))
    part = np.zeros(5 + p.batch + target, dtype=np.int32)
    items = ctypes.c_int32(0)
    st = lib().decode_attn_partition(ctypes.byref(plan), lens.ctypes.data, int(items_per_head),
                                     part.ctypes.data, part.size, ctypes.byref(items))
    if check and st != DA_OK:
        raise DecodeAttnError(st, "decode_attn_partition")
    return part[:5 + p.batch + items.value], items.value


def decode_attn_schedule(plan: Plan, seq_lens_host, check: bool = True):
    """Largest-first work order for the plan's grid from host lengths (a list
    or int32 array); returns an int32 NumPy array of B*H_kv*S work items."""
    import numpy as np
    lens = np.ascontiguousarray(np.asarray(seq_lens_host, dtype=np.int32))
    p = plan.problem
    n = p.batch * p.num_kv_heads * plan.num_splits
    order = np.empty(max(n, 1), dtype=np.int32)
    st = lib().decode_attn_schedule(ctypes.byref(plan), lens.ctypes.data, order.ctypes.data, n)
    if check and st != DA_OK:
        raise DecodeAttnError(st, "decode_attn_schedule")
    return order[:n]


def decode_attn_flashmask_summarize(plan: Plan, intervals, summary, stream: int = 0,
                                    check: bool = True) -> int:
    st = lib().decode_attn_flashmask_summarize(ctypes.byref(plan), _ptr(intervals), _ptr(summary),
                                               stream)
    if check and st != DA_OK:
        raise DecodeAttnError(st, "decode_attn_flashmask_summarize")
    return st


def decode_attn_run(plan: Plan, args: Args, stream: int = 0, check: bool = True) -> int:
    st = lib().decode_attn_run(ctypes.byref(plan), ctypes.byref(args), stream)
    if check and st != DA_OK:
        raise DecodeAttnError(st, "decode_attn_run")
    return st


def decode_attn_combine(plan: Plan, workspace, workspace_bytes: int, out, lse=None,
                        stream: int = 0, check: bool = True) -> int:
    st = lib().decode_attn_combine(ctypes.byref(plan), _ptr(workspace), int(workspace_bytes),
                                   _ptr(out), _ptr(lse), stream)
    if check and st != DA_OK:
        raise DecodeAttnError(st, "decode_attn_combine")
    return st


def decode_attn_forward(plan: Plan, args: Args, out, lse=None, stream: int = 0,
                        check: bool = True) -> int:
    st = lib().decode_attn_forward(ctypes.byref(plan), ctypes.byref(args), _ptr(out), _ptr(lse),
                                   stream)
    if check and st != DA_OK:
        raise DecodeAttnError(st, "decode_attn_forward")
    return st


def decode_attn_forward_static(plan: Plan, args: Args, out, lse=None, stream: int = 0,
                               check: bool = True) -> int:
    st = lib().decode_attn_forward_static(ctypes.byref(plan), ctypes.byref(args), _ptr(out),
                                          _ptr(lse), stream)
    if check and st != DA_OK:
        raise DecodeAttnError(st, "decode_attn_forward_static")
    return st


def decode_attn_workspace_init(plan: Plan, workspace, workspace_bytes: int, stream: int = 0,
                               check: bool = True) -> int:
    st = lib().decode_attn_workspace_init(ctypes.byref(plan), _ptr(workspace),
                                          int(workspace_bytes), stream)
    if check and st != DA_OK:
        raise DecodeAttnError(st, "decode_attn_workspace_init")
    return st


def decode_attn_append(plan: Plan, k_new, v_new, k, v, k_scale, v_scale, k_resid, v_resid,
                       seq_lens, status=None, stream: int = 0, check: bool = True) -> int:
    a = AppendArgs(k_new=_ptr(k_new), v_new=_ptr(v_new), k=_ptr(k), v=_ptr(v),
                   k_scale=_ptr(k_scale), v_scale=_ptr(v_scale), k_resid=_ptr(k_resid),
                   v_resid=_ptr(v_resid), seq_lens=_ptr(seq_lens), status=_ptr(status))
    st = lib().decode_attn_append(ctypes.byref(plan), ctypes.byref(a), stream)
    if check and st != DA_OK:
        raise DecodeAttnError(st, "decode_attn_append")
    return st


def decode_attn_timestamps(plan: Plan, args: Args, out, lse, stamps, stream: int = 0,
                           check: bool = True):
    """Timestamp instance of decode_attn_forward's launches; ``stamps`` is a
    device uint64 tensor of [grid, 4].  Returns (status, clock rate in Hz)."""
    hz = ctypes.c_uint64(0)
    st = lib().decode_attn_timestamps(ctypes.byref(plan), ctypes.byref(args), _ptr(out), _ptr(lse),
                                      _ptr(stamps), ctypes.byref(hz), stream)
    if check and st != DA_OK:
        raise DecodeAttnError(st, "decode_attn_timestamps")
    return st, hz.value


def decode_attn_trace_indices(plan: Plan, args: Args, k_offset, v_offset, position, count,
                              k_scale_offset=None, v_scale_offset=None, out=None, lse=None,
                              stream: int = 0, check: bool = True) -> int:
    """Trace instance of the timed kernels (decode_attn_run's, or with ``out``
    decode_attn_forward's); the arrays are device tensors of B*H_kv*max_visible
    entries (int64 offsets, int32 position and count)."""
    tr = Trace(k_offset=_ptr(k_offset), v_offset=_ptr(v_offset), position=_ptr(position),
               count=_ptr(count), k_scale_offset=_ptr(k_scale_offset),
               v_scale_offset=_ptr(v_scale_offset))
    st = lib().decode_attn_trace_indices(ctypes.byref(plan), ctypes.byref(args), ctypes.byref(tr),
                                         _ptr(out), _ptr(lse), stream)
    if check and st != DA_OK:
        raise DecodeAttnError(st, "decode_attn_trace_indices")
    return st
