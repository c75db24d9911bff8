"""Balanced partition of ragged batches (decode_attn_partition): every
workgroup gets the same number of visible ordinals, requests split into pieces
at item boundaries, the combine folds each request's pieces.  Compared with the
fp64 oracle ("M4.5 - Decode Attention Kernels, Mask Programs, and Backend
Boundaries", sections 0x02B-0x02E: any disjoint exact cover of the visible rows
merges to the same result)."""
import numpy as np
import pytest

import kv_cache_amd as ka
import oracle
import synth
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu
TOL = 2e-3


@pytest.mark.parametrize("items", [1, 3, 16, 0, 400])
def test_partition_paged_ragged(items):
    # items = 1: one workgroup per head walks every request; 400: 16-row items
    lens = [1, 15, 16, 17, 300, 0, 2000, 33]
    w = synth.make_paged(6, len(lens), 32, 8, 128, lens, page_size=16, max_pages_per_seq=130)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    H.announce(f"partition paged items={items}")
    O, L, _ = H.run(w, num_splits=0, partition=items)
    H.check_rows(O, L, Or, Lr, TOL)


@pytest.mark.parametrize("lens,ns,W", [([5, 40, 300, 1, 0], 4, 16), ([64, 65, 200], 70, 10),
                                       ([3000, 100, 0, 2500], 4, 1000)])
def test_partition_contiguous_sink_window(lens, ns, W):
    w = synth.make_contiguous(8, len(lens), 16, 4, 128, lens, mask_kind="sink_window", n_sink=ns,
                              window=W, kv_capacity=max(lens) + 5)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    dw = H.DeviceWorkload(w)
    for items in (2, 0, 50):
        O, L, _ = H.run(w, num_splits=4, dw=dw, partition=items)
        H.check_rows(O, L, Or, Lr, TOL)


def test_partition_query_rows():
    w = synth.make_contiguous(21, 3, 16, 4, 128, [700, 33, 1], num_queries=2, kv_capacity=700)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    O, L, _ = H.run(w, num_splits=4, partition=5)
    H.check_rows(O, L, Or, Lr, TOL)


def test_partition_and_fixed_splits_share_a_workspace():
    # a partitioned run leaves its header in the workspace; the next fixed-split
    # run must overwrite it, and forward() must fold a partition in the combine
    t = H.torch()
    lens = [900, 0, 17, 2000]
    w = synth.make_contiguous(23, len(lens), 32, 8, 128, lens, kv_capacity=2000)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    dw = H.DeviceWorkload(w)
    plan, wsb = H.plan_for(w, 8)
    ws = t.full((wsb,), 0xFF, dtype=t.uint8, device="cuda")
    s = t.cuda.current_stream().cuda_stream
    ka.decode_attn_workspace_init(plan, ws, wsb, s)
    outs = []
    for use_part in (True, False, True):
        if use_part:
            dw.partition(plan, 7)
        else:
            dw.part, dw.part_items = None, 0
        O1, L1 = H._outputs(w)
        O2, L2 = H._outputs(w)
        ka.decode_attn_run(plan, dw.args(ws, wsb), s)
        ka.decode_attn_combine(plan, ws, wsb, O1, L1, s)
        ka.decode_attn_forward(plan, dw.args(ws, wsb), O2, L2, s)
        t.cuda.synchronize()
        a, b = O1.cpu().numpy(), O2.cpu().numpy()
        if use_part:            # forward() of a partition is run + combine
            assert np.array_equal(a, b) and np.array_equal(L1.cpu().numpy(), L2.cpu().numpy())
        H.check_rows(a.astype(np.float64), L1.cpu().numpy().astype(np.float64), Or, Lr, TOL)
        H.check_rows(b.astype(np.float64), L2.cpu().numpy().astype(np.float64), Or, Lr, TOL)
        outs.append(a)
    assert np.array_equal(outs[0], outs[2])       # fixed plan + fixed partition: bitwise repeatable


@pytest.mark.parametrize("mask", ["causal", "sink_window"])
def test_partition_int8_ragged(mask):
    # int8 codes + bf16 residual under a balanced partition: pieces cut through
    # the int8 part, the seam between sinks and window, and the residual rows
    lens = [0, 1, 100, 128, 200, 1000, 5000, 3000]
    mk = dict(mask_kind="sink_window", n_sink=4, window=900) if mask == "sink_window" else {}
    w = synth.make_int8(91, len(lens), 16, 4, 128, lens, residual_len=128, kv_capacity=5000, **mk)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    dw = H.DeviceWorkload(w)
    for items in (1, 3, 0, 100):
        H.announce(f"int8 partition {mask} items={items}")
        O, L, _ = H.run(w, num_splits=8, dw=dw, partition=items)
        H.check_rows(O, L, Or, Lr, 0.0, rtol=1e-2)
        O2, L2, _ = H.run(w, num_splits=8, dw=dw, partition=items)
        assert np.array_equal(O, O2) and np.array_equal(L, L2)      # fixed partition: bitwise repeatable


def test_partition_int8_trace_exact():
    # the partition instance's own loads: every visible row once, at the
    # oracle's code, residual and scale offsets
    lens = [700, 0, 2100, 300, 40]
    w = synth.make_int8(92, len(lens), 8, 2, 128, lens, residual_len=128, kv_capacity=2100,
                        mask_kind="sink_window", n_sink=4, window=1000)
    dw = H.DeviceWorkload(w)
    tr, plan, O, L = H.trace(w, num_splits=6, dw=dw, partition=5)
    H.check_trace(w, tr)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    H.check_rows(O, L, Or, Lr, 0.0, rtol=1e-2)


def test_partition_int8_full_ragged_batch():
    # the config-5 shape with ragged lengths (B = 16, 32q/8kv, 4 sinks + window
    # 4096, residual 128), default partition, every row against the oracle
    lens = [int(x) for x in synth.rng(93).integers(129 + 128, 16300, size=16)]
    # no 1-15-row trailing K group (its per-channel scales of a few N(0,1)
    # values can fall below fp16's normal range, which the writer refuses)
    lens = [T + 16 if 0 < (T - 128) % 128 < 16 else T for T in lens]
    lens[3] = 0
    w = synth.make_int8(93, 16, 32, 8, 128, lens, residual_len=128, kv_capacity=16384,
                        mask_kind="sink_window", n_sink=4, window=4096)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    O, L, _ = H.run(w, num_splits=0, partition=0)
    H.check_rows(O, L, Or, Lr, 0.0, rtol=1e-2)
