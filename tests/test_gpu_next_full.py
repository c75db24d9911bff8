"""GPU parity at the llama3-8b layer shape (B=8, 32 query / 8 K/V heads, d=128,
T=4096, bf16) for the variants the bench times beside the headline: C = 2
query rows, the HND layout and FlashMask intervals.  Every output row is
compared with the fp64 oracle, through the single-launch forward and through
run + combine, in the bench's automatic split count."""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

TOL = 2e-3
LENS = [4096] * 8


@pytest.fixture(autouse=True)
def _name(request):
    H.announce(request.node.nodeid)


def _check_both(w, dw=None):
    Or, Lr = oracle.attend(w.problem, w.buffers)
    dw = dw or H.DeviceWorkload(w)
    O, L, plan = H.run(w, dw=dw)
    H.check_rows(O, L, Or, Lr, TOL)
    O2, L2, _ = H.forward(w, dw=dw)
    H.check_rows(O2, L2, Or, Lr, TOL)
    return plan


def test_full_shape_two_query_rows():
    w = synth.make_contiguous(71, 8, 32, 8, 128, LENS, kv_capacity=4096, num_queries=2)
    plan = _check_both(w)
    assert plan.num_splits == 4


def test_full_shape_hnd_layout():
    w = synth.relayout(synth.make_contiguous(72, 8, 32, 8, 128, LENS, kv_capacity=4096), "contig_hnd")
    plan = _check_both(w)
    assert plan.num_splits == 4


def test_full_shape_flashmask():
    w = synth.make_contiguous(73, 8, 32, 8, 128, LENS, kv_capacity=4096)
    w.buffers["mask_intervals"] = synth.flashmask_intervals(73, w.buffers["seq_lens"], 4096)
    w.problem.mask_kind = "flashmask"
    dw = H.DeviceWorkload(w)
    plan, _ = H.plan_for(w)
    dw.summarize_mask(plan)
    _check_both(w, dw)
    # the mask hides a real share of the keys at this size
    iv = w.buffers["mask_intervals"]
    q = 4095
    hidden = ((iv[..., 0] <= q) & (q < iv[..., 1])) | ((iv[..., 2] <= q) & (q < iv[..., 3]))
    assert 0.2 < float(np.mean(hidden)) < 0.8


@pytest.fixture(scope="module")
def cfg3_base():
    return synth.config(3, 1)


@pytest.mark.parametrize("layout,table", [("paged_hnd", "dense"), ("paged", "csr")])
def test_cfg3_layouts_sampled_rows_with_partition(cfg3_base, layout, table):
    # the paged ragged batch of 32 requests (lengths 1 .. 32768) in the HND
    # page layout and with a CSR page list, fixed splits and the balanced
    # partition, on sampled rows (and the longest and shortest requests)
    w = synth.relayout(cfg3_base, layout, page_table=table)
    dw = H.DeviceWorkload(w)
    g = synth.rng(78)
    rows = [(int(b), int(h)) for b, h in zip(g.integers(0, 32, 16), g.integers(0, 32, 16))]
    rows += [(int(np.argmax(w.buffers["seq_lens"])), 5), (int(np.argmin(w.buffers["seq_lens"])), 30)]
    Or, Lr = oracle.attend(w.problem, w.buffers, heads=rows)
    O, L, plan = H.run(w, dw=dw)
    H.check_rows(O, L, Or, Lr, TOL, rows=rows)
    O, L, _ = H.run(w, dw=dw, partition=0)
    H.check_rows(O, L, Or, Lr, TOL, rows=rows)
