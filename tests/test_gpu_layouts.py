"""GPU parity for the other cache layouts of the ABI (M4.5 §0x04B-§0x04D):
contiguous HND, a cache-row index, packed ragged rows, paged HND and CSR page
lists.  Each holds the same logical data as a contiguous/paged NHD workload;
results are compared with the oracle (which reads through its own
translation) and the traced row offsets must match the oracle's exactly."""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_harness as H
from tests.test_gpu_parity import _trace_rows

pytestmark = pytest.mark.gpu

LENS = [500, 0, 77, 1031, 16]


@pytest.fixture(autouse=True)
def _name(request):
    H.announce(request.node.nodeid)


def _contig(dtype="bf16", D=128, Hq=8, Hkv=2):
    return synth.make_contiguous(51, len(LENS), Hq, Hkv, D, LENS, dtype=dtype, kv_capacity=1040)


def _paged(dtype="bf16", D=128, Hq=32, Hkv=8):
    return synth.make_paged(52, len(LENS), Hq, Hkv, D, LENS, page_size=16, dtype=dtype)


CASES = [("contig_hnd", {}), ("contig", {"cache_rows": 8}), ("contig_hnd", {"cache_rows": 7}),
         ("ragged", {})]


@pytest.mark.parametrize("layout,kw", CASES)
@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_contiguous_family(layout, kw, dtype, D):
    w = synth.relayout(_contig(dtype, D), layout, **kw)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    tol = 2e-3 if dtype == "bf16" else 1e-5
    for S in (None, 3):
        O, L, _ = H.forward(w, num_splits=S)
        H.check_rows(O, L, Or, Lr, tol)
    O, L, _ = H.run(w, num_splits=5)
    H.check_rows(O, L, Or, Lr, tol)


@pytest.mark.parametrize("layout,table", [("paged_hnd", "dense"), ("paged", "csr"), ("paged_hnd", "csr")])
@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_paged_family(layout, table, dtype, D):
    w = synth.relayout(_paged(dtype, D), layout, page_table=table)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    tol = 2e-3 if dtype == "bf16" else 1e-5
    O, L, _ = H.forward(w)
    H.check_rows(O, L, Or, Lr, tol)
    O, L, _ = H.run(w, num_splits=7)
    H.check_rows(O, L, Or, Lr, tol)


@pytest.mark.parametrize("layout,kw", CASES + [("paged_hnd", {}), ("paged", {"page_table": "csr"})])
def test_trace_offsets_match_oracle(layout, kw):
    base = _paged() if layout.startswith("paged") else _contig()
    _trace_rows(synth.relayout(base, layout, **kw), 4)


def test_few_query_rows_on_hnd_and_csr():
    for w in (synth.relayout(synth.make_contiguous(53, 3, 8, 4, 128, [300, 2, 90], kv_capacity=300,
                                                   num_queries=2), "contig_hnd"),
              synth.relayout(synth.make_paged(54, 3, 8, 4, 128, [300, 2, 90], num_queries=2),
                             "paged_hnd", page_table="csr")):
        Or, Lr = oracle.attend(w.problem, w.buffers)
        O, L, _ = H.forward(w)
        H.check_rows(O, L, Or, Lr, 2e-3)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_ring_sink_window_layout(dtype, D):
    lens = [5000, 3, 700, 0, 4100]
    w = synth.make_contiguous(55, len(lens), 8, 2, D, lens, dtype=dtype, kv_capacity=5000,
                              mask_kind="sink_window", n_sink=4, window=600)
    w = synth.relayout(w, "ring")
    Or, Lr = oracle.attend(w.problem, w.buffers)
    tol = 2e-3 if dtype == "bf16" else 1e-5
    O, L, _ = H.forward(w)
    H.check_rows(O, L, Or, Lr, tol)
    O, L, _ = H.run(w, num_splits=5)
    H.check_rows(O, L, Or, Lr, tol)
    _trace_rows(w, 3)
