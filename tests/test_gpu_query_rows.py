"""GPU parity for few-query decode (C > 1 query rows per request, bottom-right
causal alignment, M4.5 §0x08B-§0x08C): a workgroup serves the C*g virtual
heads of its K/V head, each with its own visible end."""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name(request):
    H.announce(request.node.nodeid)


LENS = [0, 1, 2, 5, 300, 1000, 129]


@pytest.mark.parametrize("Hq,Hkv,C", [(8, 2, 2), (8, 4, 4), (4, 4, 8), (8, 8, 2)])
@pytest.mark.parametrize("S", [None, 1, 6])
def test_query_rows_contiguous_bf16(Hq, Hkv, C, S):
    w = synth.make_contiguous(41, len(LENS), Hq, Hkv, 128, LENS, kv_capacity=1024, num_queries=C)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    dw = H.DeviceWorkload(w)
    O, L, _ = H.run(w, num_splits=S, dw=dw)
    H.check_rows(O, L, Or, Lr, 2e-3)
    O2, L2, _ = H.forward(w, num_splits=S, dw=dw)
    H.check_rows(O2, L2, Or, Lr, 2e-3)


@pytest.mark.parametrize("C", [2, 4])
def test_query_rows_fp32_d64(C):
    w = synth.make_contiguous(42, len(LENS), 4, 2, 64, LENS, dtype="f32", kv_capacity=1024, num_queries=C)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    O, L, _ = H.forward(w, num_splits=5)
    H.check_rows(O, L, Or, Lr, 1e-5)


def test_query_rows_paged():
    w = synth.make_paged(43, 4, 32, 8, 128, [3000, 1, 517, 4096], page_size=16, num_queries=2)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    O, L, _ = H.forward(w)
    H.check_rows(O, L, Or, Lr, 2e-3)
    O, L, _ = H.run(w, num_splits=40)
    H.check_rows(O, L, Or, Lr, 2e-3)


@pytest.mark.parametrize("policy", ["window", "groups"])
def test_query_rows_int8(policy):
    w = synth.make_int8(44, 3, 8, 4, 128, [1000, 130, 2], residual_len=128, num_queries=2,
                        residual_policy=policy)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    O, L, _ = H.forward(w, num_splits=4)
    H.check_rows(O, L, Or, Lr, 0.0, rtol=1e-2)


def test_query_row_c1_layout_is_the_decode_layout():
    """C = 1 written explicitly gives the same bytes as the default decode."""
    w = synth.make_contiguous(45, 3, 8, 2, 128, [70, 0, 900], kv_capacity=1024)
    O1, L1, _ = H.forward(w, num_splits=3)
    w.problem.num_queries = 1
    O2, L2, _ = H.forward(w, num_splits=3)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
