"""GPU checks of the host-built work order (decode_attn_schedule): any
permutation of the work items leaves every result bit-identical, so the
scheduled runs must equal the built-in order exactly and match the oracle."""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name(request):
    H.announce(request.node.nodeid)


def _pair(w, fn, num_splits=None):
    plain = H.DeviceWorkload(w)
    sched = H.DeviceWorkload(w)
    plan, _ = H.plan_for(w, num_splits)
    sched.schedule(plan)
    a = fn(w, num_splits=num_splits, dw=plain)
    b = fn(w, num_splits=num_splits, dw=sched)
    return a, b


@pytest.mark.parametrize("S", [None, 8])
def test_schedule_paged_ragged_bitwise_equal_and_parity(S):
    w = synth.make_paged(21, 6, 32, 8, 128, [3000, 0, 517, 4096, 1, 2222], page_size=16)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    for fn in (H.run, H.forward):
        (O1, L1, _), (O2, L2, _) = [r[:3] for r in _pair(w, fn, S)]
        assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
        H.check_rows(O2, L2, Or, Lr, 2e-3)


def test_schedule_int8_sink_window():
    w = synth.make_int8(22, 3, 8, 2, 128, [1000, 100, 250], residual_len=128,
                        mask_kind="sink_window", n_sink=4, window=300)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    (O1, L1, _), (O2, L2, _) = [r[:3] for r in _pair(w, H.forward, 5)]
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    H.check_rows(O2, L2, Or, Lr, 0.0, rtol=1e-2)


def test_schedule_trace_indices_unchanged():
    w = synth.make_paged(23, 4, 8, 2, 128, [700, 33, 0, 1500], page_size=16)
    (t1, _, O1, L1), (t2, _, O2, L2) = _pair(w, H.trace, 6)
    assert t1.keys() == t2.keys()
    for key in t1:
        assert np.array_equal(t1[key], t2[key]), key
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
