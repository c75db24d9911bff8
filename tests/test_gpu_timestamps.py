"""GPU checks of the timestamp instance (decode_attn_timestamps): the same
kernels as decode_attn_forward plus per-workgroup clock reads, so its outputs
equal the forward's bit for bit; every workgroup writes ordered stamps and an
XCD id, and exactly one workgroup per (b, h_kv) folds (single launch)."""
import numpy as np
import pytest

import kv_cache_amd as ka
import oracle
import synth
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name(request):
    H.announce(request.node.nodeid)


def _stamped(w, num_splits):
    t = H.torch()
    dw = H.DeviceWorkload(w)
    plan, ws_bytes = H.plan_for(w, num_splits)
    ws = t.empty(max(ws_bytes, 16), dtype=t.uint8, device="cuda")
    s = t.cuda.current_stream().cuda_stream
    ka.decode_attn_workspace_init(plan, ws, ws_bytes, s)
    out, lse = H._outputs(w)
    p = w.problem
    grid = p.batch * p.num_kv_heads * plan.num_splits
    st = t.zeros((grid, 4), dtype=t.int64, device="cuda")
    _, hz = ka.decode_attn_timestamps(plan, dw.args(ws, ws_bytes), out, lse, st, s)
    t.cuda.synchronize()
    return (out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
            st.cpu().numpy().view(np.uint64), hz, plan)


@pytest.mark.parametrize("kind", ["bf16", "i8"])
def test_timestamps_outputs_and_stamps(kind):
    if kind == "bf16":
        w = synth.make_contiguous(81, 4, 16, 4, 128, [1000, 0, 333, 2048], kv_capacity=2048)
    else:
        w = synth.make_int8(82, 3, 8, 2, 128, [1500, 300, 0], residual_len=128,
                            mask_kind="sink_window", n_sink=4, window=700)
    O, L, st, hz, plan = _stamped(w, 6)
    Of, Lf, _ = H.forward(w, num_splits=6)
    assert np.array_equal(O, Of) and np.array_equal(L, Lf)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    H.check_rows(O, L, Or, Lr, 2e-3 if kind == "bf16" else 0.0, rtol=0.0 if kind == "bf16" else 1e-2)
    assert 1e6 <= hz <= 1e10
    start, stored, end, meta = st[:, 0], st[:, 1], st[:, 2], st[:, 3]
    assert (start > 0).all() and (start <= stored).all() and (stored <= end).all()
    assert ((meta & 0xF) < 8).all()
    folded = (meta >> np.uint64(63)).astype(bool)
    p = w.problem
    assert folded.sum() == p.batch * p.num_kv_heads
    # span of one small call: well under a second of the constant-rate clock
    assert (end.max() - start.min()) / hz < 1.0
