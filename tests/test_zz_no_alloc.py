"""The allocation-free forward (decode_attn_forward_static) against the
ordinary forward with a caller-owned workspace, through the C ABI: two calls
in a row on the library's array, the second with a smaller batch, on the
single-launch path, on the run + combine path (32 and 24 splits) and on the
int8 kernel.  Bitwise equal to decode_attn_forward and within the bf16
tolerance of the oracle."""
import numpy as np
import pytest

import kv_cache_amd as ka
import oracle
import synth
from tests import gpu_harness as gh

pytestmark = pytest.mark.gpu


def _static(w, dw, plan):
    t = gh.torch()
    out, lse = gh._outputs(w)
    args = dw.args(None, 0)
    ka.decode_attn_forward_static(plan, args, out, lse, t.cuda.current_stream().cuda_stream)
    t.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("case", [
    # (seed, B, lengths, capacity, splits): the second call of each pair is smaller
    [(0, 6, [4096, 3000, 1, 0, 2500, 4096], 4096, 0), (1, 2, [700, 33], 1024, 0)],
    [(2, 4, [8192, 5000, 123, 8000], 8192, 32), (3, 1, [4000], 4096, 24)],
])
def test_static_forward_equals_forward_twice_in_a_row(case):
    for seed, B, lens, cap, S in case:
        gh.announce("no-alloc", seed, B, lens, S)
        w = synth.make_contiguous(seed, B, 32, 8, 128, lens, kv_capacity=cap, num_splits=S)
        dw = gh.DeviceWorkload(w)
        plan, _ = gh.plan_for(w)
        O_s, L_s = _static(w, dw, plan)
        O_f, L_f, _ = gh.forward(w, dw=dw)
        assert np.array_equal(O_s, O_f, equal_nan=False) and np.array_equal(L_s, L_f)
        O_r, L_r = oracle.attend(w.problem, w.buffers)
        gh.check_rows(O_s, L_s, O_r, L_r, atol=2e-3)


def test_static_forward_int8_sink_window():
    lens = [2000, 300, 0, 1500]
    w = synth.make_int8(4, len(lens), 32, 8, 128, lens, kv_capacity=2048, mask_kind="sink_window",
                        n_sink=4, window=1024)
    dw = gh.DeviceWorkload(w)
    plan, _ = gh.plan_for(w)
    O_s, L_s = _static(w, dw, plan)
    O_f, L_f, _ = gh.forward(w, dw=dw)
    assert np.array_equal(O_s, O_f) and np.array_equal(L_s, L_f)
