"""bench.py's oracle leg: the host copy of a timed workload's input set holds
the same bytes, in the oracle's storage formats, as the device tensors it
came from (bf16 as uint16 bit patterns, fp16 scales, int8 codes, int32
tables), and the timing record carries its fields.  CPU tensors stand in for
the device ones."""
import numpy as np
import pytest
import torch

import bench
import synth


class _Held:
    """The attributes of a timed workload that the oracle leg reads."""

    def __init__(self, w):
        self.torch = torch
        self.prob = w.problem
        self.call_bytes = 1 << 20
        d = {}
        for k, a in w.buffers.items():
            if k == "seq_lens":
                continue
            if a.dtype == np.uint16:
                d[k] = torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
            else:
                d[k] = torch.from_numpy(a.copy())
        self.sets = [d]
        self.seq_lens = torch.from_numpy(w.buffers["seq_lens"].copy())

    host_buffers = bench.GpuWorkload.host_buffers


@pytest.mark.parametrize("make", [
    lambda: synth.make_int8(3, 2, 8, 2, 128, [700, 300], mask_kind="sink_window", n_sink=4, window=256),
    lambda: synth.make_paged(4, 3, 8, 2, 128, [33, 1, 70], page_size=16, max_pages_per_seq=8),
    lambda: synth.make_contiguous(5, 1, 4, 4, 64, [256], dtype="f32"),
])
def test_host_copy_is_the_oracle_input(make):
    w = make()
    held = _Held(w)
    hb = held.host_buffers()
    assert set(hb) == set(w.buffers)
    for k, a in w.buffers.items():
        assert hb[k].dtype == a.dtype and hb[k].shape == a.shape, k
        assert hb[k].tobytes() == a.tobytes(), k
    r = bench.oracle_timing(held, 10.0, 1, single_thread=True)
    assert r["runs"] == 1 and r["s_per_call"] > 0
    assert r["gpu_speedup"] == pytest.approx(r["s_per_call"] / 10e-6, rel=1e-2)


def test_sample_stats():
    s = sorted(float(x) for x in range(1, 101))
    assert bench.sample_stats(s) == {"count": 100, "min": 1.0, "median": 51.0, "p95": 96.0, "max": 100.0}


def test_host_info_fields():
    h = bench.host_info()
    assert h["cpu_count"] >= 1 and 1 <= h["affinity"] <= h["cpu_count"]
