"""The int8 K/V path against the bf16 path on the GPU, where the format is
exact ("M8.6 - Live-Data Quantization: Activations and KV Cache", section
0x0CB: attention over the quantized cache must equal attention over the
decoded values, with one shared softmax):

* exact quantization: values on the int8 grid (c * 2^-k with one +-127 per
  K group and channel, and per V row) quantize without error, so the int8
  kernel on the quantized cache and the bf16 kernel on the same values give
  the same output within the bf16 tolerance;
* residual only: a window inside the bf16 residual never reads a code, so the
  int8 and bf16 kernels agree the same way."""
import numpy as np
import pytest

import oracle
import synth
from oracle.numerics import decode_bf16
from tests import gpu_harness as H
from tests.test_int8_format import _exact_grid_values

pytestmark = pytest.mark.gpu


def _bf16_twin(w, kf, vf, exact=True, **mask):
    p = w.problem
    lens = w.buffers["seq_lens"]
    wb = synth.make_contiguous(0, p.batch, p.num_q_heads, p.num_kv_heads, p.head_dim, lens,
                               kv_capacity=kf.shape[1], poison_tail=False, **mask)
    wb.buffers["q"] = w.buffers["q"]
    wb.buffers["k"] = synth.bf16_bits(kf)
    wb.buffers["v"] = synth.bf16_bits(vf)
    if exact:      # grid values: bf16 holds them exactly
        assert np.array_equal(decode_bf16(wb.buffers["k"]), kf.astype(np.float64))
        assert np.array_equal(decode_bf16(wb.buffers["v"]), vf.astype(np.float64))
    return wb


@pytest.mark.parametrize("mask", [dict(), dict(mask_kind="sink_window", n_sink=4, window=1500)])
def test_exact_quantization_int8_equals_bf16(mask):
    B, T, Hkv, D, G = 4, 4096, 8, 128, 128
    kf, vf = _exact_grid_values(synth.rng(31), B, T, Hkv, D, G)
    lens = [4096, 2944, 256, 100]      # quantized counts are whole groups of 128
    w = synth.make_int8(31, B, 32, Hkv, D, lens, k_group=G, residual_len=128, kv_capacity=T,
                        values=(kf, vf), **mask)
    wb = _bf16_twin(w, kf, vf, **mask)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    Ob_ref, Lb_ref = oracle.attend(wb.problem, wb.buffers)
    assert np.array_equal(Or, Ob_ref) and np.array_equal(Lr, Lb_ref)   # the format is exact here
    O8, L8, _ = H.forward(w)
    Ob, Lb, _ = H.forward(wb)
    H.check_rows(O8, L8, Ob, Lb, 2e-3)
    H.check_rows(O8, L8, Or, Lr, 2e-3)
    e, le = H.errors(O8, L8, Ob, Lb)
    H.announce(f"exact-quantization pin {mask or 'causal'}: int8 vs bf16 GPU max|dO| = {e:.3e}, "
               f"max|dLSE| = {le:.3e}")


def test_residual_only_int8_equals_bf16():
    B, T, Hkv, D = 3, 2000, 8, 128
    lens = [2000, 700, 90]
    mask = dict(mask_kind="sink_window", n_sink=0, window=100)
    w = synth.make_int8(32, B, 32, Hkv, D, lens, residual_len=128, kv_capacity=T, **mask)
    kf, vf = w.float_kv
    wb = _bf16_twin(w, kf, vf, exact=False, **mask)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    Ob_ref, Lb_ref = oracle.attend(wb.problem, wb.buffers)
    assert np.array_equal(Or, Ob_ref) and np.array_equal(Lr, Lb_ref)   # no code is visible
    O8, L8, _ = H.forward(w)
    Ob, Lb, _ = H.forward(wb)
    H.check_rows(O8, L8, Ob, Lb, 2e-3)
    e, le = H.errors(O8, L8, Ob, Lb)
    H.announce(f"residual-only pin: int8 vs bf16 GPU max|dO| = {e:.3e}, max|dLSE| = {le:.3e}")


def test_int8_operands_outside_fp16_range():
    """The int8 kernel feeds fp16 matrix-core operands, whose range ends at
    65504.  Inputs the format allows beyond that range give finite results
    that match the oracle: a K value of 1e5 (its group's channel scale is
    787.5, so code * scale reaches 1e5), query elements of +-7e4, a request
    whose K scales are all large, and a request with small V values (|V| ~
    0.03, whose weighted scales would fall below fp16's normal range)."""
    B, T, Hkv, D = 4, 2048, 8, 128
    g = synth.rng(33)
    kf = g.standard_normal((B, T, Hkv, D), dtype=np.float32)
    vf = g.standard_normal((B, T, Hkv, D), dtype=np.float32)
    kf[0, 100, 3, 7] = 1e5
    kf[1] *= 3e4
    vf[2] *= 0.01
    lens = [2048, 2000, 1900, 1500]
    w = synth.make_int8(33, B, 32, Hkv, D, lens, kv_capacity=T, values=(kf, vf))
    assert float(w.buffers["k_scale"][0, 0, 3, 7]) == 787.5
    q = w.buffers["q"]
    q[3, 5, 11] = synth.bf16_bits(np.float32(7e4))
    q[1, 20, 3] = synth.bf16_bits(np.float32(-7e4))
    Or, Lr = oracle.attend(w.problem, w.buffers)
    for fn in (H.forward, H.run):
        O, L, _ = fn(w)
        assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
        for b in range(B):       # each request against its own output scale
            H.check_rows(O[b:b + 1], L[b:b + 1], Or[b:b + 1], Lr[b:b + 1], 0.0, rtol=1e-2)
            e, le = H.errors(O[b:b + 1], L[b:b + 1], Or[b:b + 1], Lr[b:b + 1])
            H.announce(f"range case request {b}: max|dO| = {e:.3e} (max|O_ref| = "
                       f"{float(np.max(np.abs(Or[b]))):.3g}), max|dLSE| = {le:.3e}")
