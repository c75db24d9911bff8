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
