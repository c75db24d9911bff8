"""Pins of the int8 K/V format: the quantizer rule of M8.6 §0x02A applied along
the axes of M8.6 §0x06/§0x06A with the bf16 residual of §0x06B, and the
decoded-reference attention of M8.6 §0x0CA/§0x0CB."""
import math

import numpy as np
import pytest

import oracle
import synth
from oracle.numerics import decode_bf16, decode_f16
from oracle.quant import quantize_symmetric_rows, write_int8_cache_oracle


def test_quantizer_endpoint_zero_clip_and_error():
    g = synth.rng(1)
    x = g.standard_normal((50, 33)) * np.exp(g.standard_normal((50, 1)))
    x[3] = 0.0
    codes, s = quantize_symmetric_rows(x)
    eff = s.astype(np.float64)
    assert codes.dtype == np.int8 and s.dtype == np.float16
    assert eff[3] == 1.0 and not codes[3].any()
    for r in range(50):
        if r == 3:
            continue
        j = np.argmax(np.abs(x[r]))
        # endpoint: the largest magnitude maps to +-127 (unless fp16 rounding of
        # the scale moved it just past the endpoint, where clipping applies)
        assert abs(int(codes[r, j])) == 127
        err = np.abs(x[r] - eff[r] * codes[r])
        unclipped = np.abs(x[r] / eff[r]) <= 127
        assert np.all(err[unclipped] <= eff[r] / 2 * (1 + 1e-12))
    assert np.abs(codes).max() <= 127   # narrow range: -128 never used


def test_quantizer_rejects_bad_inputs_and_scales():
    with pytest.raises(ValueError):
        quantize_symmetric_rows(np.array([[1.0, np.nan]]))
    with pytest.raises(ValueError):
        quantize_symmetric_rows(np.array([[1e9, 1.0]]))       # scale overflows fp16
    with pytest.raises(ValueError):
        quantize_symmetric_rows(np.array([[1e-7, 0.0]]))      # subnormal fp16 scale
    with pytest.raises(ValueError):
        quantize_symmetric_rows(np.zeros((0, 4)))


def test_fp16_commit_matches_ieee_binary16():
    """The oracle's own binary16 rounding equals NumPy's IEEE conversion on
    random magnitudes across the whole range and on the edges: the largest
    finite value, the overflow midpoint 65520 (ties to even: inf), the
    smallest normal 2^-14 and the midpoint below it (ties to even: 2^-14)."""
    from oracle.quant import fp16_round
    g = synth.rng(11)
    v = np.exp(g.uniform(np.log(1e-9), np.log(1e6), 20000))
    edges = [65504.0, 65519.999, 65520.0, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25,
             2.0 ** -14 - 2.0 ** -24, 2.0 ** -24, 2.0 ** -25, 1.0, 1.0 + 2.0 ** -11, 0.0]
    v = np.concatenate([v, np.array(edges)])
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).astype(np.float64)
    assert np.array_equal(fp16_round(v), ref)


def test_quantizer_axis_equals_rows_of_the_moved_axis():
    """One scale per slice along an axis is the row quantizer applied to the
    array with that axis moved last."""
    from oracle.quant import quantize_symmetric
    g = synth.rng(12)
    x = g.standard_normal((5, 3, 7)) * np.exp(g.standard_normal((5, 3, 1)))
    for axis in range(3):
        c, s = quantize_symmetric(x, axis=axis)
        moved = np.moveaxis(x, axis, -1)
        c2, s2 = quantize_symmetric_rows(moved.reshape(-1, moved.shape[-1]))
        assert np.array_equal(np.moveaxis(c, axis, -1).reshape(c2.shape), c2)
        assert np.array_equal(s.reshape(-1).view(np.uint16), s2.view(np.uint16))


def test_ties_round_to_even():
    # scale 1 (amax 127): 2.5 -> 2, 3.5 -> 4, -2.5 -> -2
    codes, s = quantize_symmetric_rows(np.array([[127.0, 2.5, 3.5, -2.5, 0.5]]))
    assert float(s[0]) == 1.0
    assert codes.tolist() == [[127, 2, 4, -2, 0]]


@pytest.mark.parametrize("lens", [[300, 128, 5], [0, 257, 129]])
def test_writers_agree_byte_for_byte(lens):
    w = synth.make_int8(3, len(lens), 4, 2, 16, lens, k_group=64, residual_len=32,
                        kv_capacity=320)
    kf, vf = w.float_kv
    ref = write_int8_cache_oracle(kf, vf, lens, 64, 32)
    bf = w.buffers
    for b, r in ref.items():
        n_q = r["n_q"]
        assert np.array_equal(bf["k"][b, :n_q], r["k_codes"])
        assert np.array_equal(bf["v"][b, :n_q], r["v_codes"])
        assert np.array_equal(bf["k_scale"][b, :len(r["k_scale"])].view(np.uint16),
                              r["k_scale"].view(np.uint16))
        assert np.array_equal(bf["v_scale"][b, :n_q].view(np.uint16), r["v_scale"].view(np.uint16))
        n_res = len(r["k_resid_bits"])
        assert np.array_equal(bf["k_resid"][b, :n_res], r["k_resid_bits"])
        assert np.array_equal(bf["v_resid"][b, :n_res], r["v_resid_bits"])


def _decoded_reference(w):
    """Dequantize with direct multi-axis indexing into a plain f32 cache."""
    p, bf = w.problem, w.buffers
    B, T_cap, H, D = bf["k"].shape
    K = np.zeros((B, T_cap, H, D), np.float32)
    V = np.zeros((B, T_cap, H, D), np.float32)
    for b in range(B):
        T = int(bf["seq_lens"][b])
        n_q = T - min(T, p.residual_len)
        for t in range(T):
            if t < n_q:
                K[b, t] = bf["k"][b, t].astype(np.float64) * decode_f16(bf["k_scale"][b, t // p.k_group])
                V[b, t] = bf["v"][b, t].astype(np.float64) * decode_f16(bf["v_scale"][b, t])[:, None]
            else:
                K[b, t] = decode_bf16(bf["k_resid"][b, t - n_q])
                V[b, t] = decode_bf16(bf["v_resid"][b, t - n_q])
    q = decode_bf16(bf["q"]).astype(np.float32)
    prob = synth.Problem(batch=B, num_q_heads=p.num_q_heads, num_kv_heads=H, head_dim=D,
                         q_dtype="f32", kv_format="f32", kv_capacity=T_cap,
                         max_seq_len=p.max_seq_len, mask_kind=p.mask_kind, n_sink=p.n_sink,
                         window=p.window)
    return prob, dict(q=q, k=K, v=V, seq_lens=bf["seq_lens"])


@pytest.mark.parametrize("mask", [("causal", 0, 0), ("sink_window", 4, 100)])
def test_int8_oracle_equals_decoded_reference(mask):
    w = synth.make_int8(8, 2, 4, 2, 16, [300, 77], k_group=64, residual_len=32,
                        mask_kind=mask[0], n_sink=mask[1], window=mask[2])
    O, L = oracle.attend(w.problem, w.buffers)
    p2, b2 = _decoded_reference(w)
    O2, L2 = oracle.attend(p2, b2)
    # every decoded value is exact in fp32 (8-bit code x 11-bit fp16 significand)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)


def _exact_grid_values(g, B, T, H, D, k_group):
    """K: per (group, channel) values c*2^-5 with one +-127 in each group;
    V: per token values c*2^-6 with one +-127 in each row.  Both quantize
    exactly, with scales 2^-5 and 2^-6."""
    ck = g.integers(-126, 127, size=(B, T, H, D))
    for b in range(B):
        for h in range(H):
            for j in range(0, T, k_group):
                hi = min(T, j + k_group)
                t = g.integers(j, hi, size=D)
                ck[b, t, h, np.arange(D)] = 127 * np.where(g.integers(0, 2, D) == 1, 1, -1)
    cv = g.integers(-126, 127, size=(B, T, H, D))
    x = g.integers(0, D, size=(B, T, H))
    np.put_along_axis(cv, x[..., None], -127, axis=3)
    return (ck * 2.0 ** -5).astype(np.float32), (cv * 2.0 ** -6).astype(np.float32)


def test_exact_quantization_pin():
    """Values on the int8 grid quantize exactly, so the int8 and bf16 caches of
    the same values give the same oracle output."""
    B, T, H, D, G = 2, 256, 2, 16, 64
    g = synth.rng(21)
    kf, vf = _exact_grid_values(g, B, T, H, D, G)
    lens = [256, 256]
    w = synth.make_int8(21, B, 4, H, D, lens, k_group=G, residual_len=G, values=(kf, vf))
    O8, L8 = oracle.attend(w.problem, w.buffers)
    wb = synth.make_contiguous(21, B, 4, H, D, lens, dtype="bf16", poison_tail=False)
    wb.buffers["q"] = w.buffers["q"]
    wb.buffers["k"] = synth.bf16_bits(kf)
    wb.buffers["v"] = synth.bf16_bits(vf)
    assert np.array_equal(decode_bf16(wb.buffers["k"]), kf.astype(np.float64))
    Ob, Lb = oracle.attend(wb.problem, wb.buffers)
    assert np.array_equal(O8, Ob) and np.array_equal(L8, Lb)


def test_residual_only_pin():
    """A window inside the bf16 residual makes the int8 result equal the bf16
    result of the same values (the quantized region is never visible)."""
    B, T, H, D = 2, 200, 2, 16
    w = synth.make_int8(22, B, 4, H, D, [T, 150], k_group=64, residual_len=32,
                        mask_kind="sink_window", n_sink=0, window=20)
    kf, vf = w.float_kv
    O8, L8 = oracle.attend(w.problem, w.buffers)
    wb = synth.make_contiguous(22, B, 4, H, D, [T, 150], dtype="bf16", mask_kind="sink_window",
                               n_sink=0, window=20, poison_tail=False)
    wb.buffers["q"] = w.buffers["q"]
    wb.buffers["k"] = synth.bf16_bits(kf)
    wb.buffers["v"] = synth.bf16_bits(vf)
    Ob, Lb = oracle.attend(wb.problem, wb.buffers)
    assert np.array_equal(O8, Ob) and np.array_equal(L8, Lb)


def test_int8_sink_window_visible_rows_count_cfg5_shape():
    # 4 sinks + window 4096 at T = 16384: 4100 visible rows, 128 in the residual
    A = oracle.visible_positions(16384, "sink_window", 4, 4096)
    assert len(A) == 4100
    n_q = 16384 - 128
    assert int((A >= n_q).sum()) == 128
    assert math.ceil(n_q / 128) == 127


@pytest.mark.parametrize("amax,ok", [(1e9, False), (65519.0 * 127, True), (65520.0 * 127, False),
                                     (1e-7, False), ((2.0 ** -14 - 2.0 ** -25) * 127, True),
                                     ((2.0 ** -14 - 2.0 ** -24) * 127, False)])
def test_both_writers_refuse_the_same_scales(amax, ok):
    """The input module's writer and the oracle's writer accept and refuse the
    same groups at the edges of the fp16 scale range (M8.6 §0x02A)."""
    kf = np.zeros((1, 4, 1, 8), np.float32)
    kf[0, 0, 0, 0] = amax
    vf = np.ones((1, 4, 1, 8), np.float32)
    def oracle_side():
        return write_int8_cache_oracle(kf, vf, [4], 4, 0)
    def input_side():
        return synth.write_int8_cache(kf, vf, [4], 4, 0, 4, synth.rng(0))
    for fn in (oracle_side, input_side):
        if ok:
            fn()
        else:
            with pytest.raises(ValueError):
                fn()
