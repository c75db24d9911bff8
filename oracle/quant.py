"""Symmetric int8 quantizer and the int8 K/V format (test infrastructure only).

M8.6 §0x02A: for a finite non-empty row x, the scale is ``amax/qmax`` stored in
the declared qparam dtype and re-read before encoding (the stored value is the
effective qparam); an all-zero row gets scale 1 and zero codes; codes are
``clip(round(x/s), -qmax, qmax)`` with ties to even; a stored scale that is
non-finite or subnormal is rejected.  qmax = 2^(bits-1) - 1 (narrow range).

The K/V format applies that rule along the axes of M8.6 §0x06/§0x06A: K per
channel over a closed group of tokens, V per token over its channels; the
newest tokens stay in bf16 (§0x06B residual).  Decoding is ``code * scale``
for both (§0x03B, §0x03C).  This writer is independent of the input module's
writer; the CPU tests require both to produce identical bytes.
"""
from __future__ import annotations

import numpy as np


def quantize_symmetric_rows(x, bits: int = 8, qparam_dtype=np.float16):
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2 or 0 in x.shape or not np.isfinite(x).all():
        raise ValueError("expected finite, non-empty [M, K] rows")
    if not (isinstance(bits, int) and 2 <= bits <= 8):
        raise ValueError("bits must be an int in [2, 8]")
    dt = np.dtype(qparam_dtype)
    qmax = 2 ** (bits - 1) - 1
    amax = np.abs(x).max(axis=1)
    zero = amax == 0
    ideal = np.where(zero, 1.0, amax / qmax)
    with np.errstate(over="ignore", under="ignore"):
        stored = ideal.astype(dt)
    eff = stored.astype(np.float64)
    if not np.isfinite(eff).all() or np.any(eff < np.finfo(dt).tiny):
        raise ValueError("non-representable or subnormal stored scale")
    codes = np.clip(np.rint(x / eff[:, None]), -qmax, qmax)
    codes[zero] = 0
    return codes.astype(np.int8), stored


def write_int8_cache_oracle(k_f32, v_f32, seq_lens, k_group: int, residual_len: int):
    """Return, per request b, the meaningful parts of the stored format:
    ``{b: dict(n_q, k_codes[n_q,H,D], k_scale[groups,H,D], v_codes[n_q,H,D],
    v_scale[n_q,H], k_resid_bits[n_res,H,D], v_resid_bits[n_res,H,D])}``."""
    k_f32 = np.asarray(k_f32, dtype=np.float32)
    v_f32 = np.asarray(v_f32, dtype=np.float32)
    B, _, H, D = k_f32.shape
    out = {}
    for b in range(B):
        T = int(seq_lens[b])
        n_res = min(T, residual_len)
        n_q = T - n_res
        n_groups = -(-n_q // k_group)
        kc = np.zeros((n_q, H, D), np.int8)
        ks = np.zeros((n_groups, H, D), np.float16)
        vc = np.zeros((n_q, H, D), np.int8)
        vs = np.zeros((n_q, H), np.float16)
        for h in range(H):
            for j in range(n_groups):
                lo, hi = j * k_group, min((j + 1) * k_group, n_q)
                # channels become rows: one scale per channel of this group
                codes, scale = quantize_symmetric_rows(k_f32[b, lo:hi, h, :].T)
                kc[lo:hi, h, :] = codes.T
                ks[j, h, :] = scale
            if n_q:
                codes, scale = quantize_symmetric_rows(v_f32[b, :n_q, h, :])
                vc[:, h, :] = codes
                vs[:, h] = scale
        kr = _bf16_rne(k_f32[b, n_q:T])
        vr = _bf16_rne(v_f32[b, n_q:T])
        out[b] = dict(n_q=n_q, k_codes=kc, k_scale=ks, v_codes=vc, v_scale=vs,
                      k_resid_bits=kr, v_resid_bits=vr)
    return out


def _bf16_rne(x):
    """Round finite fp32 values to bf16 bit patterns, nearest, ties to even.

    Written as a comparison of distances in fp64: the candidates are the value
    truncated toward zero to 8 significant bits and its neighbour one bf16 ulp
    further from zero."""
    x = np.asarray(x, np.float32)
    w = x.view(np.uint32)
    lo_bits = (w >> 16).astype(np.uint32)                  # truncated toward zero
    hi_bits = lo_bits + 1                                  # next magnitude up
    lo = (lo_bits << 16).view(np.float32).astype(np.float64)
    hi = (hi_bits << 16).view(np.float32).astype(np.float64)
    xv = x.astype(np.float64)
    d_lo = np.abs(xv - lo)
    d_hi = np.abs(hi - xv)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((lo_bits & 1) == 1))
    return np.where(pick_hi, hi_bits, lo_bits).astype(np.uint16)
