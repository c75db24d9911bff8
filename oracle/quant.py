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

Two residual policies fix which tokens are quantized (n_q of them, the oldest):

* ``"window"``: the newest min(T, R) tokens are bf16, n_q = T - min(T, R)
  (a snapshot of the cache; the last K group may be partial);
* ``"groups"``: the streaming rule of M8.6 §0x06B -- every appended row enters
  the bf16 residual, and while the residual holds more than R rows its oldest
  G rows are closed: K quantized per channel over those G rows, V per row.
  Closed groups never change afterwards.  ``kivi_append`` is that rule applied
  to one token; ``quantized_count`` is its closed form, pinned against it.
  Rows enter as bf16, so closed groups quantize bf16 values.
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


def quantized_count(T: int, policy: str, k_group: int, residual_len: int) -> int:
    """Number n_q of oldest tokens held as int8 codes at length T."""
    T = int(T)
    if policy == "window":
        return T - min(T, residual_len)
    if policy == "groups":
        excess = T - residual_len
        return k_group * max(0, -(-excess // k_group))
    raise ValueError(policy)


def write_int8_cache_oracle(k_f32, v_f32, seq_lens, k_group: int, residual_len: int,
                            policy: str = "window"):
    """Return, per request b, the meaningful parts of the stored format:
    ``{b: dict(n_q, k_codes[n_q,H,D], k_scale[groups,H,D], v_codes[n_q,H,D],
    v_scale[n_q,H], k_resid_bits[n_res,H,D], v_resid_bits[n_res,H,D])}``.
    With ``policy="groups"`` the rows are rounded to bf16 before anything is
    quantized (they were appended as bf16 rows)."""
    k_f32 = np.asarray(k_f32, dtype=np.float32)
    v_f32 = np.asarray(v_f32, dtype=np.float32)
    if policy == "groups":
        k_f32 = (_bf16_rne(k_f32).astype(np.uint32) << 16).view(np.float32)
        v_f32 = (_bf16_rne(v_f32).astype(np.uint32) << 16).view(np.float32)
    B, _, H, D = k_f32.shape
    out = {}
    for b in range(B):
        T = int(seq_lens[b])
        n_q = quantized_count(T, policy, k_group, residual_len)
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


# ---------------------------------------------------------------------------
# Streaming append (M8.6 §0x06B, the synchronized-tail teaching state).
# ---------------------------------------------------------------------------
def kivi_empty_state(H: int, D: int) -> dict:
    """One request's cache state: closed K groups (codes [G, H, D], scales
    [H, D]), closed V rows (codes [H, D], scales [H]) and the bf16 residual
    rows (bit patterns [H, D]), oldest first."""
    return dict(H=H, D=D, k_groups=[], v_rows=[], k_resid=[], v_resid=[])


def kivi_append(state: dict, k_row_bits, v_row_bits, k_group: int, residual_len: int) -> dict:
    """Append one token (bf16 bit patterns ``[H, D]`` for K and V): the row
    joins the residual; while the residual holds more than ``residual_len``
    rows, its oldest ``k_group`` rows are closed -- K quantized per channel
    over those rows (one scale per channel and head), V per row (one scale per
    row and head) -- and leave the residual.  Raises ValueError (leaving the
    state unchanged) if a scale is not representable."""
    k_resid = state["k_resid"] + [np.asarray(k_row_bits, np.uint16)]
    v_resid = state["v_resid"] + [np.asarray(v_row_bits, np.uint16)]
    k_groups, v_rows = list(state["k_groups"]), list(state["v_rows"])
    H, D = state["H"], state["D"]
    while len(k_resid) > residual_len:
        k_old = _bits_to_f64(np.stack(k_resid[:k_group]))          # [G, H, D]
        v_old = _bits_to_f64(np.stack(v_resid[:k_group]))
        kc = np.empty(k_old.shape, np.int8)
        ks = np.empty((H, D), np.float16)
        vc = np.empty(v_old.shape, np.int8)
        vs = np.empty((k_old.shape[0], H), np.float16)
        for h in range(H):
            codes, scale = quantize_symmetric_rows(k_old[:, h, :].T)     # channels as rows
            kc[:, h, :] = codes.T
            ks[h] = scale
            codes, scale = quantize_symmetric_rows(v_old[:, h, :])       # tokens as rows
            vc[:, h, :] = codes
            vs[:, h] = scale
        k_groups.append((kc, ks))
        for i in range(k_old.shape[0]):
            v_rows.append((vc[i], vs[i]))
        del k_resid[:k_group]
        del v_resid[:k_group]
    return dict(H=H, D=D, k_groups=k_groups, v_rows=v_rows, k_resid=k_resid, v_resid=v_resid)


def kivi_state_parts(state: dict) -> dict:
    """The state in the layout of ``write_int8_cache_oracle``'s per-request
    dict (n_q, codes, scales, residual bits)."""
    H, D = state["H"], state["D"]
    n_q = len(state["v_rows"])
    kc = (np.concatenate([g[0] for g in state["k_groups"]]) if state["k_groups"]
          else np.zeros((0, H, D), np.int8))
    ks = (np.stack([g[1] for g in state["k_groups"]]) if state["k_groups"]
          else np.zeros((0, H, D), np.float16))
    vc = np.stack([r[0] for r in state["v_rows"]]) if n_q else np.zeros((0, H, D), np.int8)
    vs = np.stack([r[1] for r in state["v_rows"]]) if n_q else np.zeros((0, H), np.float16)
    kr = np.stack(state["k_resid"]) if state["k_resid"] else np.zeros((0, H, D), np.uint16)
    vr = np.stack(state["v_resid"]) if state["v_resid"] else np.zeros((0, H, D), np.uint16)
    return dict(n_q=n_q, k_codes=kc, k_scale=ks, v_codes=vc, v_scale=vs,
                k_resid_bits=kr, v_resid_bits=vr)


def kivi_state_from_parts(parts: dict, k_group: int) -> dict:
    """Inverse of ``kivi_state_parts`` for a state whose quantized rows form
    whole groups."""
    kc, ks = parts["k_codes"], parts["k_scale"]
    n_q = int(parts["n_q"])
    if n_q % k_group:
        raise ValueError("closed rows must form whole groups")
    H, D = parts["k_resid_bits"].shape[1:] if parts["k_resid_bits"].size else kc.shape[1:]
    return dict(H=H, D=D,
                k_groups=[(kc[j * k_group:(j + 1) * k_group].copy(), ks[j].copy())
                          for j in range(n_q // k_group)],
                v_rows=[(parts["v_codes"][i].copy(), parts["v_scale"][i].copy()) for i in range(n_q)],
                k_resid=[r.copy() for r in parts["k_resid_bits"]],
                v_resid=[r.copy() for r in parts["v_resid_bits"]])


def _bits_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
