"""Symmetric int8 quantizer and the int8 K/V format (test infrastructure only).

The rule (M8.6 §0x02A): the elements that share one scale are quantized with
scale = amax / qmax, where amax is their largest magnitude and qmax =
2^(bits-1) - 1 (narrow range, so -128 never occurs); the scale is committed
to its storage type (fp16 here) before any code is formed, and the committed
value is the one used; codes are x / scale rounded to the nearest integer
(ties to even) and clipped to [-qmax, qmax]; a group of zeros uses the exact
sentinel scale 1 and zero codes; a committed scale that is infinite or below
the smallest normal fp16 value is refused.

The K/V format applies the rule along the axes of M8.6 §0x06/§0x06A: K shares
a scale per channel across a closed group of tokens, V per token across its
channels; the newest tokens stay in bf16 (§0x06B residual).  Decoding is
``code * scale`` for both (§0x03B, §0x03C).  This writer is independent of the
input module's writer; the CPU tests require both to produce identical bytes.

Two residual policies fix which tokens are quantized (n_q of them, the oldest):

* ``"window"``: the newest min(T, R) tokens are bf16, n_q = T - min(T, R)
  (a snapshot of the cache; the last K group may be partial);
* ``"groups"``: the streaming rule of M8.6 §0x06B: a new row always enters
  the bf16 residual, and whenever the residual has grown past R rows its
  oldest G rows are closed (K per channel over them, V per row) and leave it,
  so the closed count is the smallest multiple of G that leaves at most R
  rows open.  ``kivi_append`` applies the rule to one token by comparing that
  count before and after the token; closed groups are never touched again.
  Rows enter as bf16, so closed groups quantize bf16 values.
"""
from __future__ import annotations

import numpy as np

FP16_MAX = 65504.0
FP16_MIN_NORMAL = 2.0 ** -14


def fp16_round(v):
    """Nearest binary16 value of each non-negative fp64 ``v`` (ties to even),
    returned as fp64: inf past the largest finite value, subnormal values on
    the 2^-24 grid below 2^-14.  A binary16 number in [2^(e-1), 2^e) has 11
    significant bits, so its spacing is 2^(e-11) (never below 2^-24)."""
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    spacing = np.ldexp(1.0, np.maximum(e - 11, -24))
    r = np.rint(v / spacing) * spacing
    return np.where(r > FP16_MAX, np.inf, r)


def quantize_symmetric(x, axis, bits: int = 8):
    """Quantize ``x`` with one fp16 scale per slice along ``axis`` (the
    elements along ``axis`` share a scale).  Returns ``(codes int8 with x's
    shape, scales float16 with x's shape minus axis)``.  Raises ValueError for
    an empty or non-finite input or a refused committed scale."""
    x = np.asarray(x, dtype=np.float64)
    if x.size == 0 or not np.isfinite(x).all():
        raise ValueError("expected finite, non-empty values")
    if not (isinstance(bits, int) and 2 <= bits <= 8):
        raise ValueError("bits must be an int in [2, 8]")
    qmax = (1 << (bits - 1)) - 1
    peak = np.abs(x).max(axis=axis, keepdims=True)
    raw = np.divide(peak, qmax, out=np.ones_like(peak), where=peak > 0)
    committed = fp16_round(raw)
    if not np.all(np.isfinite(committed) & (committed >= FP16_MIN_NORMAL)):
        raise ValueError("committed fp16 scale is infinite or not normal")
    codes = np.clip(np.rint(x / committed), -qmax, qmax).astype(np.int8)
    return codes, np.squeeze(committed, axis=axis).astype(np.float16)


def quantize_symmetric_rows(x, bits: int = 8):
    """``quantize_symmetric`` of an ``[M, K]`` array with one scale per row."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2:
        raise ValueError("expected [M, K] rows")
    return quantize_symmetric(x, axis=1, bits=bits)


def quantized_count(T: int, policy: str, k_group: int, residual_len: int) -> int:
    """Number n_q of oldest tokens held as int8 codes at length T."""
    T = int(T)
    if policy == "window":
        return T - min(T, residual_len)
    if policy == "groups":
        excess = T - residual_len
        return k_group * max(0, -(-excess // k_group))
    raise ValueError(policy)


def _close_block(k_rows, v_rows):
    """Quantize one block of consecutive tokens (``[n, H, D]`` fp64 each) in
    the K/V format: K shares a scale per (head, channel) over the block's
    tokens, V per (token, head) over the channels.  Returns (K codes [n, H,
    D], K scales [H, D], V codes [n, H, D], V scales [n, H])."""
    kc, ks = quantize_symmetric(k_rows, axis=0)
    vc, vs = quantize_symmetric(v_rows, axis=2)
    return kc, ks, vc, vs


def _via_bf16(x):
    """fp32 values after a round trip through bf16 (nearest, ties to even)."""
    return (_bf16_rne(x).astype(np.uint32) << 16).view(np.float32)


def write_int8_cache_oracle(k_f32, v_f32, seq_lens, k_group: int, residual_len: int,
                            policy: str = "window"):
    """Return, per request b, the meaningful parts of the stored format:
    ``{b: dict(n_q, k_codes[n_q,H,D], k_scale[groups,H,D], v_codes[n_q,H,D],
    v_scale[n_q,H], k_resid_bits[n_res,H,D], v_resid_bits[n_res,H,D])}``.
    The quantized tokens are closed in blocks of ``k_group`` (the last block of
    the window policy may be shorter).  With ``policy="groups"`` the rows are
    rounded to bf16 first (they were appended as bf16 rows)."""
    k = np.asarray(k_f32, dtype=np.float32)
    v = np.asarray(v_f32, dtype=np.float32)
    if policy == "groups":
        k, v = _via_bf16(k), _via_bf16(v)
    H, D = k.shape[2], k.shape[3]
    out = {}
    for b, T in enumerate(int(t) for t in seq_lens):
        n_q = quantized_count(T, policy, k_group, residual_len)
        blocks = [_close_block(k[b, lo:min(lo + k_group, n_q)].astype(np.float64),
                               v[b, lo:min(lo + k_group, n_q)].astype(np.float64))
                  for lo in range(0, n_q, k_group)]
        part = [[blk[i] for blk in blocks] for i in range(4)]
        out[b] = dict(
            n_q=n_q,
            k_codes=np.concatenate(part[0]) if blocks else np.zeros((0, H, D), np.int8),
            k_scale=np.stack(part[1]) if blocks else np.zeros((0, H, D), np.float16),
            v_codes=np.concatenate(part[2]) if blocks else np.zeros((0, H, D), np.int8),
            v_scale=np.concatenate(part[3]) if blocks else np.zeros((0, H), np.float16),
            k_resid_bits=_bf16_rne(k[b, n_q:T]),
            v_resid_bits=_bf16_rne(v[b, n_q:T]))
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
#
# A request's state: closed K groups (codes [G, H, D], scales [H, D]), closed V
# rows (codes [H, D], scales [H]) and the open bf16 rows (bit patterns [H, D]),
# oldest first.  The number of closed rows is a function of the token count
# alone (``quantized_count`` under the "groups" policy), so one append closes
# exactly the rows that count says became closed.
# ---------------------------------------------------------------------------
def kivi_empty_state(H: int, D: int) -> dict:
    return dict(H=H, D=D, k_groups=[], v_rows=[], k_resid=[], v_resid=[])


def kivi_append(state: dict, k_row_bits, v_row_bits, k_group: int, residual_len: int) -> dict:
    """Return the state after appending one token (bf16 bit patterns
    ``[H, D]`` for K and V).  The open rows that the new token count closes
    are quantized in blocks of ``k_group`` and move to the closed lists.  The
    given state is never modified; a refused scale raises ValueError."""
    open_k = list(state["k_resid"]) + [np.asarray(k_row_bits, np.uint16)]
    open_v = list(state["v_resid"]) + [np.asarray(v_row_bits, np.uint16)]
    n_closed = len(state["v_rows"])
    newly = quantized_count(n_closed + len(open_k), "groups", k_group, residual_len) - n_closed
    k_groups, v_rows = list(state["k_groups"]), list(state["v_rows"])
    for lo in range(0, newly, k_group):
        kc, ks, vc, vs = _close_block(_bits_to_f64(np.stack(open_k[lo:lo + k_group])),
                                      _bits_to_f64(np.stack(open_v[lo:lo + k_group])))
        k_groups.append((kc, ks))
        v_rows.extend(zip(vc, vs))
    return dict(H=state["H"], D=state["D"], k_groups=k_groups, v_rows=v_rows,
                k_resid=open_k[newly:], v_resid=open_v[newly:])


def kivi_state_parts(state: dict) -> dict:
    """The state in the layout of ``write_int8_cache_oracle``'s per-request
    dict (n_q, codes, scales, residual bits)."""
    H, D = state["H"], state["D"]
    n_q = len(state["v_rows"])

    def cat(items, shape, dtype, join):
        return join(items) if items else np.zeros(shape, dtype)
    return dict(
        n_q=n_q,
        k_codes=cat([c for c, _ in state["k_groups"]], (0, H, D), np.int8, np.concatenate),
        k_scale=cat([s for _, s in state["k_groups"]], (0, H, D), np.float16, np.stack),
        v_codes=cat([c for c, _ in state["v_rows"]], (0, H, D), np.int8, np.stack),
        v_scale=cat([s for _, s in state["v_rows"]], (0, H), np.float16, np.stack),
        k_resid_bits=cat(state["k_resid"], (0, H, D), np.uint16, np.stack),
        v_resid_bits=cat(state["v_resid"], (0, H, D), np.uint16, np.stack))


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
