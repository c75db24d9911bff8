"""Decode attention by its plain definition, in fp64 (test infrastructure only).

For every output row (b, h_q), with ``h_kv = h_q // g`` and ``g = H_q/H_kv``
(M4.5 §0x03A, §0x04A):

    s_t = (q . k_t) * scale,  scale = 1/sqrt(d_h)       (M4.5 §0x01, §0x05D)
    O   = softmax(s over the visible set A_b) @ V        (M4.5 §0x01)
    LSE = m + ln(sum_t e^(s_t - m)),  m = max s           (M4.5 §0x02B)

and for an empty A_b (length 0 or everything masked): ``O = 0``, ``LSE = -inf``
(M4.5 §0x02C).  The visible set comes from ``visibility.visible_positions``;
rows are located through ``address`` with the oracle's own translation and
decoded from the stored bytes (``numerics``); int8 rows are ``code * scale``
with the K scale of the token's 128-token group and channel and the V scale
of the token (M8.6 §0x03B, §0x03C), and the tokens from n_q on (the newest
``min(T_b, R)`` under the window policy, the unclosed tail under the group
policy; ``quant.quantized_count``) come from the bf16 residual, row t - n_q
(M8.6 §0x06B/§0x06C: one shared softmax over both regions).

``split_attend`` is the Flash-Decoding reference: it summarizes each
physical split of the visible positions (M4.5 §0x02A, §0x03I), merges the
states in the order given (§0x02B, §0x02C) and finalizes.  It exists to pin
the algebra (partition invariance, §0x02E) and to check GPU workspace states.
"""
from __future__ import annotations

import math

import numpy as np

from .address import (csr_page, hnd_offset, nhd_offset, paged_hnd_offset, paged_nhd_offset,
                      ragged_nhd_offset, ring_slot)
from .numerics import decode, decode_bf16, decode_f16
from . import flashmask
from .quant import quantized_count
from .state import EMPTY, finalize, merge_state, summarize_allowed
from .visibility import query_row_length, visible_positions


def _scale(prob) -> float:
    return float(prob.softmax_scale) if prob.softmax_scale else 1.0 / math.sqrt(prob.head_dim)


def gather_rows(prob, buf, b: int, h_kv: int, positions, scale_offsets=None):
    """K and V rows (fp64, ``[n, D]``) of the given logical positions of
    request b and K/V head h_kv, plus the element offset of each row inside the
    buffer it was read from and the region tag (0: main cache or int8 codes,
    1: bf16 residual).  For the int8 format, ``scale_offsets`` (a dict, if
    given) receives the element offsets of the scales each row was decoded
    with: ``"k"`` the first element of its K scale row in ``k_scale``, ``"v"``
    its V scale in ``v_scale`` (-1 for residual rows)."""
    D = prob.head_dim
    H = prob.num_kv_heads
    positions = np.asarray(positions, dtype=np.int64)
    n = positions.size
    lane = np.arange(D, dtype=np.int64)
    region = np.zeros(n, dtype=np.int8)
    if prob.kv_format in ("f32", "bf16"):
        layout = prob.layout
        if layout in ("contig", "contig_hnd"):
            bidx = buf.get("cache_batch_idx")
            c = int(bidx[b]) if bidx is not None else b
            fn = nhd_offset if layout == "contig" else hnd_offset
            offs = fn(c, positions, h_kv, 0, prob.kv_capacity, H, D)
        elif layout == "ragged":
            offs = ragged_nhd_offset(buf["indptr"], b, positions, h_kv, 0, H, D)
        elif layout == "ring":
            bidx = buf.get("cache_batch_idx")
            c = int(bidx[b]) if bidx is not None else b
            slots = ring_slot(positions, prob.n_sink, prob.window)
            offs = nhd_offset(c, slots, h_kv, 0, prob.n_sink + prob.window, H, D)
        elif layout in ("paged", "paged_hnd"):
            P = prob.page_size
            if getattr(prob, "page_table", "dense") == "csr":
                pages = np.array([csr_page(buf["indptr"], buf["block_table"], b, j)
                                  for j in (positions // P)], dtype=np.int64)
            else:
                pages = buf["block_table"][b][positions // P].astype(np.int64)
            fn = paged_nhd_offset if layout == "paged" else paged_hnd_offset
            offs = fn(pages, positions % P, h_kv, 0, P, H, D)
        else:
            raise ValueError(prob.layout)
        idx = offs[:, None] + lane[None, :]
        kflat = buf["k"].reshape(-1)
        vflat = buf["v"].reshape(-1)
        K = decode(kflat[idx], prob.kv_format)
        V = decode(vflat[idx], prob.kv_format)
        return K.reshape(n, D), V.reshape(n, D), offs, region
    if prob.kv_format == "i8":
        if prob.layout != "contig":
            raise ValueError("int8 format is contiguous")
        T = int(buf["seq_lens"][b])
        R = prob.residual_len
        G = prob.k_group
        n_q = quantized_count(T, getattr(prob, "residual_policy", "window"), G, R)
        K = np.empty((n, D), dtype=np.float64)
        V = np.empty((n, D), dtype=np.float64)
        offs = np.empty(n, dtype=np.int64)
        quant = positions < n_q
        region[~quant] = 1
        tq = positions[quant]
        ks_off = np.full(n, -1, dtype=np.int64)
        vs_off = np.full(n, -1, dtype=np.int64)
        if tq.size:
            o = nhd_offset(b, tq, h_kv, 0, prob.kv_capacity, H, D)
            offs[quant] = o
            idx = o[:, None] + lane[None, :]
            kc = buf["k"].reshape(-1)[idx].astype(np.float64)
            vc = buf["v"].reshape(-1)[idx].astype(np.float64)
            # K scale row of the token's group, V scale of the token (M8.6 §0x06A)
            n_groups = -(-prob.kv_capacity // G)
            ks_off[quant] = ((b * n_groups + tq // G) * H + h_kv) * D
            vs_off[quant] = (b * prob.kv_capacity + tq) * H + h_kv
            ks = decode_f16(buf["k_scale"].reshape(-1)[ks_off[quant][:, None] + lane[None, :]])  # [n, D]
            vs = decode_f16(buf["v_scale"].reshape(-1)[vs_off[quant]])                            # [n]
            K[quant] = kc * ks
            V[quant] = vc * vs[:, None]
        if scale_offsets is not None:
            scale_offsets["k"], scale_offsets["v"] = ks_off, vs_off
        tr = positions[~quant]
        if tr.size:
            o = nhd_offset(b, tr - n_q, h_kv, 0, R, H, D)
            offs[~quant] = o
            idx = o[:, None] + lane[None, :]
            K[~quant] = decode_bf16(buf["k_resid"].reshape(-1)[idx])
            V[~quant] = decode_bf16(buf["v_resid"].reshape(-1)[idx])
        return K, V, offs, region
    raise ValueError(prob.kv_format)


def attend(prob, buf, heads=None, with_trace: bool = False):
    """Exact decode attention.

    Returns ``(O [B, H_q, D], LSE [B, H_q])`` in fp64, and with ``with_trace``
    also ``{(b, h_kv): dict(positions, offsets, regions, k_scale_offsets,
    v_scale_offsets)}`` of every row read (in position order; the scale
    offsets are those of ``gather_rows``, -1 outside the int8 codes).
    ``heads`` optionally restricts the work to a list of ``(b, h_q)`` rows
    (the other rows are returned as NaN).

    With ``prob.num_queries = C > 1`` (few-query decode / append, M4.5
    §0x08B-§0x08C) q is ``[B, C, H_q, D]``, the results are ``[B, C, H_q, D]``
    and ``[B, C, H_q]``, and query row i of request b sees the keys visible to
    a decode at length ``T_b - C + 1 + i`` (``visibility.query_row_length``):
    bottom-right causal alignment, the C new rows being the last C of the
    cache.  The trace then lists the rows of the last query row (the union)."""
    B, Hq, Hkv, D = prob.batch, prob.num_q_heads, prob.num_kv_heads, prob.head_dim
    C = int(getattr(prob, "num_queries", 1) or 1)
    g = Hq // Hkv
    scale = _scale(prob)
    q = decode(buf["q"], prob.q_dtype).reshape(B, C, Hq, D)
    O = np.full((B, C, Hq, D), np.nan)
    LSE = np.full((B, C, Hq), np.nan)
    trace = {}
    want = None
    if heads is not None:
        want = {}
        for (b, hq) in heads:
            want.setdefault((int(b), int(hq) // g), []).append(int(hq) % g)
    for b in range(B):
        T = int(buf["seq_lens"][b])
        for qi in range(C):
            if prob.mask_kind == "flashmask":
                A = flashmask.visible_columns(query_row_length(T, C, qi), buf["mask_intervals"][b])
            else:
                A = visible_positions(query_row_length(T, C, qi), prob.mask_kind, prob.n_sink,
                                      prob.window)
            last = qi == C - 1
            for h in range(Hkv):
                if want is not None and (b, h) not in want:
                    continue
                rows = range(g) if want is None else sorted(set(want[(b, h)]))
                if A.size == 0:
                    for i in rows:
                        O[b, qi, h * g + i] = 0.0
                        LSE[b, qi, h * g + i] = -math.inf
                    if with_trace and last:
                        none = np.zeros(0, np.int64)
                        trace[(b, h)] = dict(positions=A, offsets=none, regions=np.zeros(0, np.int8),
                                             k_scale_offsets=none, v_scale_offsets=none)
                    continue
                so = {}
                K, V, offs, region = gather_rows(prob, buf, b, h, A, scale_offsets=so)
                if with_trace and last:
                    minus = np.full(A.size, -1, np.int64)
                    trace[(b, h)] = dict(positions=A, offsets=offs, regions=region,
                                         k_scale_offsets=so.get("k", minus),
                                         v_scale_offsets=so.get("v", minus))
                for i in rows:
                    s = (K @ q[b, qi, h * g + i]) * scale
                    m = np.max(s)
                    w = np.exp(s - m)
                    l = np.sum(w)
                    O[b, qi, h * g + i] = (w @ V) / l
                    LSE[b, qi, h * g + i] = m + math.log(l)
    if C == 1:
        O, LSE = O[:, 0], LSE[:, 0]
    if with_trace:
        return O, LSE, trace
    return O, LSE


def split_attend(prob, buf, b: int, h_q: int, bounds, order=None):
    """Flash-Decoding reference for one output row.

    ``bounds`` is a list of half-open intervals ``[start, end)`` over the
    visible positions of request b (indices into the sorted visible list, so
    any disjoint exact cover is legal, M4.5 §0x02E).  Returns the per-split
    states, the merged state and ``(O, LSE)``."""
    g = prob.num_q_heads // prob.num_kv_heads
    h = h_q // g
    scale = _scale(prob)
    q = decode(buf["q"], prob.q_dtype).reshape(prob.batch, prob.num_q_heads, prob.head_dim)[b, h_q]
    T = int(buf["seq_lens"][b])
    A = visible_positions(T, prob.mask_kind, prob.n_sink, prob.window)
    states = []
    for (lo, hi) in bounds:
        pos = A[lo:hi]
        if pos.size == 0:
            states.append(EMPTY(prob.head_dim))
            continue
        K, V, _, _ = gather_rows(prob, buf, b, h, pos)
        states.append(summarize_allowed((K @ q) * scale, V))
    acc = EMPTY(prob.head_dim)
    for i in (order if order is not None else range(len(states))):
        acc = merge_state(acc, states[i])
    return states, acc, finalize(acc)
