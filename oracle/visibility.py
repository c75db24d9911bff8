"""Visible key positions of the decode row (test infrastructure only).

The decode row of request b is its newest position; the caller states the
number of committed key rows visible to it, ``T`` (it includes the row's own
key, M4.5 §0x08B/§0x08D: one-token decode reads every committed row).

* causal: the full-cache set ``{0, ..., T-1}`` (M5.4 §0x03, with frontier F=T;
  M4.5 §0x05E: with S_q = 1 every committed row is visible);
* sink + sliding window: the union of the first ``min(n_sink, T)`` positions
  and the recent interval ``{max(0, T-W), ..., T-1}`` (M5.4 §0x04 and §0x05).
  The union is taken as a set, so early overlap is counted once.

Visibility is a predicate on logical positions (M4.5 §0x05A), never on ring
slots or packed rows.
"""
import numpy as np


def visible_positions(T: int, mask_kind: str = "causal", n_sink: int = 0,
                      window: int = 0) -> np.ndarray:
    T = int(T)
    if T <= 0:
        return np.zeros(0, dtype=np.int64)
    if mask_kind == "causal":
        return np.arange(T, dtype=np.int64)
    if mask_kind == "sink_window":
        if window <= 0:
            raise ValueError("sliding window requires W > 0")
        if n_sink < 0:
            raise ValueError("negative sink count")
        sink = set(range(min(n_sink, T)))
        recent = set(range(max(0, T - window), T))
        return np.array(sorted(sink | recent), dtype=np.int64)
    raise ValueError(mask_kind)


def visible_count(T: int, mask_kind: str = "causal", n_sink: int = 0,
                  window: int = 0) -> int:
    """Closed-form cardinality, M5.4 §0x05: min(K_s,F) + min(W,F) - I(F)."""
    T = int(T)
    if T <= 0:
        return 0
    if mask_kind == "causal":
        return T
    ks = min(n_sink, T)
    overlap = max(0, ks - max(0, T - window))
    return ks + min(window, T) - overlap


def query_row_length(T_total: int, C: int, i: int) -> int:
    """Few-query decode (M4.5 §0x08B): with T committed rows and C new rows,
    new row i sits at absolute position T + i and may read positions
    [0, T + i + 1).  The cache holds T_total = T + C rows (the new rows are
    staged in it), so row i sees what a one-row decode of visible length
    T_total - C + 1 + i sees (negative lengths see nothing)."""
    return max(0, int(T_total) - int(C) + 1 + int(i))
