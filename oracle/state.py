"""Split-state algebra in fp64 (test infrastructure only).

M4.5 §0x02A: the summary of a non-empty allowed set A is
``(valid, m, l, u)`` with ``m = max s``, ``l = sum e^(s-m)``,
``u = sum e^(s-m) v`` (u not divided by l).
M4.5 §0x02B: the binary merge moves both states into the frame of the larger
maximum.  §0x02C: the empty identity ``(False, -inf, 0, 0)``, with the validity
branch taken before any exponential; an all-masked row finalizes to ``O = 0``
and ``LSE = -inf``.  §0x02F: the equivalent (LSE, O) merge.  §0x03B: balanced
per-request split bounds.  §0x03E: workspace bytes per state.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass
class State:
    valid: bool
    m: float
    l: float
    u: np.ndarray


def EMPTY(d: int) -> State:
    return State(False, -math.inf, 0.0, np.zeros(d, dtype=np.float64))


def summarize_allowed(scores, values, allowed=None) -> State:
    """Summary of one split; ``allowed`` is a boolean mask over its rows."""
    scores = np.asarray(scores, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    if values.ndim == 1:
        values = values[:, None]
    if allowed is not None:
        allowed = np.asarray(allowed, dtype=bool)
        scores = scores[allowed]
        values = values[allowed]
    if scores.size == 0:                      # validity branch first
        return EMPTY(values.shape[1])
    m = float(np.max(scores))
    w = np.exp(scores - m)
    return State(True, m, float(np.sum(w)), w @ values)


def merge_state(a: State, b: State) -> State:
    if not a.valid:
        return b
    if not b.valid:
        return a
    m = max(a.m, b.m)
    alpha = math.exp(a.m - m)
    beta = math.exp(b.m - m)
    return State(True, m, alpha * a.l + beta * b.l, alpha * a.u + beta * b.u)


def finalize(s: State):
    """(O, LSE); the all-masked policy gives O = 0 and LSE = -inf."""
    if not s.valid:
        return np.zeros_like(s.u), -math.inf
    return s.u / s.l, s.m + math.log(s.l)


def lse_merge(a, b):
    """Merge two normalized output states ``(valid, LSE, O)`` (M4.5 §0x02F)."""
    va, La, Oa = a
    vb, Lb, Ob = b
    if not va:
        return b
    if not vb:
        return a
    p = max(La, Lb)
    L = p + math.log(math.exp(La - p) + math.exp(Lb - p))
    return (True, L, math.exp(La - L) * np.asarray(Oa) + math.exp(Lb - L) * np.asarray(Ob))


def balanced_bounds(T: int, S: int):
    """Per-request quotient/remainder bounds: split s gets q + [s < r] rows."""
    if S <= 0:
        raise ValueError("split count must be positive")
    q, r = divmod(int(T), int(S))
    out = []
    for s in range(S):
        start = s * q + min(s, r)
        out.append((start, start + q + (1 if s < r else 0)))
    return out


def workspace_bytes_mlu(n_states: int, d_v: int, b_u: int = 4, b_state: int = 4,
                        b_valid: int = 1) -> int:
    """(m,l,u) payload: N * (d_v*b_u + 2*b_state + b_valid)."""
    return n_states * (d_v * b_u + 2 * b_state + b_valid)


def workspace_bytes_lse_o(n_states: int, d_v: int, b_o: int = 2, b_state: int = 4,
                          b_valid: int = 1) -> int:
    """(LSE,O) payload: N * (d_v*b_O + b_state + b_valid)."""
    return n_states * (d_v * b_o + b_state + b_valid)
