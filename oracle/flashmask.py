"""FlashMask column-interval masks for the decode row (test infrastructure only).

M4.5 §0x06A: key column j carries two half-open masked intervals of query
rows, ``U_j = [UTS_j, UTE_j)`` and ``L_j = [LTS_j, LTE_j)``; score (q, j) is
hidden iff ``q`` lies in either.  The decode row of request b sits at absolute
position ``q = T_b - 1`` and reads columns ``j < T_b`` (M4.5 §0x08B), so its
visible set is ``{j < T_b : q not in U_j and q not in L_j}``.

§0x06C: a K/V column block J of width Bc is summarized by the minimum and the
maximum of each of the four vectors over J (eight values, in the order
UTS_min, UTS_max, UTE_min, UTE_max, LTS_min, LTS_max, LTE_min, LTE_max).

§0x06D: for query rows [q0, q1) and one interval family with starts s_j and
ends e_j, every score is hidden when ``q0 >= max s`` and ``q1 <= min e``
(COVERS); some score may be hidden when ``q1 > min s`` and ``q0 < max e``
(OVERLAPS); otherwise none is (DISJOINT).  A tile is SKIP when either family
COVERS, FULL when both are DISJOINT, PARTIAL otherwise.
"""
from __future__ import annotations

import numpy as np

COVERS, OVERLAPS, DISJOINT = "covers", "overlaps", "disjoint"


def masked(q: int, iv) -> bool:
    """Is query row q hidden from the column with intervals iv = (UTS, UTE, LTS, LTE)?"""
    uts, ute, lts, lte = (int(x) for x in iv)
    return (uts <= q < ute) or (lts <= q < lte)


def visible_columns(T: int, intervals_b) -> np.ndarray:
    """Visible key positions of the decode row of a request of length T."""
    T = int(T)
    q = T - 1
    return np.array([j for j in range(T) if not masked(q, intervals_b[j])], dtype=np.int64)


def block_summary(intervals_b, bc: int) -> np.ndarray:
    """[ceil(L/bc), 8] int32 summary of the [L, 4] interval vectors."""
    iv = np.asarray(intervals_b, dtype=np.int64)
    L = iv.shape[0]
    nb = -(-L // bc)
    out = np.empty((nb, 8), dtype=np.int64)
    for J in range(nb):
        blk = iv[J * bc:(J + 1) * bc]
        for v in range(4):
            out[J, 2 * v] = blk[:, v].min()
            out[J, 2 * v + 1] = blk[:, v].max()
    return out.astype(np.int32)


def family_relation(q0: int, q1: int, s_min: int, s_max: int, e_min: int, e_max: int) -> str:
    if q0 >= s_max and q1 <= e_min:
        return COVERS
    if q1 > s_min and q0 < e_max:
        return OVERLAPS
    return DISJOINT


def classify_tile(q0: int, q1: int, summary_row) -> str:
    s = [int(x) for x in summary_row]
    upper = family_relation(q0, q1, s[0], s[1], s[2], s[3])
    lower = family_relation(q0, q1, s[4], s[5], s[6], s[7])
    if COVERS in (upper, lower):
        return "SKIP"
    if upper == DISJOINT and lower == DISJOINT:
        return "FULL"
    return "PARTIAL"
