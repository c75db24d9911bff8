"""Read-side address translation (test infrastructure only).

Element offsets of one K or V element, from M4.5 §0x04B (contiguous NHD/HND
strides), §0x04C (packed ragged rows through indptr) and §0x04D (paged NHD/HND
through a dense block table or a CSR page list); page segments of a logical
interval from §0x04E.  K and V have separate bases.
"""


def nhd_offset(c: int, t: int, h_kv: int, x: int, T_c: int, H_kv: int, D: int) -> int:
    """Token-major cache ``[B_c, T_c, H_kv, D]``: ((c*T_c + t)*H_kv + h)*D + x."""
    return ((c * T_c + t) * H_kv + h_kv) * D + x


def hnd_offset(c: int, t: int, h_kv: int, x: int, T_c: int, H_kv: int, D: int) -> int:
    """Head-major cache ``[B_c, H_kv, T_c, D]``: ((c*H_kv + h)*T_c + t)*D + x."""
    return ((c * H_kv + h_kv) * T_c + t) * D + x


def paged_nhd_offset(page: int, r: int, h_kv: int, x: int, P: int, H_kv: int, D: int) -> int:
    """Page pool ``[N_pages, P, H_kv, D]``: ((page*P + r)*H_kv + h)*D + x."""
    return ((page * P + r) * H_kv + h_kv) * D + x


def paged_hnd_offset(page: int, r: int, h_kv: int, x: int, P: int, H_kv: int, D: int) -> int:
    """Page pool ``[N_pages, H_kv, P, D]``: ((page*H_kv + h)*P + r)*D + x."""
    return ((page * H_kv + h_kv) * P + r) * D + x


def ragged_nhd_offset(indptr, r: int, t: int, h_kv: int, x: int, H_kv: int, D: int) -> int:
    """Packed ragged cache ``[sum_r T_r, H_kv, D]``: request r's token t is
    packed row indptr[r] + t; offset ((indptr[r] + t)*H_kv + h)*D + x."""
    return ((int(indptr[r]) + t) * H_kv + h_kv) * D + x


def csr_page(kv_page_indptr, kv_page_indices, r: int, j: int) -> int:
    """Physical page of logical block j of request r from a CSR page list."""
    return int(kv_page_indices[int(kv_page_indptr[r]) + j])


def ring_slot(t, n_sink: int, window: int):
    """Fixed-capacity sink + window cache (M5.4 §0x04, "logical position is
    not ring slot"): sink position t < n_sink keeps slot t; any other position
    lives in ring slot n_sink + (t mod W).  The slot is an address only."""
    import numpy as _np
    t = _np.asarray(t)
    return _np.where(t < n_sink, t, n_sink + t % window)


def page_of(block_table_row, t: int, P: int):
    """Logical block j = t // P, row r = t mod P, physical page = table[j]."""
    j, r = divmod(int(t), int(P))
    return int(block_table_row[j]), r


def paged_segments(block_table_row, start: int, end: int, P: int):
    """Split [start, end) into per-page segments (page, first_row, rows)."""
    out = []
    pos = int(start)
    while pos < end:
        j, r = divmod(pos, P)
        seg_end = min(end, (j + 1) * P)
        out.append((int(block_table_row[j]), r, seg_end - pos))
        pos = seg_end
    return out
