"""Seeded synthetic decode-attention workloads.

This module only *produces inputs*: a problem description (the decode
coordinate of "M4.5 - Decode Attention Kernels, Mask Programs, and Backend
Boundaries", §0x00B/§0x07A) and the raw stored bytes of q, the K/V cache and
its metadata.  It contains none of the attention arithmetic.  Both the CPU
oracle and the GPU path consume exactly the arrays built here, so they see
identical bytes.

Storage conventions (the library's ABI, restated for the generators):

* bf16 tensors are ``uint16`` arrays holding the bit patterns, produced from
  float32 draws by round-to-nearest-even on the bits;
* fp16 tensors are ``numpy.float16``; fp32 tensors are ``float32``;
* q is ``[B, H_q, D]`` (the single decode row squeezed);
* contiguous K/V is token-major NHD ``[B, T_cap, H_kv, D]``;
* paged K/V is a page pool ``[N_pages, P, H_kv, D]`` addressed through a dense
  ``block_table [B, max_pages_per_seq]`` (int32);
* the int8 format stores K codes ``[B, T_cap, H_kv, D]`` with one fp16 scale per
  (batch, K/V head, 128-token group, channel) in ``k_scale [B, ceil(T_cap/G),
  H_kv, D]``, V codes ``[B, T_cap, H_kv, D]`` with one fp16 scale per (batch,
  token, K/V head) in ``v_scale [B, T_cap, H_kv]``, and the newest
  ``min(T_b, R)`` tokens of request b as bf16 rows in ``k_resid/v_resid
  [B, R, H_kv, D]`` (residual row ``t - n_q`` holds token t, with
  ``n_q = T_b - min(T_b, R)``).

The int8 writer below is the cache *writer* (the producer of the stored
format, "M8.6 - Live-Data Quantization: Activations and KV Cache", §0x02A
quantizer rule applied along the axes of §0x06/§0x06A with the residual of
§0x06B).  It is input production, not part of the decode path; the oracle
package carries its own independent writer and the CPU tests require the two
to agree byte for byte.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Problem", "Workload", "rng", "bf16_bits", "draw_bf16", "make_contiguous",
    "make_paged", "make_int8", "config", "CONFIG_NAMES",
]


@dataclasses.dataclass
class Problem:
    """Static decode coordinate (one call).  Field names follow the C ABI."""
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    q_dtype: str = "bf16"          # "f32" | "bf16"
    kv_format: str = "bf16"        # "f32" | "bf16" | "i8"
    layout: str = "contig"         # "contig" | "paged"
    kv_capacity: int = 0           # contiguous token capacity T_cap
    page_size: int = 0             # paged only
    max_pages_per_seq: int = 0
    num_pages: int = 0
    max_seq_len: int = 0           # bound on seq_lens (plan-time)
    mask_kind: str = "causal"      # "causal" | "sink_window"
    n_sink: int = 0
    window: int = 0
    softmax_scale: float = 0.0     # 0 -> 1/sqrt(head_dim)
    num_splits: int = 0            # 0 -> auto
    k_group: int = 0               # int8 only: tokens per K scale group
    residual_len: int = 0          # int8 only: bf16 residual rows
    residual_policy: str = "window"  # int8 only: "window" | "groups" (which tokens are bf16)
    num_queries: int = 1           # C query rows per request (q is [B, C, H_q, D] when C > 1)
    page_table: str = "dense"      # paged: "dense" | "csr"
    cache_rows: int = 0            # contiguous: cache rows B_c (0: B); ragged: packed rows
    num_page_entries: int = 0      # CSR page list length

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


@dataclasses.dataclass
class Workload:
    problem: Problem
    buffers: dict          # name -> numpy array (stored bytes)
    name: str = ""
    note: str = ""


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def bf16_bits(x) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (NaN kept quiet)."""
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = np.uint16(0x7FC0)
    return rounded


def draw_bf16(g: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return bf16_bits(x)


def _draw(g, shape, dtype):
    if dtype == "f32":
        return g.standard_normal(size=shape, dtype=np.float32)
    if dtype == "bf16":
        return draw_bf16(g, shape)
    raise ValueError(dtype)


BF16_POISON = np.array([0x7FC0, 0x7F80, 0xFF80, 0x476A, 0xC76A], dtype=np.uint16)
# quiet NaN, +Inf, -Inf, +59904, -59904 (bf16 bit patterns)


def _poison_like(g, shape, dtype):
    if dtype == "bf16":
        return g.choice(BF16_POISON, size=shape)
    if dtype == "f32":
        return g.choice(np.array([np.nan, np.inf, -np.inf, 6e4, -6e4], np.float32), size=shape)
    if dtype == "i8":
        return g.integers(-128, 128, size=shape, dtype=np.int8)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# contiguous NHD cache
# --------------------------------------------------------------------------
def make_contiguous(seed: int, B: int, H_q: int, H_kv: int, D: int, seq_lens,
                    dtype: str = "bf16", kv_capacity: int | None = None,
                    mask_kind: str = "causal", n_sink: int = 0, window: int = 0,
                    num_splits: int = 0, q_scale: float = 1.0,
                    poison_tail: bool = True, num_queries: int = 1) -> Workload:
    """q, K, V ~ N(0,1) (q optionally multiplied by ``q_scale`` before rounding).

    Token slots at or beyond ``seq_lens[b]`` (allocated, never visible) are
    filled with NaN/Inf/huge values so that a read of them would show.
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int32).reshape(B)
    T_cap = int(kv_capacity if kv_capacity is not None else max(1, int(seq_lens.max(initial=0))))
    g = rng(seed)
    qshape = (B, H_q, D) if num_queries == 1 else (B, num_queries, H_q, D)
    qf = g.standard_normal(size=qshape, dtype=np.float32) * np.float32(q_scale)
    q = qf if dtype == "f32" else bf16_bits(qf)
    k = _draw(g, (B, T_cap, H_kv, D), dtype)
    v = _draw(g, (B, T_cap, H_kv, D), dtype)
    if poison_tail:
        for b in range(B):
            T = int(seq_lens[b])
            if T < T_cap:
                k[b, T:] = _poison_like(g, k[b, T:].shape, dtype)
                v[b, T:] = _poison_like(g, v[b, T:].shape, dtype)
    prob = Problem(batch=B, num_q_heads=H_q, num_kv_heads=H_kv, head_dim=D,
                   q_dtype=dtype, kv_format=dtype, layout="contig",
                   kv_capacity=T_cap, max_seq_len=int(seq_lens.max(initial=0)),
                   mask_kind=mask_kind, n_sink=n_sink, window=window,
                   num_splits=num_splits, num_queries=num_queries)
    return Workload(prob, dict(q=q, k=k, v=v, seq_lens=seq_lens))


# --------------------------------------------------------------------------
# paged NHD cache with a dense block table
# --------------------------------------------------------------------------
def make_paged(seed: int, B: int, H_q: int, H_kv: int, D: int, seq_lens,
               page_size: int = 16, dtype: str = "bf16",
               max_pages_per_seq: int | None = None, spare_frac: float = 0.10,
               mask_kind: str = "causal", n_sink: int = 0, window: int = 0,
               num_splits: int = 0, num_queries: int = 1) -> Workload:
    """Paged pool.  Every visible logical page maps to a seeded random
    permutation of the pool; everything that is allocated but not visible holds
    garbage:

    * rows ``T_b mod P .. P-1`` of each request's last page: NaN/Inf/±59904;
    * block-table slots ``>= ceil(T_b/P)``: out-of-pool ids (-1, N_pages+7,
      INT32_MAX) and in-pool ids of other requests' pages;
    * spare pool pages (``spare_frac`` beyond the pages in use): NaN/Inf.
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int32).reshape(B)
    P = int(page_size)
    g = rng(seed)
    pages_needed = [(int(T) + P - 1) // P for T in seq_lens]
    used = int(sum(pages_needed))
    spare = int(math.ceil(used * spare_frac)) if used else 1
    N_pages = max(1, used + spare)
    maxp = int(max_pages_per_seq if max_pages_per_seq is not None
               else max(1, max(pages_needed, default=1)))
    qshape = (B, H_q, D) if num_queries == 1 else (B, num_queries, H_q, D)
    qf = g.standard_normal(size=qshape, dtype=np.float32)
    q = qf if dtype == "f32" else bf16_bits(qf)
    perm = g.permutation(N_pages).astype(np.int32)
    table = np.empty((B, maxp), dtype=np.int32)
    garbage_ids = np.array([-1, N_pages + 7, np.iinfo(np.int32).max], dtype=np.int64)
    k = np.empty((N_pages, P, H_kv, D), dtype=np.float32 if dtype == "f32" else np.uint16)
    v = np.empty_like(k)
    # spare pages first get poison; used pages are overwritten below
    cursor = 0
    for b in range(B):
        n = pages_needed[b]
        phys = perm[cursor:cursor + n]
        cursor += n
        table[b, :n] = phys
        tail = maxp - n
        if tail > 0:
            other = g.integers(0, N_pages, size=tail)
            pick = g.integers(0, 2, size=tail).astype(bool)
            junk = np.where(pick, other, g.choice(garbage_ids, size=tail))
            table[b, n:] = junk.astype(np.int64).clip(np.iinfo(np.int32).min,
                                                       np.iinfo(np.int32).max).astype(np.int32)
    for pidx in perm[cursor:]:
        k[pidx] = _poison_like(g, k[pidx].shape, dtype)
        v[pidx] = _poison_like(g, v[pidx].shape, dtype)
    # fill used pages in pool order (draw order is fixed by the seed)
    used_pages = perm[:cursor]
    chunk = 4096
    for start in range(0, len(used_pages), chunk):
        ids = used_pages[start:start + chunk]
        k[ids] = _draw(g, (len(ids), P, H_kv, D), dtype)
        v[ids] = _draw(g, (len(ids), P, H_kv, D), dtype)
    for b in range(B):
        T = int(seq_lens[b])
        if T % P and pages_needed[b]:
            last = table[b, pages_needed[b] - 1]
            r0 = T % P
            k[last, r0:] = _poison_like(g, k[last, r0:].shape, dtype)
            v[last, r0:] = _poison_like(g, v[last, r0:].shape, dtype)
    prob = Problem(batch=B, num_q_heads=H_q, num_kv_heads=H_kv, head_dim=D,
                   q_dtype=dtype, kv_format=dtype, layout="paged",
                   page_size=P, max_pages_per_seq=maxp, num_pages=N_pages,
                   max_seq_len=int(seq_lens.max(initial=0)), mask_kind=mask_kind,
                   n_sink=n_sink, window=window, num_splits=num_splits, num_queries=num_queries)
    return Workload(prob, dict(q=q, k=k, v=v, block_table=table, seq_lens=seq_lens))


# --------------------------------------------------------------------------
# int8 K/V with fp16 scales and a bf16 residual window (cache writer)
# --------------------------------------------------------------------------
QMAX = 127


# Ideal scales at or above the midpoint between the largest finite fp16 value
# (65504) and the next step (65536) round to infinity; below the midpoint
# between the largest subnormal (2^-14 - 2^-24) and the smallest normal
# (2^-14) they round to a subnormal.  Both are refused.
_F16_INF_FROM = 65520.0
_F16_NORMAL_FROM = 2.0 ** -14 - 2.0 ** -25


def _store_scale_f16(amax: np.ndarray) -> np.ndarray:
    """fp16 scale per element of amax (>= 0): amax/127 committed to fp16,
    and 1 where amax is 0."""
    amax = np.asarray(amax, dtype=np.float64)
    ideal = np.ones_like(amax)
    nz = amax != 0
    ideal[nz] = amax[nz] / QMAX
    if np.any(ideal >= _F16_INF_FROM) or np.any(ideal < _F16_NORMAL_FROM):
        raise ValueError("stored fp16 scale is non-finite or subnormal")
    return ideal.astype(np.float16)


def _codes(x: np.ndarray, s_eff: np.ndarray) -> np.ndarray:
    c = np.clip(np.rint(x / s_eff), -QMAX, QMAX)
    return c.astype(np.int8)


def quantized_tokens(T: int, k_group: int, residual_len: int, policy: str) -> int:
    """Tokens stored as int8 at length T: "window" keeps the newest
    min(T, R) as bf16; "groups" closes whole groups of k_group tokens as soon
    as more than R tokens are unclosed."""
    if policy == "window":
        return T - min(T, residual_len)
    closed = 0
    while T - closed > residual_len:
        closed += k_group
    return closed


def write_int8_cache(k_f32: np.ndarray, v_f32: np.ndarray, seq_lens, k_group: int,
                     residual_len: int, T_cap: int, g: np.random.Generator,
                     policy: str = "window"):
    """Quantize per request: tokens ``[0, n_q)`` to int8 codes, the rest to bf16.

    K: one scale per (group of ``k_group`` quantized tokens, channel), taken over
    the tokens of the group that are quantized (a partial last group uses only
    its own rows).  V: one scale per token over its channels.  Under the
    "groups" policy every token was appended as a bf16 row, so the values are
    rounded to bf16 before quantization.
    Slots that hold no visible data are filled with garbage (codes) or NaN
    (scales, residual rows).
    """
    if policy == "groups":
        k_f32 = (bf16_bits(k_f32).astype(np.uint32) << 16).view(np.float32)
        v_f32 = (bf16_bits(v_f32).astype(np.uint32) << 16).view(np.float32)
    B, _, H_kv, D = k_f32.shape
    R, G = residual_len, k_group
    n_groups = (T_cap + G - 1) // G
    kc = g.integers(-128, 128, size=(B, T_cap, H_kv, D), dtype=np.int8)
    vc = g.integers(-128, 128, size=(B, T_cap, H_kv, D), dtype=np.int8)
    ks = np.full((B, n_groups, H_kv, D), np.nan, dtype=np.float16)
    vs = np.full((B, T_cap, H_kv), np.nan, dtype=np.float16)
    kr = np.full((B, max(R, 1), H_kv, D), 0x7FC0, dtype=np.uint16)
    vr = np.full((B, max(R, 1), H_kv, D), 0x7FC0, dtype=np.uint16)
    for b in range(B):
        T = int(seq_lens[b])
        n_q = quantized_tokens(T, G, R, policy)
        n_res = T - n_q
        if n_q > 0:
            kq = k_f32[b, :n_q].astype(np.float64)      # [n_q, H, D]
            for j in range((n_q + G - 1) // G):
                blk = kq[j * G:min((j + 1) * G, n_q)]    # [<=G, H, D]
                s = _store_scale_f16(np.abs(blk).max(axis=0))        # [H, D]
                ks[b, j] = s
                kc[b, j * G:j * G + blk.shape[0]] = _codes(blk, s.astype(np.float64)[None])
            vq = v_f32[b, :n_q].astype(np.float64)      # [n_q, H, D]
            s = _store_scale_f16(np.abs(vq).max(axis=2))              # [n_q, H]
            vs[b, :n_q] = s
            vc[b, :n_q] = _codes(vq, s.astype(np.float64)[..., None])
        if n_res > 0:
            kr[b, :n_res] = bf16_bits(k_f32[b, n_q:T])
            vr[b, :n_res] = bf16_bits(v_f32[b, n_q:T])
    return dict(k=kc, v=vc, k_scale=ks, v_scale=vs, k_resid=kr, v_resid=vr)


def make_int8(seed: int, B: int, H_q: int, H_kv: int, D: int, seq_lens,
              k_group: int = 128, residual_len: int = 128,
              kv_capacity: int | None = None, mask_kind: str = "causal",
              n_sink: int = 0, window: int = 0, num_splits: int = 0,
              outlier_channels: int = 3, outlier_mult: float = 20.0,
              values=None, residual_policy: str = "window", num_queries: int = 1) -> Workload:
    """int8 K (per channel per group) / int8 V (per token) / bf16 residual.

    ``outlier_channels`` channels per (batch, K/V head), drawn once from the
    seed independently for K and for V, are multiplied by ``outlier_mult``
    after the N(0,1) draw and before quantization.  ``values`` may supply the
    float32 K and V tensors directly (used for exact-quantization cases).
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int32).reshape(B)
    T_cap = int(kv_capacity if kv_capacity is not None else max(1, int(seq_lens.max(initial=0))))
    g = rng(seed)
    qshape = (B, H_q, D) if num_queries == 1 else (B, num_queries, H_q, D)
    q = bf16_bits(g.standard_normal(size=qshape, dtype=np.float32))
    if values is None:
        kf = g.standard_normal(size=(B, T_cap, H_kv, D), dtype=np.float32)
        vf = g.standard_normal(size=(B, T_cap, H_kv, D), dtype=np.float32)
        for arr in (kf, vf):
            for b in range(B):
                for h in range(H_kv):
                    ch = g.choice(D, size=outlier_channels, replace=False)
                    arr[b, :, h, ch] *= np.float32(outlier_mult)
    else:
        kf, vf = (np.asarray(a, dtype=np.float32) for a in values)
    bufs = write_int8_cache(kf, vf, seq_lens, k_group, residual_len, T_cap, g, residual_policy)
    bufs.update(q=q, seq_lens=seq_lens)
    prob = Problem(batch=B, num_q_heads=H_q, num_kv_heads=H_kv, head_dim=D,
                   q_dtype="bf16", kv_format="i8", layout="contig",
                   kv_capacity=T_cap, max_seq_len=int(seq_lens.max(initial=0)),
                   mask_kind=mask_kind, n_sink=n_sink, window=window,
                   num_splits=num_splits, k_group=k_group, residual_len=residual_len,
                   residual_policy=residual_policy, num_queries=num_queries)
    w = Workload(prob, bufs)
    w.float_kv = (kf, vf)
    return w


# --------------------------------------------------------------------------
# the five decode workloads at their full sizes
# --------------------------------------------------------------------------
CONFIG_NAMES = {
    1: "tiny: B=1 H_q=H_kv=4 d=64 T=256 fp32 contiguous causal S=4",
    2: "llama3-8b-layer: B=8 H_q=32 H_kv=8 d=128 T=4096 bf16 contiguous causal",
    3: "paged-ragged: B=32 H_q=32 H_kv=8 d=128 bf16 P=16 T~U[1,32768]",
    4: "long-context: B=1 H_q=32 H_kv=8 d=128 T=131072 bf16 contiguous causal",
    5: "int8-sink-window: B=16 H_q=32 H_kv=8 d=128 T=16384 int8 K/V + bf16 residual 128, 4 sinks + window 4096",
}


def ragged_lengths(seed: int, B: int, lo: int = 1, hi: int = 32768) -> np.ndarray:
    return rng(seed + 1_000_003).integers(lo, hi + 1, size=B).astype(np.int32)


def config(i: int, seed: int = 0, num_splits: int = 0, **over) -> Workload:
    """Full-size workload i (1..5)."""
    if i == 1:
        w = make_contiguous(seed, 1, 4, 4, 64, [256], dtype="f32",
                            num_splits=num_splits or 4)
    elif i == 2:
        w = make_contiguous(seed, 8, 32, 8, 128, [4096] * 8, num_splits=num_splits)
    elif i == 3:
        w = make_paged(seed, 32, 32, 8, 128, ragged_lengths(seed, 32),
                       page_size=16, max_pages_per_seq=2048, num_splits=num_splits)
    elif i == 4:
        T = over.pop("T", 131072)
        lens = over.pop("seq_lens", [T])
        w = make_contiguous(seed, len(lens), 32, 8, 128, lens,
                            kv_capacity=max(max(lens), 1), num_splits=num_splits)
    elif i == 5:
        w = make_int8(seed, 16, 32, 8, 128, [16384] * 16, mask_kind="sink_window",
                      n_sink=4, window=4096, num_splits=num_splits)
    else:
        raise ValueError(i)
    w.name = f"cfg{i}"
    w.note = CONFIG_NAMES[i]
    return w


def append_rows(seed: int, B: int, H_kv: int, D: int, outlier_channels: int = 3,
                outlier_mult: float = 20.0):
    """One new token per request for an append: bf16 bit patterns of K and V,
    ``[B, H_kv, D]`` each, N(0,1) with the outlier channels scaled."""
    g = rng(seed + 7919)
    kf = g.standard_normal(size=(B, H_kv, D), dtype=np.float32)
    vf = g.standard_normal(size=(B, H_kv, D), dtype=np.float32)
    for arr in (kf, vf):
        for b in range(B):
            for h in range(H_kv):
                ch = g.choice(D, size=outlier_channels, replace=False)
                arr[b, h, ch] *= np.float32(outlier_mult)
    return bf16_bits(kf), bf16_bits(vf)


# --------------------------------------------------------------------------
# the same logical cache in the other layouts of the ABI
# --------------------------------------------------------------------------
def relayout(w: Workload, layout: str, page_table: str = "dense", cache_rows: int = 0,
             seed: int = 0) -> Workload:
    """Copy of ``w`` (contiguous NHD or paged NHD, not int8) whose K/V bytes are
    stored in another layout; the logical data (q, lengths, every visible K/V
    row) is unchanged.

    * from contiguous NHD with a sink + window mask: ``"ring"`` (only the
      visible rows, sinks in slots 0 .. n_sink-1 and the window in ring slots
      n_sink + t mod W; the other slots poisoned);
    * from contiguous NHD: ``"contig"`` with ``cache_rows`` > B (request b in a
      seeded random cache row, the other rows NaN, plus ``cache_batch_idx``),
      ``"contig_hnd"`` (``[B_c, H_kv, T_cap, D]``, same cache rows) or
      ``"ragged"`` (rows packed as ``[sum T_b, H_kv, D]`` with ``indptr``);
    * from paged NHD: ``"paged"`` or ``"paged_hnd"`` (pool ``[N_pages, H_kv, P, D]``),
      with ``page_table="csr"`` turning the dense table into ``indptr`` plus the
      list of pages (followed by a few garbage entries).
    """
    p = dataclasses.replace(w.problem)
    buf = dict(w.buffers)
    g = rng(seed + 4242)
    lens = [int(t) for t in buf["seq_lens"]]
    if w.problem.layout == "contig" and layout == "ring":
        if p.mask_kind != "sink_window":
            raise ValueError("the ring layout holds a sink + window cache")
        ns, W = p.n_sink, p.window
        k, v = buf["k"], buf["v"]
        kr = _poison_like(g, (p.batch, ns + W) + k.shape[2:], _dt_name(k))
        vr = _poison_like(g, (p.batch, ns + W) + v.shape[2:], _dt_name(v))
        for b, T in enumerate(lens):
            keep = [t for t in range(T) if t < ns or t >= T - W]
            for t in keep:
                slot = t if t < ns else ns + t % W
                kr[b, slot] = k[b, t]
                vr[b, slot] = v[b, t]
        buf.update(k=kr, v=vr)
        p.layout, p.kv_capacity = "ring", ns + W
        return Workload(p, buf)
    if w.problem.layout == "contig" and layout in ("contig", "contig_hnd", "ragged"):
        k, v = buf["k"], buf["v"]
        B = p.batch
        if layout == "ragged":
            indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
            rows = max(1, int(indptr[-1]))
            kp = _poison_like(g, (rows,) + k.shape[2:], _dt_name(k))
            vp = _poison_like(g, (rows,) + v.shape[2:], _dt_name(v))
            for b, T in enumerate(lens):
                kp[indptr[b]:indptr[b] + T] = k[b, :T]
                vp[indptr[b]:indptr[b] + T] = v[b, :T]
            buf.update(k=kp, v=vp, indptr=indptr)
            p.layout, p.cache_rows, p.kv_capacity = "ragged", rows, 0
            return Workload(p, buf)
        if cache_rows:
            if cache_rows < B:
                raise ValueError("cache_rows < B")
            perm = g.permutation(cache_rows)[:B].astype(np.int32)
            kc = _poison_like(g, (cache_rows,) + k.shape[1:], _dt_name(k))
            vc = _poison_like(g, (cache_rows,) + v.shape[1:], _dt_name(v))
            kc[perm] = k
            vc[perm] = v
            k, v = kc, vc
            buf["cache_batch_idx"] = perm
            p.cache_rows = cache_rows
        if layout == "contig_hnd":
            k = np.ascontiguousarray(k.transpose(0, 2, 1, 3))
            v = np.ascontiguousarray(v.transpose(0, 2, 1, 3))
        buf.update(k=k, v=v)
        p.layout = layout
        return Workload(p, buf)
    if w.problem.layout == "paged" and layout in ("paged", "paged_hnd"):
        if layout == "paged_hnd":
            buf["k"] = np.ascontiguousarray(buf["k"].transpose(0, 2, 1, 3))
            buf["v"] = np.ascontiguousarray(buf["v"].transpose(0, 2, 1, 3))
        if page_table == "csr":
            P = p.page_size
            table = buf["block_table"]
            n = [(T + P - 1) // P for T in lens]
            indptr = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
            garbage = np.array([-1, p.num_pages + 7, np.iinfo(np.int32).max], dtype=np.int32)
            entries = np.concatenate([table[b, :n[b]] for b in range(p.batch)] + [garbage])
            buf["block_table"] = entries.astype(np.int32)
            buf["indptr"] = indptr
            p.page_table, p.num_page_entries, p.max_pages_per_seq = "csr", int(entries.size), 0
        p.layout = layout
        return Workload(p, buf)
    raise ValueError(f"cannot make {layout} from {w.problem.layout}")


def _dt_name(a: np.ndarray) -> str:
    return "f32" if a.dtype == np.float32 else "bf16"


# --------------------------------------------------------------------------
# FlashMask column intervals for the decode row
# --------------------------------------------------------------------------
FLASHMASK_OPEN = 1 << 30     # an end that no query row reaches


def flashmask_intervals(seed: int, seq_lens, L: int, block: int = 16) -> np.ndarray:
    """int32 [B, L, 4] (UTS, UTE, LTS, LTE) per key column, seeded, chosen so
    that the decode row q = T_b - 1 of each request meets whole blocks that it
    cannot see (documents closed before q: LT = [doc_end, open)), whole blocks
    it sees (empty intervals) and blocks with scattered hidden columns (UT
    intervals around q), in runs of a few blocks.  Columns >= T_b get random
    intervals."""
    g = rng(seed + 5151)
    B = len(seq_lens)
    iv = np.zeros((B, L, 4), dtype=np.int64)
    iv[:, :, 2] = FLASHMASK_OPEN      # LT empty: [open, open)
    iv[:, :, 3] = FLASHMASK_OPEN
    for b, T in enumerate(int(t) for t in seq_lens):
        q = T - 1
        j = 0
        while j < L:
            run = int(g.integers(1, 5)) * block
            kind = int(g.integers(0, 3))
            hi = min(L, j + run)
            if kind == 0 and q >= 0:          # a closed document: hidden from q on
                iv[b, j:hi, 2] = int(g.integers(max(0, q - 3), q + 1))
                iv[b, j:hi, 3] = FLASHMASK_OPEN
            elif kind == 2 and q >= 0:        # scattered hidden columns around q
                hide = g.random(hi - j) < 0.4
                lo_ = g.integers(max(0, q - 5), q + 1, size=hi - j)
                up_ = g.integers(q + 1, q + 6, size=hi - j)
                iv[b, j:hi, 0] = np.where(hide, lo_, 0)
                iv[b, j:hi, 1] = np.where(hide, up_, 0)
            j = hi
        if T < L:                              # never read: random garbage intervals
            iv[b, T:, :2] = np.sort(g.integers(0, L, size=(L - T, 2)), axis=1)
    return iv.astype(np.int32)
