"""Pins of the oracle by closed forms, invariances and brute force.

These tie ``oracle.attend`` to what the mathematics fixes, independently of the
oracle's own code paths: a pure-Python ``math.fsum`` softmax, the dense
softmax restricted and renormalized by the retained mass (M5.4 §0x02K),
partition invariance (M4.5 §0x02E), layout invariance (M4.5 §0x04, the
translators must recover the same payload), and closed forms of softmax.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from oracle.numerics import decode


def brute_force(prob, buf):
    """Independent pure-Python reference: explicit loops, math.fsum, direct
    multi-axis indexing of the stored arrays (no flat offsets)."""
    B, Hq, Hkv, D = prob.batch, prob.num_q_heads, prob.num_kv_heads, prob.head_dim
    g = Hq // Hkv
    scale = 1.0 / math.sqrt(D)
    q = decode(buf["q"], prob.q_dtype)
    O = np.zeros((B, Hq, D))
    L = np.zeros((B, Hq))
    for b in range(B):
        T = int(buf["seq_lens"][b])
        for hq in range(Hq):
            h = hq // g
            keys = []
            for t in range(T):
                if prob.mask_kind == "sink_window" and not (t < prob.n_sink or t >= T - prob.window):
                    continue
                if prob.layout == "contig":
                    krow = decode(buf["k"][b, t, h], prob.kv_format)
                    vrow = decode(buf["v"][b, t, h], prob.kv_format)
                else:
                    page = int(buf["block_table"][b, t // prob.page_size])
                    krow = decode(buf["k"][page, t % prob.page_size, h], prob.kv_format)
                    vrow = decode(buf["v"][page, t % prob.page_size, h], prob.kv_format)
                s = math.fsum(float(q[b, hq, x]) * float(krow[x]) for x in range(D)) * scale
                keys.append((s, vrow))
            if not keys:
                O[b, hq] = 0.0
                L[b, hq] = -math.inf
                continue
            m = max(s for s, _ in keys)
            w = [math.exp(s - m) for s, _ in keys]
            l = math.fsum(w)
            for x in range(D):
                O[b, hq, x] = math.fsum(wi * float(v[x]) for wi, (_, v) in zip(w, keys)) / l
            L[b, hq] = m + math.log(l)
    return O, L


TINY = [
    dict(kind="contig", B=2, Hq=4, Hkv=2, D=8, lens=[13, 40], dtype="f32"),
    dict(kind="contig", B=2, Hq=4, Hkv=1, D=4, lens=[0, 7], dtype="bf16"),
    dict(kind="paged", B=2, Hq=2, Hkv=2, D=8, lens=[9, 33], dtype="bf16", P=4),
    dict(kind="contig", B=2, Hq=4, Hkv=2, D=8, lens=[3, 29], dtype="bf16",
         mask=("sink_window", 2, 5)),
    dict(kind="paged", B=1, Hq=4, Hkv=4, D=4, lens=[17], dtype="f32", P=3,
         mask=("sink_window", 3, 4)),
]


def build(c, seed=0):
    mk, ns, W = c.get("mask", ("causal", 0, 0))
    if c["kind"] == "contig":
        return synth.make_contiguous(seed, c["B"], c["Hq"], c["Hkv"], c["D"], c["lens"],
                                     dtype=c["dtype"], kv_capacity=max(c["lens"]) + 3,
                                     mask_kind=mk, n_sink=ns, window=W)
    return synth.make_paged(seed, c["B"], c["Hq"], c["Hkv"], c["D"], c["lens"],
                            page_size=c["P"], dtype=c["dtype"], mask_kind=mk,
                            n_sink=ns, window=W, max_pages_per_seq=max(c["lens"]) // c["P"] + 3)


@pytest.mark.parametrize("c", TINY)
@pytest.mark.parametrize("seed", [0, 1])
def test_brute_force_tiny(c, seed):
    w = build(c, seed)
    O, L = oracle.attend(w.problem, w.buffers)
    Ob, Lb = brute_force(w.problem, w.buffers)
    assert np.max(np.abs(O - Ob)) <= 1e-13
    fin = np.isfinite(Lb)
    assert np.array_equal(fin, np.isfinite(L))
    assert np.max(np.abs(L[fin] - Lb[fin]), initial=0) <= 1e-13
    assert np.all(L[~fin] == -math.inf) and np.all(O[~fin] == 0)


def test_masked_softmax_equals_renormalized_dense():
    """M5.4 §0x02K: selected attention = dense softmax restricted to A and
    divided by the retained mass."""
    w = synth.make_contiguous(3, 1, 2, 1, 16, [50], dtype="f32", mask_kind="sink_window",
                              n_sink=3, window=11)
    p, bf = w.problem, w.buffers
    O, _ = oracle.attend(p, bf)
    q = bf["q"].astype(np.float64)
    K = bf["k"][0, :50, 0].astype(np.float64)
    V = bf["v"][0, :50, 0].astype(np.float64)
    A = oracle.visible_positions(50, "sink_window", 3, 11)
    for hq in range(2):
        s = K @ q[0, hq] / 4.0
        pd = np.exp(s - s.max())
        pd /= pd.sum()
        M = pd[A].sum()
        ref = (pd[A] / M) @ V[A]
        assert np.max(np.abs(ref - O[0, hq])) < 1e-14


def _close_forms_case(kind):
    D, T = 16, 37
    g = synth.rng(11)
    q = g.standard_normal((1, 2, D)).astype(np.float32)
    k = g.standard_normal((1, T, 1, D)).astype(np.float32)
    v = g.standard_normal((1, T, 1, D)).astype(np.float32)
    if kind == "identical_keys":
        k[0, :, 0] = k[0, 0, 0]
    elif kind == "equal_values":
        v[0, :, 0] = v[0, 5, 0]
    elif kind == "zero_query":
        q[:] = 0
    elif kind == "dominant":
        k[0, :, 0] = 0
        k[0, 17, 0] = q[0, 0] * 64.0          # s = 64 |q|^2 / 4, others 0
    prob = synth.Problem(batch=1, num_q_heads=2, num_kv_heads=1, head_dim=D, q_dtype="f32",
                         kv_format="f32", kv_capacity=T, max_seq_len=T)
    return prob, dict(q=q, k=k, v=v, seq_lens=np.array([T], np.int32))


def test_closed_forms():
    p, b = _close_forms_case("identical_keys")
    O, L = oracle.attend(p, b)
    V = b["v"][0, :, 0].astype(np.float64)
    s = float(b["q"][0, 0].astype(np.float64) @ b["k"][0, 0, 0].astype(np.float64)) / 4.0
    assert np.max(np.abs(O[0, 0] - V.mean(0))) < 1e-14
    assert abs(L[0, 0] - (s + math.log(37))) < 1e-13
    p, b = _close_forms_case("equal_values")
    O, _ = oracle.attend(p, b)
    assert np.max(np.abs(O[0] - b["v"][0, 5, 0].astype(np.float64))) < 1e-14
    p, b = _close_forms_case("zero_query")
    O, L = oracle.attend(p, b)
    assert np.max(np.abs(O[0] - b["v"][0, :, 0].astype(np.float64).mean(0))) < 1e-14
    assert np.allclose(L[0], math.log(37), atol=1e-14)
    p, b = _close_forms_case("dominant")
    O, _ = oracle.attend(p, b)
    assert np.max(np.abs(O[0, 0] - b["v"][0, 17, 0])) < 1e-9


def test_single_visible_row_is_exact():
    w = synth.make_contiguous(5, 1, 2, 2, 8, [1], dtype="bf16", kv_capacity=4)
    O, _ = oracle.attend(w.problem, w.buffers)
    for h in range(2):
        assert np.array_equal(O[0, h], decode(w.buffers["v"][0, 0, h], "bf16"))


def test_masked_rows_do_not_matter():
    """Rows outside the visible set may hold NaN or 1e30 (M4.5 §0x02G keeps
    masked values deliberately large)."""
    w = synth.make_contiguous(6, 1, 2, 1, 8, [30], dtype="f32", kv_capacity=30,
                              mask_kind="sink_window", n_sink=2, window=9)
    O1, L1 = oracle.attend(w.problem, w.buffers)
    hidden = [t for t in range(30) if t not in set(oracle.visible_positions(30, "sink_window", 2, 9))]
    w.buffers["k"][0, hidden] = np.nan
    w.buffers["v"][0, hidden] = 1e30
    O2, L2 = oracle.attend(w.problem, w.buffers)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_empty_and_all_masked_rows():
    w = synth.make_contiguous(7, 3, 4, 2, 8, [0, 5, 0], dtype="bf16", kv_capacity=8)
    O, L = oracle.attend(w.problem, w.buffers)
    for b in (0, 2):
        assert np.all(O[b] == 0) and not np.signbit(O[b]).any()
        assert np.all(L[b] == -math.inf)
    assert np.all(np.isfinite(L[1]))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_partition_invariance(seed):
    """M4.5 §0x02E: any disjoint exact cover, any merge order."""
    w = synth.make_contiguous(seed, 2, 4, 2, 16, [97, 64], dtype="bf16", kv_capacity=100)
    O, L = oracle.attend(w.problem, w.buffers)
    g = synth.rng(seed + 50)
    for b in range(2):
        T = int(w.buffers["seq_lens"][b])
        for hq in range(4):
            for S in range(1, 17):
                _, _, (o, lse) = oracle.split_attend(w.problem, w.buffers, b, hq,
                                                     oracle.balanced_bounds(T, S))
                assert np.max(np.abs(o - O[b, hq])) <= 1e-12 and abs(lse - L[b, hq]) <= 1e-12
            cuts = sorted(g.choice(np.arange(0, T + 1), size=6, replace=True).tolist())
            bounds = list(zip([0] + cuts, cuts + [T]))      # may contain empty splits
            order = g.permutation(len(bounds))
            _, _, (o, lse) = oracle.split_attend(w.problem, w.buffers, b, hq, bounds, order)
            assert np.max(np.abs(o - O[b, hq])) <= 1e-12 and abs(lse - L[b, hq]) <= 1e-12


def test_paged_equals_contiguous_and_pool_permutation():
    """The same logical rows stored contiguously or in a permuted page pool
    give identical oracle output (M4.5 §0x04: translation recovers the same
    payload)."""
    B, Hq, Hkv, D, P = 3, 4, 2, 8, 4
    lens = [10, 1, 17]
    wc = synth.make_contiguous(9, B, Hq, Hkv, D, lens, dtype="bf16", kv_capacity=20)
    maxp = 6
    for perm_seed in (0, 1):
        gg = synth.rng(100 + perm_seed)
        N = B * maxp + 2
        perm = gg.permutation(N)
        k = np.full((N, P, Hkv, D), 0x7FC0, np.uint16)
        v = np.full((N, P, Hkv, D), 0x7FC0, np.uint16)
        table = np.full((B, maxp), -1, np.int32)
        cur = 0
        for b, T in enumerate(lens):
            for j in range((T + P - 1) // P):
                table[b, j] = perm[cur]
                cur += 1
                rows = range(j * P, min(T, (j + 1) * P))
                for t in rows:
                    k[table[b, j], t % P] = wc.buffers["k"][b, t]
                    v[table[b, j], t % P] = wc.buffers["v"][b, t]
        prob = synth.Problem(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, layout="paged",
                             page_size=P, max_pages_per_seq=maxp, num_pages=N, max_seq_len=17)
        bufs = dict(q=wc.buffers["q"], k=k, v=v, block_table=table, seq_lens=wc.buffers["seq_lens"])
        Op, Lp = oracle.attend(prob, bufs)
        Oc, Lc = oracle.attend(wc.problem, wc.buffers)
        assert np.array_equal(Op, Oc) and np.array_equal(Lp, Lc)


def test_head_permutation_equivariance():
    """Permuting K/V heads together with their query groups permutes O."""
    w = synth.make_contiguous(12, 1, 8, 4, 8, [21], dtype="f32")
    O, _ = oracle.attend(w.problem, w.buffers)
    perm = np.array([2, 0, 3, 1])
    qperm = np.concatenate([[2 * p, 2 * p + 1] for p in perm])
    b2 = dict(w.buffers)
    b2["k"] = w.buffers["k"][:, :, perm]
    b2["v"] = w.buffers["v"][:, :, perm]
    b2["q"] = w.buffers["q"][:, qperm]
    O2, _ = oracle.attend(w.problem, b2)
    assert np.array_equal(O2, O[:, qperm])


def test_trace_lists_each_visible_row_once():
    w = synth.make_paged(4, 2, 4, 2, 8, [19, 7], page_size=4, mask_kind="sink_window",
                         n_sink=2, window=6, max_pages_per_seq=8)
    _, _, tr = oracle.attend(w.problem, w.buffers, with_trace=True)
    for (b, h), t in tr.items():
        pos, offs = t["positions"], t["offsets"]
        T = int(w.buffers["seq_lens"][b])
        assert list(pos) == [t for t in range(T) if t < 2 or t >= T - 6]
        assert len(set(offs.tolist())) == len(offs)
        for t, o in zip(pos, offs):
            page = w.buffers["block_table"][b, t // 4]
            assert o == ((page * 4 + t % 4) * 2 + h) * 8


def test_trace_int8_rows_and_scales_are_the_stored_elements():
    """Every traced int8 row, K scale row and V scale points at the element
    the format stores for (b, t, h) (NumPy's own multi-index flattening), and
    residual rows at row t - n_q of the residual buffer."""
    lens = [300, 130, 5]
    w = synth.make_int8(9, 3, 4, 2, 16, lens, k_group=32, residual_len=16, kv_capacity=320,
                        mask_kind="sink_window", n_sink=3, window=100)
    _, _, tr = oracle.attend(w.problem, w.buffers, with_trace=True)
    kc, ks, vs, kr = (w.buffers[x] for x in ("k", "k_scale", "v_scale", "k_resid"))
    for (b, h), t in tr.items():
        n_q = lens[b] - min(lens[b], 16)
        for pos, off, reg, ko, vo in zip(t["positions"], t["offsets"], t["regions"],
                                         t["k_scale_offsets"], t["v_scale_offsets"]):
            if pos < n_q:
                assert reg == 0
                assert off == np.ravel_multi_index((b, pos, h, 0), kc.shape)
                assert ko == np.ravel_multi_index((b, pos // 32, h, 0), ks.shape)
                assert vo == np.ravel_multi_index((b, pos, h), vs.shape)
            else:
                assert reg == 1 and ko == -1 and vo == -1
                assert off == np.ravel_multi_index((b, pos - n_q, h, 0), kr.shape)


@pytest.mark.parametrize("C,T_list", [(3, [8, 3, 0]), (2, [5, 1]), (4, [6, 9])])
def test_few_query_rows_brute_force(C, T_list):
    """C > 1 against a pure-Python loop over the C x T score rectangle with the
    bottom-right causal predicate j <= T - C + i (M4.5 §0x08B)."""
    B, Hq, Hkv, D = len(T_list), 4, 2, 8
    w = synth.make_contiguous(11, B, Hq, Hkv, D, T_list, dtype="f32", kv_capacity=12, num_queries=C)
    O, L = oracle.attend(w.problem, w.buffers)
    q = w.buffers["q"].astype(np.float64)
    k = w.buffers["k"].astype(np.float64)
    v = w.buffers["v"].astype(np.float64)
    for b, T in enumerate(T_list):
        for i in range(C):
            for hq in range(Hq):
                h = hq // (Hq // Hkv)
                keys = [j for j in range(T) if j <= T - C + i]
                if not keys:
                    assert np.all(O[b, i, hq] == 0) and L[b, i, hq] == -math.inf
                    continue
                s = [math.fsum(q[b, i, hq, x] * k[b, j, h, x] for x in range(D)) / math.sqrt(D) for j in keys]
                m = max(s)
                e = [math.exp(t - m) for t in s]
                den = math.fsum(e)
                for x in range(D):
                    ref = math.fsum(e[n] * v[b, keys[n], h, x] for n in range(len(keys))) / den
                    assert abs(O[b, i, hq, x] - ref) < 1e-12
                assert abs(L[b, i, hq] - (m + math.log(den))) < 1e-12



@pytest.mark.parametrize("layout,kw", [("contig_hnd", {}), ("contig", {"cache_rows": 7}),
                                       ("contig_hnd", {"cache_rows": 6}), ("ragged", {})])
def test_contiguous_relayouts_give_identical_results(layout, kw):
    w = synth.make_contiguous(13, 4, 8, 2, 16, [9, 0, 33, 20], dtype="f32", kv_capacity=40)
    O, L = oracle.attend(w.problem, w.buffers)
    w2 = synth.relayout(w, layout, **kw)
    O2, L2 = oracle.attend(w2.problem, w2.buffers)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)


@pytest.mark.parametrize("layout,table", [("paged_hnd", "dense"), ("paged", "csr"), ("paged_hnd", "csr")])
def test_paged_relayouts_give_identical_results(layout, table):
    w = synth.make_paged(14, 3, 4, 2, 16, [37, 5, 64], page_size=8, dtype="f32")
    O, L = oracle.attend(w.problem, w.buffers)
    w2 = synth.relayout(w, layout, page_table=table)
    O2, L2 = oracle.attend(w2.problem, w2.buffers)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)



@pytest.mark.parametrize("lens", [[9, 0, 33, 20], [2, 5, 7, 40]])
def test_ring_layout_gives_identical_results(lens):
    w = synth.make_contiguous(15, 4, 8, 2, 16, lens, dtype="f32", kv_capacity=40,
                              mask_kind="sink_window", n_sink=2, window=5)
    O, L = oracle.attend(w.problem, w.buffers)
    w2 = synth.relayout(w, "ring")
    O2, L2 = oracle.attend(w2.problem, w2.buffers)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)
