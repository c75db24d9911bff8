"""Host-side checks of the C ABI: the library loads, exports every function
the header declares, and the planner validates, admits and sizes calls
(no GPU needed: problems carry an explicit CU count)."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import kv_cache_amd as ka
import synth
from tests.conftest import ROOT


def header_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+char\s*\*|da_status)\s+(\w+)\s*\(", text, flags=re.M)
    return names


def test_library_loads_and_exports_every_declared_symbol():
    L = ka.lib()
    names = header_functions()
    assert set(names) >= {"decode_attn_plan", "decode_attn_run", "decode_attn_combine",
                          "decode_attn_forward", "decode_attn_workspace_init",
                          "decode_attn_schedule", "decode_attn_partition", "decode_attn_append",
                          "decode_attn_flashmask_summarize",
                          "decode_attn_trace_indices", "decode_attn_reason",
                          "decode_attn_status_string"}
    for n in names:
        assert hasattr(L, n), n


def test_struct_sizes_match_header_layout():
    assert ctypes.sizeof(ka.Problem) == 28 * 4
    assert ctypes.sizeof(ka.Plan) == 8 + 112 + 16 + 8 + 16
    assert ctypes.sizeof(ka.Args) == 10 * 8 + 8 + 5 * 8 + 8 + 2 * 4


def P(**kw):
    base = dict(batch=8, num_q_heads=32, num_kv_heads=8, head_dim=128, q_dtype="bf16",
                kv_format="bf16", layout="contig", kv_capacity=4096, max_seq_len=4096)
    base.update(kw)
    return synth.Problem(**base)


def plan(p, cus=256):
    return ka.decode_attn_plan(ka.problem_from(p, num_cus=cus), check=False)


def test_workspace_and_auto_splits_llama_shape():
    st, pl, ws, rs = plan(P())
    assert st == ka.DA_OK and rs == 0
    S = pl.num_splits
    states = 8 * 32 * S * (128 + 2) * 4
    counters = 8 * 8 * 4
    header = (8 + 5) * 4          # partition header [W, L, B, 0, P_0..P_B]
    rup = lambda x: (x + 255) // 256 * 256
    assert ws == rup(states) + rup(counters) + rup(header) == pl.workspace_bytes
    assert S * pl.chunk >= 4096 and (S - 1) * pl.chunk < 4096
    assert pl.chunk == -(-4096 // S)  # equal chunks, no tile rounding: 4 x 1024 rows on 256 CUs
    assert 8 * 8 * S >= 256          # at least one workgroup per CU
    assert abs(pl.problem.softmax_scale - 1 / math.sqrt(128)) < 1e-8


def test_auto_split_regimes():
    # B*H_kv below the CU count: about one workgroup per CU, splits of 256..4096 rows
    st, pl, _, _ = plan(P(batch=1, kv_capacity=131072, max_seq_len=131072))
    assert st == ka.DA_OK and (pl.num_splits, pl.chunk) == (32, 4096)
    st, pl, _, _ = plan(P(batch=16, kv_format="i8", kv_capacity=16384, max_seq_len=16384,
                          mask_kind="sink_window", n_sink=4, window=4096, k_group=128,
                          residual_len=128))
    # weighted chunk: (4100 visible + 128 residual rows counted twice) / 2
    assert st == ka.DA_OK and (pl.num_splits, pl.chunk) == (2, 2114)
    st, pl, _, _ = plan(P(batch=2, max_seq_len=300, kv_capacity=300))
    assert st == ka.DA_OK and (pl.num_splits, pl.chunk) == (2, 256)      # never below 256 rows
    # bf16 chunks of whole 64-row steps where the split count stays: 3000 / 4 = 750 -> 768
    st, pl, _, _ = plan(P(max_seq_len=3000, kv_capacity=3000))
    assert st == ka.DA_OK and (pl.num_splits, pl.chunk) == (4, 768)
    st, pl, _, _ = plan(P(max_seq_len=4100, kv_capacity=4100))
    assert st == ka.DA_OK and (pl.num_splits, pl.chunk) == (4, 1088)
    # ... but not where the split count would drop: 8224 / 32 = 257, and 320-row splits would be 26
    st, pl, _, _ = plan(P(batch=1, max_seq_len=8224, kv_capacity=8224))
    assert st == ka.DA_OK and (pl.num_splits, pl.chunk) == (32, 257)
    # FlashMask splits hold at most 64 tiles of 16 keys
    st, pl, _, _ = plan(P(batch=1, mask_kind="flashmask", max_seq_len=32768, kv_capacity=32768))
    assert st == ka.DA_OK and pl.chunk == 1024 and pl.num_splits == 32
    # B*H_kv filling the CUs: about 3 workgroups per CU, splits of at most 1024 rows
    st, pl, _, _ = plan(P(batch=32, layout="paged", page_size=16, max_pages_per_seq=2048,
                          num_pages=40000, kv_capacity=0, max_seq_len=32768))
    assert st == ka.DA_OK and (pl.num_splits, pl.chunk) == (32, 1024)
    st, pl, _, _ = plan(P(batch=64, max_seq_len=4096, kv_capacity=4096))
    assert st == ka.DA_OK and (pl.num_splits, pl.chunk) == (4, 1024)
    # the same problem on a device with more CUs than B*H_kv: the first regime again
    st, pl, _, _ = plan(P(batch=64, max_seq_len=4096, kv_capacity=4096), cus=1024)
    assert st == ka.DA_OK and (pl.num_splits, pl.chunk) == (2, 2048)


@pytest.mark.parametrize("S", [1, 8, 32, 128])
def test_explicit_split_counts_long_context(S):
    st, pl, ws, _ = plan(P(batch=1, kv_capacity=131072, max_seq_len=131072, num_splits=S))
    assert st == ka.DA_OK
    assert pl.num_splits == S and pl.chunk == 131072 // S


def test_uneven_splits_have_partial_tail():
    st, pl, _, _ = plan(P(batch=1, kv_capacity=131072, max_seq_len=131071, num_splits=128))
    assert st == ka.DA_OK and pl.num_splits == 128
    assert pl.chunk * 127 < 131071 < pl.chunk * 128


def test_flashmask_chunks_stay_tile_aligned():
    # FlashMask classifies 16-key blocks, so its splits start on block boundaries
    st, pl, _, _ = plan(P(mask_kind="flashmask", max_seq_len=4000, kv_capacity=4000, num_splits=12))
    assert st == ka.DA_OK and pl.chunk % 16 == 0 and pl.num_splits * pl.chunk >= 4000
    st, pl, _, _ = plan(P(max_seq_len=4000, kv_capacity=4000, num_splits=12))
    assert st == ka.DA_OK and pl.chunk == 334


def test_sink_window_bounds_visible_rows():
    st, pl, _, _ = plan(P(batch=16, kv_format="i8", kv_capacity=16384, max_seq_len=16384,
                          mask_kind="sink_window", n_sink=4, window=4096, k_group=128,
                          residual_len=128))
    assert st == ka.DA_OK
    assert pl.max_visible == 4100
    assert pl.num_splits * pl.chunk >= 4100


def test_zero_length_plan():
    st, pl, ws, _ = plan(P(batch=1, kv_capacity=1, max_seq_len=0))
    assert st == ka.DA_OK and pl.num_splits == 1


@pytest.mark.parametrize("kw", [
    dict(num_q_heads=30),                               # H_q % H_kv != 0
    dict(num_kv_heads=0),
    dict(batch=-1),
    dict(layout="paged", page_size=0, num_pages=10, max_pages_per_seq=300, kv_capacity=0),
    dict(page_size=16),                                 # page size on a contiguous layout
    dict(mask_kind="sink_window", n_sink=4, window=0),  # W must be > 0
    dict(mask_kind="sink_window", n_sink=-1, window=8),
    dict(num_splits=-1),
    dict(softmax_scale=-1.0),
    dict(softmax_scale=float("nan")),
    dict(kv_capacity=100),                              # capacity below max_seq_len
    dict(layout="paged", page_size=16, num_pages=10, max_pages_per_seq=10, kv_capacity=0),
    dict(kv_format="i8", k_group=0, residual_len=128),
    dict(n_sink=3),                                     # sink count on a causal mask
])
def test_malformed_calls_are_invalid_not_unsupported(kw):
    st, _, _, rs = plan(P(**kw))
    assert st == ka.DA_ERR_INVALID and rs == 0


def test_unsupported_reports_every_failed_predicate():
    p = P(head_dim=96, num_q_heads=48, num_kv_heads=3, q_dtype="f32", num_splits=100000)
    st, _, _, rs = plan(p)
    assert st == ka.DA_ERR_UNSUPPORTED
    want = (1 << 0) | (1 << 2) | (1 << 3) | (1 << 8)    # head dim, group 16, q dtype, splits
    assert rs & want == want
    names = ka.reason_names(rs)
    assert any("head_dim_qk" in n for n in names)


def test_unsupported_int8_paged_and_out_dtype():
    p = P(kv_format="i8", layout="paged", page_size=16, num_pages=4096, max_pages_per_seq=256,
          kv_capacity=0, k_group=100, residual_len=128)
    pr = ka.problem_from(p, num_cus=256)
    pr.out_dtype = 1
    st, _, _, rs = ka.decode_attn_plan(pr, check=False)
    assert st == ka.DA_ERR_UNSUPPORTED
    assert rs & (1 << 6) and rs & (1 << 7) and rs & (1 << 4)


def test_int8_row_stride_bound():
    # 32-bit in-phase row offsets: H_kv * d may not exceed 2^20 bytes per position
    kw = dict(kv_format="i8", batch=1, max_seq_len=256, kv_capacity=256, k_group=128, residual_len=128)
    st, _, _, rs = plan(P(num_q_heads=8192, num_kv_heads=8192, **kw))
    assert st == ka.DA_OK and rs == 0
    st, _, _, rs = plan(P(num_q_heads=8200, num_kv_heads=8200, **kw))
    assert st == ka.DA_ERR_UNSUPPORTED and rs == 1 << 9


def test_plan_mismatch_detected_without_gpu():
    st, pl, ws, _ = plan(P())
    assert st == ka.DA_OK
    pl.num_splits += 1                      # caller edits a frozen field
    args = ka.Args()
    assert ka.decode_attn_run(pl, args, check=False) == ka.DA_ERR_PLAN_MISMATCH
    assert ka.decode_attn_combine(pl, 16, ws, 16, check=False) == ka.DA_ERR_PLAN_MISMATCH
    assert ka.decode_attn_forward(pl, args, 16, check=False) == ka.DA_ERR_PLAN_MISMATCH
    assert ka.decode_attn_workspace_init(pl, 256, ws, check=False) == ka.DA_ERR_PLAN_MISMATCH


def test_run_rejects_null_pointers_and_small_workspace_without_gpu():
    st, pl, ws, _ = plan(P())
    args = ka.Args()
    assert ka.decode_attn_run(pl, args, check=False) == ka.DA_ERR_INVALID
    args = ka.make_args(16, 16, 16, 16, 256, ws - 4)
    assert ka.decode_attn_run(pl, args, check=False) == ka.DA_ERR_WORKSPACE
    args = ka.make_args(8, 16, 16, 16, 256, ws)          # misaligned q
    assert ka.decode_attn_run(pl, args, check=False) == ka.DA_ERR_INVALID
    assert ka.decode_attn_combine(pl, 256, ws - 1, 16, check=False) == ka.DA_ERR_WORKSPACE
    args = ka.make_args(16, 16, 16, 16, 256, ws)
    assert ka.decode_attn_forward(pl, args, None, check=False) == ka.DA_ERR_INVALID
    args = ka.make_args(16, 16, 16, 16, 256, ws - 4)
    assert ka.decode_attn_forward(pl, args, 16, check=False) == ka.DA_ERR_WORKSPACE
    assert ka.decode_attn_workspace_init(pl, 256, ws - 1, check=False) == ka.DA_ERR_WORKSPACE
    assert ka.decode_attn_workspace_init(pl, None, ws, check=False) == ka.DA_ERR_WORKSPACE


def test_static_forward_rejects_before_any_launch_without_gpu():
    """The allocation-free forward refuses, on the host and before touching
    the device, a plan whose workspace exceeds the library's array and a call
    that brings a workspace of its own."""
    st, pl, ws, _ = plan(P(batch=64, num_splits=64))
    assert st == ka.DA_OK and ws > ka.STATIC_WORKSPACE_BYTES
    assert ka.decode_attn_forward_static(pl, ka.Args(), 16, check=False) == ka.DA_ERR_WORKSPACE
    st, pl, ws, _ = plan(P())
    assert ws <= ka.STATIC_WORKSPACE_BYTES
    args = ka.make_args(16, 16, 16, 16, 256, ws)
    assert ka.decode_attn_forward_static(pl, args, 16, check=False) == ka.DA_ERR_INVALID
    assert ka.decode_attn_forward_static(pl, ka.Args(), 16, check=False) == ka.DA_ERR_INVALID
    pl.chunk += 1
    assert ka.decode_attn_forward_static(pl, ka.Args(), 16, check=False) == ka.DA_ERR_PLAN_MISMATCH


def test_reason_and_status_text():
    for i in range(ka.NUM_REASONS):
        assert ka.decode_attn_reason(i)
    assert ka.decode_attn_reason(99) == "unknown reason bit"
    assert ka.decode_attn_status_string(0) == "ok"


def _work_rows(pl, lens):
    """Rows of each work item (b*H_kv + h)*S + s under the plan's chunking."""
    p = pl.problem
    S, H, chunk = pl.num_splits, p.num_kv_heads, pl.chunk
    rows = {}
    for b, T in enumerate(lens):
        n_vis = T if p.mask_kind == 0 else min(T, p.n_sink + p.window)
        for h in range(H):
            for s in range(S):
                rows[(b * H + h) * S + s] = max(0, min(n_vis, (s + 1) * chunk) - s * chunk)
    return rows


@pytest.mark.parametrize("mask", [None, (4, 300)])
def test_schedule_is_a_largest_first_permutation(mask):
    rng = np.random.default_rng(5)
    lens = rng.integers(0, 4096, size=13).tolist() + [0, 4096, 1]
    kw = dict(batch=len(lens), max_seq_len=4096, kv_capacity=4096)
    if mask:
        kw.update(mask_kind="sink_window", n_sink=mask[0], window=mask[1])
    st, pl, ws, _ = plan(P(**kw))
    assert st == ka.DA_OK
    order = ka.decode_attn_schedule(pl, lens)
    n = pl.problem.batch * pl.problem.num_kv_heads * pl.num_splits
    assert sorted(order.tolist()) == list(range(n))
    rows = _work_rows(pl, lens)
    sizes = [rows[i] for i in order.tolist()]
    assert all(a >= b for a, b in zip(sizes, sizes[1:])), "not largest first"
    # the H_kv heads of one (request, split) sit at consecutive positions, so
    # they go to different XCDs
    H, S = pl.problem.num_kv_heads, pl.num_splits
    for i in range(0, n, H):
        it = order[i:i + H]
        b, h, s = it // (S * H), (it // S) % H, it % S
        assert len(set(b.tolist())) == 1 and len(set(s.tolist())) == 1
        assert sorted(h.tolist()) == list(range(H))


def test_schedule_rejects_bad_arguments():
    st, pl, ws, _ = plan(P(batch=2, max_seq_len=100, kv_capacity=100))
    with pytest.raises(ka.DecodeAttnError):
        ka.decode_attn_schedule(pl, [50, 101])
    with pytest.raises(ka.DecodeAttnError):
        ka.decode_attn_schedule(pl, [50, -1])
    pl.num_splits += 1
    with pytest.raises(ka.DecodeAttnError):
        ka.decode_attn_schedule(pl, [50, 50])


def test_append_rejects_unsupported_plans_and_null_buffers_without_gpu():
    st, pl, ws, _ = plan(P(kv_format="i8", k_group=128, residual_len=128, residual_policy="window"))
    assert st == ka.DA_OK
    assert ka.decode_attn_append(pl, *([16] * 9), check=False) == ka.DA_ERR_UNSUPPORTED
    st, pl, ws, _ = plan(P(kv_format="i8", k_group=128, residual_len=128, residual_policy="groups"))
    assert st == ka.DA_OK
    assert ka.decode_attn_append(pl, *([16] * 8), None, check=False) == ka.DA_ERR_INVALID
    pl.chunk += 16
    assert ka.decode_attn_append(pl, *([16] * 9), check=False) == ka.DA_ERR_PLAN_MISMATCH
    # G < R is accepted (a NULL buffer is then the error); G above 256 is not
    st, pl, ws, _ = plan(P(kv_format="i8", k_group=32, residual_len=128, residual_policy="groups"))
    assert st == ka.DA_OK
    assert ka.decode_attn_append(pl, *([16] * 8), None, check=False) == ka.DA_ERR_INVALID
    st, pl, ws, _ = plan(P(kv_format="i8", k_group=512, residual_len=512, residual_policy="groups"))
    assert st == ka.DA_OK
    assert ka.decode_attn_append(pl, *([16] * 9), check=False) == ka.DA_ERR_UNSUPPORTED


def test_groups_policy_plan_checks():
    # closing G rows must leave a residual row: G <= R
    st, _, _, _ = plan(P(kv_format="i8", k_group=128, residual_len=64, residual_policy="groups"))
    assert st == ka.DA_ERR_INVALID
    # capacity must hold G * ceil((max_seq_len - R) / G) quantized rows
    st, _, _, _ = plan(P(kv_format="i8", k_group=128, residual_len=128, residual_policy="groups",
                         max_seq_len=4097, kv_capacity=4000))
    assert st == ka.DA_ERR_INVALID
    st, _, _, _ = plan(P(kv_format="i8", k_group=128, residual_len=128, residual_policy="groups",
                         max_seq_len=4097, kv_capacity=4096))
    assert st == ka.DA_OK


def test_query_rows_plan_checks_and_workspace():
    # C query rows per request: (H_q/H_kv) * C virtual heads per K/V head
    st, pl, ws, rs = plan(P(num_queries=2))
    assert st == ka.DA_OK and pl.problem.num_queries == 2
    S = pl.num_splits
    rup = lambda x: (x + 255) // 256 * 256
    assert ws == rup(8 * 2 * 32 * S * 130 * 4) + rup(8 * 8 * 4) + rup((8 + 5) * 4)
    st, pl, ws, rs = plan(P(num_queries=0))
    assert st == ka.DA_OK and pl.problem.num_queries == 1
    st, _, _, rs = plan(P(num_queries=4))              # 4 * 4 = 16 virtual heads
    assert st == ka.DA_ERR_UNSUPPORTED and rs == 1 << 12
    st, _, _, rs = plan(P(num_queries=2, mask_kind="sink_window", n_sink=4, window=64))
    assert st == ka.DA_ERR_UNSUPPORTED and rs == 1 << 12
    st, _, _, rs = plan(P(num_queries=8, num_q_heads=8, num_kv_heads=8))
    assert st == ka.DA_OK
    assert ka.decode_attn_reason(12)


def test_flashmask_plan_domain():
    st, pl, _, rs = plan(P(mask_kind="flashmask"))
    assert st == ka.DA_OK and pl.chunk <= 1024
    for kw in (dict(kv_format="f32", q_dtype="f32"), dict(head_dim=64), dict(num_queries=2),
               dict(num_splits=2),                        # 4096 / 2 keys per split > 1024
               dict(max_seq_len=131073, kv_capacity=131073, num_splits=256)):   # > DA_FLASHMASK_MAX_SEQ
        st, _, _, rs = plan(P(mask_kind="flashmask", **kw))
        assert st == ka.DA_ERR_UNSUPPORTED and rs & (1 << 11), kw
    st, _, _, _ = plan(P(mask_kind="flashmask", window=4))
    assert st == ka.DA_ERR_INVALID
    st, _, _, _ = plan(P(mask_kind="flashmask", max_seq_len=131072, kv_capacity=131072, num_splits=256))
    assert st == ka.DA_OK


# ---------------------------------------------------------------- balanced partition
def _pieces(part, B, H_unused=None):
    """Expand a partition descriptor into per-item pieces (b, slot, lo, hi)."""
    W, L, Bd = int(part[0]), int(part[1]), int(part[2])
    P = [int(x) for x in part[4:5 + B]]
    first = [int(x) for x in part[5 + B:5 + B + W]]
    items = []
    for i in range(W):
        x, xe, b, got = i * L, min((i + 1) * L, P[B]), first[i], []
        while x < xe:
            if P[b + 1] <= x:
                b += 1
                continue
            got.append((b, i - P[b] // L, x - P[b], min(xe, P[b + 1]) - P[b]))
            x = min(xe, P[b + 1])
            b += 1
        items.append(got)
    return W, L, P, items


@pytest.mark.parametrize("mask", [None, (4, 300)])
@pytest.mark.parametrize("target", [0, 7, 64])
def test_partition_covers_every_visible_ordinal_once(mask, target):
    rng = np.random.default_rng(11)
    lens = rng.integers(0, 4096, size=13).tolist() + [0, 4096, 1, 0]
    kw = dict(batch=len(lens), max_seq_len=4096, kv_capacity=4096)
    if mask:
        kw.update(mask_kind="sink_window", n_sink=mask[0], window=mask[1])
    st, pl, ws, _ = plan(P(**kw))
    assert st == ka.DA_OK
    part, W = ka.decode_attn_partition(pl, lens, items_per_head=target)
    B, S = len(lens), pl.num_splits
    n_vis = [min(t, mask[0] + mask[1]) if mask else t for t in lens]
    W2, L, Pfx, items = _pieces(part, B)
    assert W2 == W and part[2] == B and part[3] == 0 and L % 16 == 0
    assert Pfx == list(np.concatenate([[0], np.cumsum(n_vis)]))
    want = target or (3 * pl.num_cus) // pl.problem.num_kv_heads
    assert W <= want and W == -(-sum(n_vis) // L)
    seen = {b: [] for b in range(B)}
    for i, got in enumerate(items):
        assert 0 < sum(hi - lo for _, _, lo, hi in got) <= L          # equal work, last may be short
        for b, j, lo, hi in got:
            assert 0 <= j < S and 0 <= lo < hi <= n_vis[b]
            seen[b].append((j, lo, hi))
    for b in range(B):
        pieces = sorted(seen[b])
        assert [j for j, _, _ in pieces] == list(range(len(pieces)))   # slots 0, 1, ... in order
        assert sum(hi - lo for _, lo, hi in pieces) == n_vis[b]
        edges = [lo for _, lo, _ in pieces] + [n_vis[b]] if pieces else [0]
        assert edges[0] == 0 and all(pieces[k][2] == edges[k + 1] for k in range(len(pieces)))
        n_pieces = (Pfx[b + 1] - 1) // L - Pfx[b] // L + 1 if n_vis[b] else 0
        assert len(pieces) == n_pieces <= S                              # the combine's count


def test_partition_bounds_pieces_by_the_plan_and_rejects_bad_arguments():
    st, pl, ws, _ = plan(P(batch=3, max_seq_len=4096, kv_capacity=4096, num_splits=4))
    part, W = ka.decode_attn_partition(pl, [4096, 4096, 4096], items_per_head=1000)
    _, L, _, _ = _pieces(part, 3)
    assert L * (pl.num_splits - 1) >= 4096                 # no request has more than S pieces
    part, W = ka.decode_attn_partition(pl, [0, 0, 0])
    assert W == 0 and list(part[4:8]) == [0, 0, 0, 0]
    with pytest.raises(ka.DecodeAttnError):
        ka.decode_attn_partition(pl, [1, 4097, 0])
    st, pl1, ws, _ = plan(P(batch=3, max_seq_len=4096, kv_capacity=4096, num_splits=1))
    assert ka.decode_attn_partition(pl1, [5, 5, 5], check=False)[1] == 0
    L_ = ka.lib()
    buf = np.zeros(4, dtype=np.int32)
    items = ctypes.c_int32(0)
    assert L_.decode_attn_partition(ctypes.byref(pl), np.array([1, 2, 3], dtype=np.int32).ctypes.data, 0,
                                    buf.ctypes.data, buf.size, ctypes.byref(items)) == ka.DA_ERR_INVALID
    assert L_.decode_attn_partition(ctypes.byref(pl1), np.array([1, 2, 3], dtype=np.int32).ctypes.data, 0,
                                    np.zeros(4096, dtype=np.int32).ctypes.data, 4096,
                                    ctypes.byref(items)) == ka.DA_ERR_UNSUPPORTED
    pl.chunk += 16
    with pytest.raises(ka.DecodeAttnError):
        ka.decode_attn_partition(pl, [5, 5, 5])


def test_partition_rejected_where_unsupported_without_gpu():
    # fp32 (and FlashMask) run only on the fixed splits; a partition item
    # count without a descriptor is malformed.  Both fail before any device work.
    st, pl, ws, _ = plan(P(kv_format="f32", q_dtype="f32"))
    assert st == ka.DA_OK
    a = ka.make_args(16, 16, 16, 16, 16, ws, partition=16, partition_items=1)
    assert ka.decode_attn_run(pl, a, check=False) == ka.DA_ERR_UNSUPPORTED


def test_partition_default_item_count_follows_the_kernel():
    # one dispatch round of the partition instance: 3 workgroups per CU for
    # bf16, 2 for int8 (its partition instance's register budget)
    # (the plan's split count caps a request's pieces, L >= n_max / (S - 1), so
    # the plan reserves 12 states per row here)
    lens = [4096] * 8
    for fmt, per_cu in (("bf16", 3), ("i8", 2)):
        kw = dict(batch=8, max_seq_len=4096, kv_capacity=4096, num_splits=12)
        if fmt == "i8":
            kw.update(kv_format="i8", k_group=128, residual_len=128)
        st, pl, ws, _ = plan(P(**kw))
        assert st == ka.DA_OK
        part, W = ka.decode_attn_partition(pl, lens)
        want = per_cu * pl.num_cus // pl.problem.num_kv_heads
        assert W <= want and W >= want - want // 8, (fmt, W, want)
    st, pl, ws, _ = plan(P())
    a = ka.make_args(16, 16, 16, 16, 16, ws, partition_items=3)
    assert ka.decode_attn_run(pl, a, check=False) == ka.DA_ERR_INVALID
    a = ka.make_args(16, 16, 16, 16, 16, ws, partition=16, partition_items=-1)
    assert ka.decode_attn_run(pl, a, check=False) == ka.DA_ERR_INVALID
