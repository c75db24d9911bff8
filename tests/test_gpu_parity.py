"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerances: max-abs 1e-5 for fp32 inputs, 2e-3 for bf16 inputs (fp32
accumulation), 1e-2 relative (max|dO| <= 1e-2 max|O_ref|) for int8 K/V against
the decoded-input oracle.  Indices are compared exactly."""
import math

import numpy as np
import pytest

import oracle
import synth
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-3}


@pytest.fixture(autouse=True)
def _name(request):
    H.announce(request.node.nodeid)


# ---------------------------------------------------------------- config 1
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_cfg1_tiny_fp32(seed):
    w = synth.config(1, seed)
    O, L, plan = H.run(w)
    assert plan.num_splits == 4
    Or, Lr = oracle.attend(w.problem, w.buffers)
    H.check_rows(O, L, Or, Lr, TOL["f32"])


# ---------------------------------------------------------------- config 2
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_cfg2_llama_shape_auto_splits(seed):
    w = synth.config(2, seed)
    O, L, plan = H.run(w)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    H.check_rows(O, L, Or, Lr, TOL["bf16"])


def test_cfg2_split_sweep_and_repeatability():
    w = synth.config(2, 0)
    dw = H.DeviceWorkload(w)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    for S in (1, 2, 3, 5, 8, 16, 32, 64):
        O, L, plan = H.run(w, num_splits=S, dw=dw)
        H.check_rows(O, L, Or, Lr, TOL["bf16"])
    O1, L1, _ = H.run(w, num_splits=16, dw=dw)
    O2, L2, _ = H.run(w, num_splits=16, dw=dw)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)     # fixed plan: bitwise repeatable


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D,Hq,Hkv", [(64, 4, 4), (128, 8, 4), (128, 32, 8), (64, 16, 2), (128, 8, 1)])
def test_small_contiguous_ragged(dtype, D, Hq, Hkv):
    lens = [1, 17, 250, 0, 1000, 63]
    w = synth.make_contiguous(3, len(lens), Hq, Hkv, D, lens, dtype=dtype, kv_capacity=1030)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    dw = H.DeviceWorkload(w)
    for S in (0, 1, 7, 16):
        O, L, _ = H.run(w, num_splits=S, dw=dw)
        H.check_rows(O, L, Or, Lr, TOL[dtype])


@pytest.mark.parametrize("C", [1, 2])
def test_first_tile_at_capacity_and_empty_splits(C):
    # capacity equal to the longest request: first tiles reach past the
    # capacity (clamped) and past request ends (poison rows beyond T must not
    # leak), and splits past short requests are empty; single launch and
    # run + combine
    lens = [40, 33, 0, 17, 1]
    w = synth.make_contiguous(31, len(lens), 16, 4, 128, lens, kv_capacity=40, num_queries=C)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    dw = H.DeviceWorkload(w)
    for S in (0, 1, 2, 3):
        O, L, _ = H.run(w, num_splits=S, dw=dw)
        H.check_rows(O, L, Or, Lr, TOL["bf16"])
        O2, L2, _ = H.forward(w, num_splits=S, dw=dw)
        H.check_rows(O2, L2, Or, Lr, TOL["bf16"])


def test_peaky_scores_stress():
    """q scaled by sqrt(d): score std ~ 11, exercising the online rescale."""
    w = synth.make_contiguous(4, 4, 32, 8, 128, [4096, 3000, 17, 2049], q_scale=math.sqrt(128))
    Or, Lr = oracle.attend(w.problem, w.buffers)
    for S in (1, 16):
        O, L, _ = H.run(w, num_splits=S)
        H.check_rows(O, L, Or, Lr, TOL["bf16"])


def test_workspace_states_match_oracle_split_reference():
    """Each written (m, l, u) equals the oracle summary of the same split
    (chunk policy over the visible rows), or the identity when empty."""
    lens = [300, 40, 0]
    w = synth.make_contiguous(5, 3, 8, 2, 128, lens, kv_capacity=300)
    O, L, plan, wsb = H.run(w, num_splits=4, want_ws=True)
    u, m, l = H.split_workspace(wsb, plan)
    S, C = plan.num_splits, plan.chunk
    for b, T in enumerate(lens):
        n = T
        bounds = [(min(s * C, n), min((s + 1) * C, n)) for s in range(S)]
        for hq in range(8):
            states, _, _ = oracle.split_attend(w.problem, w.buffers, b, hq, bounds)
            for s, st in enumerate(states):
                if not st.valid:
                    assert m[b, hq, s] == -np.inf and l[b, hq, s] == 0 and not u[b, hq, s].any()
                else:
                    assert abs(m[b, hq, s] - st.m) <= 2e-5 * max(1, abs(st.m))
                    scale = math.exp(st.m - m[b, hq, s])   # GPU frame differs from the oracle's by rounding of m
                    assert abs(l[b, hq, s] - st.l * scale) <= 1e-4 * st.l
                    assert H.max_abs(u[b, hq, s], st.u * scale) <= 2e-3 * max(1.0, np.abs(st.u).max())


# ---------------------------------------------------------------- config 4
@pytest.fixture(scope="module")
def cfg4():
    w = synth.config(4, 0)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    return w, H.DeviceWorkload(w), Or, Lr


@pytest.mark.parametrize("S", [1, 8, 32, 128, 0])
def test_cfg4_long_context_split_sweep(cfg4, S):
    w, dw, Or, Lr = cfg4
    O, L, plan = H.run(w, num_splits=S, dw=dw)
    if S:
        assert plan.num_splits == S
    H.check_rows(O, L, Or, Lr, TOL["bf16"])


def test_cfg4_uneven_and_empty_variants():
    # T = 131071 (every S > 1 has a partial split), then [131071, 0] in one batch
    w = synth.config(4, 1, T=131071)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    dw = H.DeviceWorkload(w)
    for S in (8, 128, 0):
        O, L, _ = H.run(w, num_splits=S, dw=dw)
        H.check_rows(O, L, Or, Lr, TOL["bf16"])
    w2 = synth.config(4, 1, seq_lens=[131071, 0])
    O2, L2, _ = H.run(w2, num_splits=32)
    Or2, Lr2 = oracle.attend(w2.problem, w2.buffers)
    H.check_rows(O2, L2, Or2, Lr2, TOL["bf16"])
    assert np.all(O2[1] == 0) and np.all(np.isneginf(L2[1]))
    # the non-empty row is unchanged by the empty neighbour (same data, same plan width)
    w3 = synth.make_contiguous(9, 1, 32, 8, 128, [0], kv_capacity=16)
    O3, L3, _ = H.run(w3, num_splits=4)
    assert np.all(O3 == 0) and not np.signbit(O3).any() and np.all(np.isneginf(L3))


# ---------------------------------------------------------------- config 3
def test_paged_small_ragged_with_poison():
    lens = [1, 15, 16, 17, 300, 0, 2000, 33]
    w = synth.make_paged(6, len(lens), 32, 8, 128, lens, page_size=16, max_pages_per_seq=130)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    dw = H.DeviceWorkload(w)
    for S in (0, 1, 5, 64):
        O, L, _ = H.run(w, num_splits=S, dw=dw)
        H.check_rows(O, L, Or, Lr, TOL["bf16"])


@pytest.mark.parametrize("P", [1, 3, 8, 32])
def test_paged_other_page_sizes(P):
    lens = [40, 7, 100]
    w = synth.make_paged(7, 3, 8, 2, 64, lens, page_size=P, max_pages_per_seq=100 // P + 2)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    O, L, _ = H.run(w, num_splits=3)
    H.check_rows(O, L, Or, Lr, TOL["bf16"])


# ---------------------------------------------------------------- masks
MASK_CASES = [
    # (lens, n_sink, window): window >= T, sinks overlapping the window, S > T
    ([5, 40, 300, 1, 0], 4, 16),
    ([100, 33], 0, 200),
    ([64, 65, 200], 70, 10),
    ([16384], 4, 4096),
]


@pytest.mark.parametrize("lens,ns,W", MASK_CASES)
def test_sink_window_contiguous(lens, ns, W):
    w = synth.make_contiguous(8, len(lens), 16, 4, 128, lens, mask_kind="sink_window",
                              n_sink=ns, window=W, kv_capacity=max(lens) + 5)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    dw = H.DeviceWorkload(w)
    for S in (0, 1, 3, 64):
        O, L, _ = H.run(w, num_splits=S, dw=dw)
        H.check_rows(O, L, Or, Lr, TOL["bf16"])


def test_sink_window_paged():
    lens = [1000, 3, 77]
    w = synth.make_paged(9, 3, 8, 8, 64, lens, page_size=16, mask_kind="sink_window", n_sink=2,
                         window=50, max_pages_per_seq=64)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    O, L, _ = H.run(w, num_splits=4)
    H.check_rows(O, L, Or, Lr, TOL["bf16"])


# ---------------------------------------------------------------- int8 (config 5)
# The int8 kernel has two instances for one or few heads per group: grids of
# at most 2 workgroups per CU of the plan run the one with the larger register
# budget (which takes the sinks as an extra tile of the first window phase),
# larger grids the other.  A plan for 1 CU forces the second on any grid.
I8_CUS = [0, 1]


@pytest.mark.parametrize("cus", I8_CUS)
def test_int8_small_with_residual_and_mask(cus):
    w = synth.make_int8(10, 3, 16, 4, 128, [1000, 100, 250], mask_kind="sink_window",
                        n_sink=4, window=300, kv_capacity=1000)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    dw = H.DeviceWorkload(w)
    for S in (0, 1, 4):
        O, L, _ = H.run(w, num_splits=S, dw=dw, num_cus=cus)
        H.check_rows(O, L, Or, Lr, 0.0, rtol=1e-2)
        O, L, _ = H.forward(w, num_splits=S, dw=dw, num_cus=cus)
        H.check_rows(O, L, Or, Lr, 0.0, rtol=1e-2)


def test_int8_causal_small():
    w = synth.make_int8(11, 2, 8, 2, 64, [700, 50], k_group=64, residual_len=32, kv_capacity=700)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    O, L, _ = H.run(w, num_splits=3)
    H.check_rows(O, L, Or, Lr, 0.0, rtol=1e-2)


@pytest.mark.parametrize("cus", I8_CUS)
def test_int8_scale_table_edges(cus):
    # many 64-token groups in one split (several phases of the staged scale
    # table) and a window whose first group is the sinks' last group (the two
    # position runs share a scale row)
    w = synth.make_int8(14, 2, 8, 2, 128, [4000, 1500], k_group=64, residual_len=64,
                        kv_capacity=4000)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    dw = H.DeviceWorkload(w)
    for S in (1, 2, 0):
        O, L, _ = H.run(w, num_splits=S, dw=dw, num_cus=cus)
        H.check_rows(O, L, Or, Lr, 0.0, rtol=1e-2)
    w = synth.make_int8(15, 2, 8, 2, 128, [1000, 700], mask_kind="sink_window", n_sink=100,
                        window=890, k_group=64, residual_len=64, kv_capacity=1000)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    dw = H.DeviceWorkload(w)
    for S in (1, 3, 0):
        O, L, _ = H.run(w, num_splits=S, dw=dw, num_cus=cus)
        H.check_rows(O, L, Or, Lr, 0.0, rtol=1e-2)
    # no sinks (one run), and sinks covering whole requests (T <= n_sink) next
    # to a request whose sink run ends inside a tile
    for n_sink, window in ((0, 333), (517, 200)):
        w = synth.make_int8(16, 3, 8, 2, 128, [1200, 400, 517], mask_kind="sink_window",
                            n_sink=n_sink, window=window, k_group=128, residual_len=128,
                            kv_capacity=1200)
        Or, Lr = oracle.attend(w.problem, w.buffers)
        dw = H.DeviceWorkload(w)
        for S in (1, 2, 0):
            O, L, _ = H.run(w, num_splits=S, dw=dw, num_cus=cus)
            H.check_rows(O, L, Or, Lr, 0.0, rtol=1e-2)


# ---------------------------------------------------------------- exact indices
def _trace_rows(w, S, forward=False, partition=None, num_cus=0):
    """The trace instance of the kernel the timed call runs loads exactly the
    oracle's rows, and computes the same output as the product instance."""
    tr, plan, O, L = H.trace(w, num_splits=S, forward=forward, partition=partition, num_cus=num_cus)
    n = H.check_trace(w, tr)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    tol = 1e-5 if w.problem.kv_format == "f32" else 2e-3
    if w.problem.kv_format == "i8":
        H.check_rows(O, L, Or, Lr, 0.0, rtol=1e-2)
    else:
        H.check_rows(O, L, Or, Lr, tol)
    return n


@pytest.mark.parametrize("forward", [False, True])
def test_trace_indices_contiguous_and_mask(forward):
    _trace_rows(synth.make_contiguous(12, 3, 8, 4, 128, [500, 0, 77], mask_kind="sink_window",
                                      n_sink=3, window=64, kv_capacity=500), 5, forward)
    _trace_rows(synth.make_contiguous(13, 2, 4, 4, 64, [33, 257], dtype="f32", kv_capacity=260), 3,
                forward)
    # causal contiguous NHD: the speculative first tile, including a capacity-bound one
    _trace_rows(synth.make_contiguous(16, 3, 8, 2, 128, [1000, 1, 777], kv_capacity=1000), 4, forward)


@pytest.mark.parametrize("forward", [False, True])
def test_trace_indices_staggered_sweeps(forward):
    # splits of whole 64-row steps start their sweep at staggered steps and
    # wrap (requests 0 and 1); request 2's second split is shorter and keeps the
    # plain order, so the first tile requested before its length arrived (at
    # the staggered start of a full split) is not the one it uses
    lens = [2048, 2048, 1500]
    w = synth.make_contiguous(19, 3, 8, 2, 128, lens, kv_capacity=2048)
    _trace_rows(w, 2, forward)
    w = synth.make_contiguous(20, 2, 16, 4, 128, [4096, 4000], kv_capacity=4096, num_queries=2)
    _trace_rows(w, 4, forward)


def test_trace_indices_paged_cfg3_shape():
    lens = [1, 16, 17, 4099, 0, 250]
    w = synth.make_paged(14, len(lens), 32, 8, 128, lens, page_size=16, max_pages_per_seq=260)
    _trace_rows(w, 8)
    _trace_rows(w, 8, forward=True)
    _trace_rows(w, 8, partition=0)


@pytest.mark.parametrize("cus", I8_CUS)
@pytest.mark.parametrize("forward", [False, True])
def test_trace_indices_int8(forward, cus):
    _trace_rows(synth.make_int8(15, 2, 16, 4, 128, [1000, 60], mask_kind="sink_window", n_sink=4,
                                window=300, kv_capacity=1000), 4, forward, num_cus=cus)
    # sinks split over two splits, and sinks that end inside a tile next to the window
    _trace_rows(synth.make_int8(18, 3, 8, 2, 128, [1000, 700, 30], mask_kind="sink_window", n_sink=20,
                                window=500, kv_capacity=1000), 0, forward, num_cus=cus)
    # long splits: several scale-staging phases per split, causal over codes and residual
    _trace_rows(synth.make_int8(17, 2, 32, 8, 128, [7000, 3000], kv_capacity=7000), 1, forward,
                num_cus=cus)