"""Pins of the oracle against values the pages print (tests/golden/*.json).

Each fixture file names the page and section it restates."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import fp16_model
from oracle.state import State
from tests.conftest import GOLDEN


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- §0x02G
def test_worked_three_split_trace_bit_exact():
    fx = load("split_state_worked_trace.json")
    states = []
    for i, (sc, vals) in enumerate(zip(fx["scores"], fx["values"])):
        allowed = [s is not None for s in sc]
        sc = [0.0 if s is None else s for s in sc]
        states.append(oracle.summarize_allowed(sc, vals, allowed))
    for st, ref in zip(states, fx["splits"]):
        assert st.valid == ref["valid"]
        if ref["valid"]:
            assert st.m == ref["m"]
            assert st.l == ref["l"]
            assert list(st.u) == ref["u"]
        else:
            assert st.m == -math.inf and st.l == 0 and not st.u.any()
    acc = oracle.EMPTY(2)
    for st in states:
        acc = oracle.merge_state(acc, st)
    assert acc.m == fx["merged"]["m"]
    assert acc.l == fx["merged"]["l"]
    assert list(acc.u) == fx["merged"]["u"]
    O, lse = oracle.finalize(acc)
    assert list(O) == fx["O"]
    assert lse == fx["LSE"]


def test_worked_trace_trees_and_dense_agree():
    fx = load("split_state_worked_trace.json")
    states = []
    flat_s, flat_v = [], []
    for sc, vals in zip(fx["scores"], fx["values"]):
        allowed = [s is not None for s in sc]
        states.append(oracle.summarize_allowed([0.0 if s is None else s for s in sc], vals, allowed))
        for s, v in zip(sc, vals):
            if s is not None:
                flat_s.append(s)
                flat_v.append(v)
    seq = oracle.EMPTY(2)
    for st in states:
        seq = oracle.merge_state(seq, st)
    bal = oracle.merge_state(oracle.merge_state(states[0], states[1]), states[2])
    bal2 = oracle.merge_state(states[0], oracle.merge_state(states[1], states[2]))
    perm = oracle.merge_state(oracle.merge_state(states[2], states[0]), states[1])
    dense = oracle.summarize_allowed(flat_s, flat_v)
    O_ref, _ = oracle.finalize(dense)
    for st in (seq, bal, bal2, perm):
        O, _ = oracle.finalize(st)
        assert np.max(np.abs(O - O_ref)) <= fx["tree_spread_max"]


# ---------------------------------------------------------------- §0x02F
def test_lse_merge_not_average():
    fx = load("lse_not_average.json")
    A = oracle.summarize_allowed(fx["split_A"]["scores"], fx["split_A"]["values"])
    Bs = oracle.summarize_allowed(fx["split_B"]["scores"], fx["split_B"]["values"])
    OA, LA = oracle.finalize(A)
    OB, LB = oracle.finalize(Bs)
    assert OA[0] == fx["O_A"] and OB[0] == fx["O_B"]
    assert (OA[0] + OB[0]) / 2 == fx["naive_average"]
    O, _ = oracle.finalize(oracle.merge_state(A, Bs))
    assert round(O[0], fx["O_digits"]) == fx["O"]
    # the (LSE, O) ABI gives the same row
    _, L2, O2 = oracle.lse_merge((True, LA, OA), (True, LB, OB))
    assert round(O2[0], fx["O_digits"]) == fx["O"]
    assert abs(LA - (10 + math.log(2))) < 1e-15 and abs(LB - math.log(2)) < 1e-15


# ---------------------------------------------------------------- §0x02H
def test_fp16_reduction_order_fixture():
    fx = load("fp16_reduction_order.json")
    s, v = fx["scores"], fx["values"]
    assert fp16_model.sequential(s, v) == fx["sequential"]
    assert fp16_model.balanced(s, v) == fx["balanced"]
    assert fp16_model.sequential(s, v, fx["permuted_order_reading"]) == fx["permuted"]
    exact = oracle.finalize(oracle.summarize_allowed(s, v))[0][0]
    assert exact == fx["exact_output"]


# ---------------------------------------------------------------- §0x03B/§0x03G
def test_balanced_split_bounds():
    fx = load("split_bounds.json")
    for case in fx["balanced"]:
        b = oracle.balanced_bounds(case["T"], case["S"])
        assert [e - s for s, e in b] == case["lengths"]
        assert b[0][0] == 0 and b[-1][1] == case["T"]
        assert all(b[i][1] == b[i + 1][0] for i in range(len(b) - 1))
    cap = fx["capacity"]
    active = 0
    for T in cap["T"]:
        b = oracle.balanced_bounds(T, cap["S"])
        lens = [e - s for s, e in b]
        if T == cap["T"][0]:
            assert lens == cap["first_request_lengths"]
        active += sum(1 for n in lens if n) * cap["H_q"]
    owners = cap["B"] * cap["H_q"] * cap["S_capacity"]
    assert owners == cap["producer_owners"]
    assert active == cap["active_owners"]
    assert owners - active == cap["identity_owners"]
    assert cap["B"] * cap["H_q"] == cap["reducer_owners"]
    mc = fx["main_call"]
    assert mc["B"] * mc["H_q"] * mc["S"] == mc["producer_owners"]
    assert mc["B"] * mc["H_q"] * (mc["S"] - 1) == mc["nonempty_binary_merges"]


# ---------------------------------------------------------------- §0x04
def test_address_translation_fixture():
    fx = load("address_translation.json")
    gq = fx["gqa"]
    assert gq["h_q"] // (gq["H_q"] // gq["H_kv"]) == gq["h_kv"]
    c = fx["contiguous"]
    co = c["coord"]
    o = oracle.nhd_offset(co["c"], co["t"], co["h_kv"], co["x"], c["T_c"], c["H_kv"], c["d_h"])
    assert o == c["nhd_offset"] and o * c["elem_bytes"] == c["nhd_bytes"]
    o = oracle.hnd_offset(co["c"], co["t"], co["h_kv"], co["x"], c["T_c"], c["H_kv"], c["d_h"])
    assert o == c["hnd_offset"] and o * c["elem_bytes"] == c["hnd_bytes"]
    # strides are the differences of unit steps
    T_c, H, D = c["T_c"], c["H_kv"], c["d_h"]
    nhd = [oracle.nhd_offset(1, 0, 0, 0, T_c, H, D), oracle.nhd_offset(0, 1, 0, 0, T_c, H, D),
           oracle.nhd_offset(0, 0, 1, 0, T_c, H, D), oracle.nhd_offset(0, 0, 0, 1, T_c, H, D)]
    assert nhd == c["nhd_strides"]
    hnd = [oracle.hnd_offset(1, 0, 0, 0, T_c, H, D), oracle.hnd_offset(0, 0, 1, 0, T_c, H, D),
           oracle.hnd_offset(0, 1, 0, 0, T_c, H, D), oracle.hnd_offset(0, 0, 0, 1, T_c, H, D)]
    assert hnd == c["hnd_strides"]
    p = fx["paged"]
    segs = oracle.paged_segments(p["block_table"], p["split"][0], p["split"][1], p["P"])
    assert [list(s) for s in segs] == p["segments"]
    a, e, P = p["split"][0], p["split"][1], p["P"]
    assert len(segs) == 1 + (e - 1) // P - a // P
    from oracle.address import page_of
    for page, toks in p["tokens_in_page"].items():
        for t in toks:
            assert page_of(p["block_table"], t, P)[0] == int(page)
    # the last page of T=10 holds two visible rows; rows 2, 3 are tail
    vis = oracle.visible_positions(p["T"])
    last = [t for t in vis if t // P == len(p["block_table"]) - 1]
    assert [t % P for t in last] == [0, 1]
    assert sorted(set(range(P)) - {t % P for t in last}) == p["last_page_invisible_rows"]


# ---------------------------------------------------------------- M5.4 §0x03-§0x05
def test_window_and_sink_sets():
    fx = load("visible_sets.json")
    for case in fx["window"]:
        got = oracle.visible_positions(case["F"], "sink_window", 0, case["W"])
        assert list(got) == case["visible"]
    for case in fx["sink_recent"]:
        got = oracle.visible_positions(case["F"], "sink_window", case["K_s"], case["W"])
        assert list(got) == case["visible"]
        assert oracle.visible_count(case["F"], "sink_window", case["K_s"], case["W"]) == len(case["visible"])
    ff = fx["sink_recent_first_full_F"]
    sizes = {F: len(oracle.visible_positions(F, "sink_window", ff["K_s"], ff["W"])) for F in range(0, 12)}
    assert min(F for F, n in sizes.items() if n == ff["size"]) == ff["F"]
    om = fx["sink_recent_first_middle_omission_F"]
    first_gap = min(F for F in range(1, 12)
                    if list(oracle.visible_positions(F, "sink_window", om["K_s"], om["W"]))
                    != list(range(len(oracle.visible_positions(F, "sink_window", om["K_s"], om["W"])))))
    assert first_gap == om["F"]
    led = fx["read_ledger"]
    win = sum(len(oracle.visible_positions(F, "sink_window", 0, led["W"])) for F in led["frontiers"])
    full = sum(len(oracle.visible_positions(F)) for F in led["frontiers"])
    assert (win, full) == (led["window_instances"], led["full_instances"])
    assert win * led["bytes_per_instance"] == led["window_bytes"]
    assert full * led["bytes_per_instance"] == led["full_bytes"]
    rb = fx["row_bytes"]
    assert rb["d_h"] * (rb["b_K"] + rb["b_V"]) == rb["B_row"]
    assert rb["L"] * rb["H_kv"] * rb["B_row"] == rb["bytes_per_token_all_layers"]


def test_sink_window_cardinality_closed_form_exhaustive():
    for Ks in range(0, 6):
        for W in range(1, 7):
            for F in range(0, 20):
                s = oracle.visible_positions(F, "sink_window", Ks, W)
                assert len(s) == oracle.visible_count(F, "sink_window", Ks, W)
                assert len(set(s.tolist())) == len(s)
                assert all(0 <= t < F for t in s)
                # brute-force predicate
                ref = [t for t in range(F) if t < Ks or t >= F - W]
                assert s.tolist() == ref


def test_window_requires_positive_width():
    with pytest.raises(ValueError):
        oracle.visible_positions(5, "sink_window", 1, 0)


# ---------------------------------------------------------------- §0x03D-§0x03G ledgers
def test_workspace_ledgers():
    fx = load("workspace_ledger.json")
    mc = fx["main_call"]
    N = mc["B"] * mc["H_q"] * mc["S"]
    assert N == mc["N_cfg"]
    assert oracle.workspace_bytes_mlu(1, mc["d_v"]) == mc["mlu_bytes_per_state"]
    assert oracle.workspace_bytes_mlu(N, mc["d_v"]) == mc["mlu_payload"]
    assert oracle.workspace_bytes_lse_o(1, mc["d_v"]) == mc["lse_o_bytes_per_state"]
    assert oracle.workspace_bytes_lse_o(N, mc["d_v"]) == mc["lse_o_payload"]
    out = mc["B"] * mc["H_q"] * mc["d_v"] * 2
    lse = mc["B"] * mc["H_q"] * 4
    assert (out, lse) == (mc["bf16_output_bytes"], mc["f32_lse_bytes"])
    assert 2 * mc["mlu_payload"] + out + lse == mc["reduction_path_mlu"]
    assert 2 * mc["lse_o_payload"] + out + lse == mc["reduction_path_lse_o"]
    gd = fx["gqa_demand"]
    uniq = sum(gd["T"]) * gd["H_kv"] * (gd["d_h"] + gd["d_v"]) * gd["b_cache"]
    dem = sum(gd["T"]) * gd["H_q"] * (gd["d_h"] + gd["d_v"]) * gd["b_cache"]
    assert (uniq, dem) == (gd["unique_kv"], gd["qhead_demand"])
    qd = len(gd["T"]) * gd["H_q"] * gd["d_h"] * 2
    assert qd == gd["q_unique"] and qd * mc["S"] == gd["q_demand_every_split"]
    assert dem + gd["q_demand_every_split"] + mc["reduction_path_mlu"] == gd["two_launch_mlu"]
    assert dem + gd["q_demand_every_split"] + mc["reduction_path_lse_o"] == gd["two_launch_lse_o"]
    hw = fx["head_width"]
    assert oracle.workspace_bytes_mlu(hw["N"], hw["d_v"]) == hw["logical"]
    assert oracle.workspace_bytes_mlu(hw["N"], hw["d_v_padded"]) == hw["capacity"]
    assert hw["capacity"] - hw["logical"] == hw["difference"]


def test_decode_phase_row():
    fx = load("phase_fixture.json")
    for r in fx["rows"]:
        T, C = r["T"], r["C"]
        # visible cells: query row i at absolute position T+i sees [0, T+i+1)
        vis = sum(len(oracle.visible_positions(T + i + 1)) for i in range(C))
        assert vis == r["visible"]
        assert C * (T + C) == r["rect"]
        assert r["rect"] - vis == r["masked"]
        assert T + C == r["post"]
        # the oracle's row rule: the cache holds T + C rows, row i sees a decode
        # of length T_total - C + 1 + i
        rows = [oracle.visible_positions(oracle.query_row_length(T + C, C, i)) for i in range(C)]
        assert sum(len(a) for a in rows) == r["visible"]
    tr = fx["append_row_trace"]
    names = tr["old_cache"] + tr["staged"]
    C = len(tr["staged"])
    for i, row in enumerate(tr["rows"]):
        got = [names[t] for t in oracle.visible_positions(oracle.query_row_length(len(names), C, i))]
        assert got == row["visible"] and row["position"] == len(tr["old_cache"]) + i



def test_ragged_indptr_fixture():
    """M4.5 §0x04C: lengths [10, 7, 5] pack with indptr [0, 10, 17, 22]; request B's
    token 6 is packed row 16 (not cache row 0 of a padded layout)."""
    fx = load("address_translation.json")["ragged"]
    indptr = np.concatenate([[0], np.cumsum(fx["lengths"])])
    assert indptr.tolist() == fx["indptr"]
    q = fx["query"]
    assert oracle.ragged_nhd_offset(indptr, q["request"], q["t"], 0, 0, 1, 1) == q["packed_row"]
    # with heads and channels the packed row keeps the NHD strides
    assert oracle.ragged_nhd_offset(indptr, 1, 6, 1, 2, 2, 4) == (16 * 2 + 1) * 4 + 2


def test_csr_and_dense_tables_name_the_same_page():
    """M4.5 §0x04D: both encodings must give the same physical page."""
    dense = np.array([[7, 3, 9, -1], [2, 5, -1, -1]])
    n = [3, 2]
    indptr = [0, 3, 5]
    indices = [7, 3, 9, 2, 5]
    for r in range(2):
        for j in range(n[r]):
            assert oracle.csr_page(indptr, indices, r, j) == dense[r, j]



def test_ring_slot_is_an_address_not_a_position():
    """M5.4 §0x04: with W = 3, original position 6 lives in slot 6 mod 3 = 0 and
    keeps position 6; sinks keep their own slots."""
    assert int(oracle.ring_slot(6, 0, 3)) == 0
    assert oracle.ring_slot(np.arange(10), 2, 3).tolist() == [0, 1, 2 + 2 % 3, 2 + 0, 2 + 1, 2 + 2, 2, 3, 4, 2]
