"""Pins of the streaming int8 append (M8.6 §0x06B, the synchronized-tail
teaching state) and of the "groups" residual policy built on it."""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from oracle.quant import (kivi_append, kivi_empty_state, kivi_state_from_parts, kivi_state_parts,
                          quantized_count, write_int8_cache_oracle)
from tests.conftest import GOLDEN


def _golden():
    with open(os.path.join(GOLDEN, "kivi_closure_counts.json")) as f:
        return json.load(f)


def _rows(seed, T, H, D):
    g = synth.rng(seed)
    k = g.standard_normal((T, H, D), dtype=np.float32)
    v = g.standard_normal((T, H, D), dtype=np.float32)
    k[:, :, 3] *= 20.0
    return k, v


@pytest.mark.parametrize("case", _golden()["cases"])
def test_closure_counts_follow_the_pages_rule(case):
    G, R, T = case["group"], case["residual"], case["appends"]
    assert quantized_count(T, "groups", G, R) == case["closed_rows"]
    assert T - quantized_count(T, "groups", G, R) == case["residual_rows"]
    # the page's rule stepped on counts alone: a row joins the residual, and
    # while the residual holds more than R rows its oldest G leave it
    closed = open_rows = 0
    for _ in range(T):
        open_rows += 1
        while open_rows > R:
            closed += G
            open_rows -= G
    assert (closed, open_rows) == (case["closed_rows"], case["residual_rows"])
    if T <= 400:
        # the same counts from the append model itself, one token at a time
        st = kivi_empty_state(1, 4)
        row = np.full((1, 4), 0x3F80, np.uint16)            # bf16 1.0
        for _ in range(T):
            st = kivi_append(st, row, row, G, R)
        assert len(st["v_rows"]) == case["closed_rows"]
        assert len(st["k_resid"]) == case["residual_rows"]


@pytest.mark.parametrize("G,R,T", [(128, 128, 300), (32, 128, 300), (16, 40, 130)])
def test_sequential_appends_equal_the_static_writer(G, R, T):
    H, D = 2, 16
    k, v = _rows(3, T, H, D)
    kb, vb = synth.bf16_bits(k), synth.bf16_bits(v)
    st = kivi_empty_state(H, D)
    closed_before = []
    for t in range(T):
        st = kivi_append(st, kb[t], vb[t], G, R)
        closed_before.append([(c.copy(), s.copy()) for c, s in st["k_groups"]])
    parts = kivi_state_parts(st)
    ref = write_int8_cache_oracle(k[None], v[None], [T], G, R, policy="groups")[0]
    assert parts["n_q"] == ref["n_q"] == quantized_count(T, "groups", G, R)
    for key in ("k_codes", "v_codes", "k_resid_bits", "v_resid_bits"):
        assert np.array_equal(parts[key], ref[key]), key
    for key in ("k_scale", "v_scale"):
        assert np.array_equal(parts[key].view(np.uint16), ref[key].view(np.uint16)), key
    # a closed group never changes afterwards (stable per-channel qparams)
    for t, groups in enumerate(closed_before):
        for j, (c, s) in enumerate(groups):
            assert np.array_equal(c, st["k_groups"][j][0])
            assert np.array_equal(s.view(np.uint16), st["k_groups"][j][1].view(np.uint16))


def test_input_writer_matches_oracle_writer_under_groups_policy():
    lens = [0, 1, 128, 129, 300, 257]
    w = synth.make_int8(4, len(lens), 4, 2, 32, lens, kv_capacity=320, residual_policy="groups")
    kf, vf = w.float_kv
    ref = write_int8_cache_oracle(kf, vf, lens, 128, 128, policy="groups")
    for b, T in enumerate(lens):
        r = ref[b]
        n_q = r["n_q"]
        assert n_q == quantized_count(T, "groups", 128, 128)
        assert np.array_equal(w.buffers["k"][b, :n_q], r["k_codes"])
        assert np.array_equal(w.buffers["v"][b, :n_q], r["v_codes"])
        ng = n_q // 128
        assert np.array_equal(w.buffers["k_scale"][b, :ng].view(np.uint16), r["k_scale"].view(np.uint16))
        assert np.array_equal(w.buffers["v_scale"][b, :n_q].view(np.uint16), r["v_scale"].view(np.uint16))
        assert np.array_equal(w.buffers["k_resid"][b, :T - n_q], r["k_resid_bits"])
        assert np.array_equal(w.buffers["v_resid"][b, :T - n_q], r["v_resid_bits"])


def test_state_round_trip_through_stored_parts():
    H, D = 2, 8
    k, v = _rows(6, 200, H, D)
    st = kivi_empty_state(H, D)
    for t in range(200):
        st = kivi_append(st, synth.bf16_bits(k[t]), synth.bf16_bits(v[t]), 64, 64)
    st2 = kivi_state_from_parts(kivi_state_parts(st), 64)
    row = synth.bf16_bits(k[0])
    a = kivi_state_parts(kivi_append(st, row, row, 64, 64))
    b = kivi_state_parts(kivi_append(st2, row, row, 64, 64))
    for key in a:
        assert np.array_equal(np.asarray(a[key]), np.asarray(b[key])), key


def test_failed_closure_leaves_the_state_unchanged():
    st = kivi_empty_state(1, 4)
    tiny = np.full((1, 4), 0x0001, np.uint16)      # bf16 9.2e-41: scale underflows fp16
    for _ in range(4):
        st = kivi_append(st, tiny, tiny, 4, 4)
    with pytest.raises(ValueError):
        kivi_append(st, tiny, tiny, 4, 4)
    assert len(st["k_resid"]) == 4 and not st["k_groups"]


def test_groups_policy_attention_equals_decoded_reference():
    lens = [300, 129, 128, 5]
    w = synth.make_int8(8, len(lens), 8, 2, 32, lens, kv_capacity=320, residual_policy="groups",
                        mask_kind="sink_window", n_sink=2, window=150)
    O, L = oracle.attend(w.problem, w.buffers)
    # decode the stored bytes by hand and run the plain definition
    p = w.problem
    for b, T in enumerate(lens):
        n_q = quantized_count(T, "groups", 128, 128)
        vis = oracle.visible_positions(T, "sink_window", 2, 150)
        for hq in range(p.num_q_heads):
            h = hq // (p.num_q_heads // p.num_kv_heads)
            K, V = [], []
            for t in vis:
                if t < n_q:
                    ks = w.buffers["k_scale"][b, t // 128, h].astype(np.float64)
                    vs = float(w.buffers["v_scale"][b, t, h])
                    K.append(w.buffers["k"][b, t, h].astype(np.float64) * ks)
                    V.append(w.buffers["v"][b, t, h].astype(np.float64) * vs)
                else:
                    K.append(oracle.decode_bf16(w.buffers["k_resid"][b, t - n_q, h]))
                    V.append(oracle.decode_bf16(w.buffers["v_resid"][b, t - n_q, h]))
            q = oracle.decode_bf16(w.buffers["q"][b, hq])
            s = np.array(K) @ q / np.sqrt(32)
            e = np.exp(s - s.max())
            assert np.allclose(O[b, hq], e @ np.array(V) / e.sum(), rtol=0, atol=1e-12)
            assert abs(L[b, hq] - (s.max() + np.log(e.sum()))) < 1e-12
