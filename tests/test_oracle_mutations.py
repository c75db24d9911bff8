"""Planted mistakes in the oracle (on the CPU) must be caught by the pins.

Each case patches one plausible mistake into the oracle and re-runs the pin
tests that should catch it; at least one must fail."""
import math

import numpy as np
import pytest

import oracle
import importlib

attend_mod = importlib.import_module("oracle.attend")
state_mod = importlib.import_module("oracle.state")
vis_mod = importlib.import_module("oracle.visibility")
from tests import test_int8_format as t8
from tests import test_oracle_math as tm
from tests import test_oracle_pins as tp


def _fails(fns):
    for fn in fns:
        try:
            fn()
        except AssertionError:
            return True
    return False


def _bf_all():
    for c in tm.TINY:
        tm.test_brute_force_tiny(c, 0)


def test_mutation_missing_softmax_scale(monkeypatch):
    monkeypatch.setattr(attend_mod, "_scale", lambda prob: 1.0)
    assert _fails([_bf_all])


def test_mutation_wrong_gqa_map(monkeypatch):
    orig = attend_mod.gather_rows

    def bad(prob, buf, b, h_kv, positions, **kw):
        # query group i of head h reads head (h+1) mod H_kv
        return orig(prob, buf, b, (h_kv + 1) % prob.num_kv_heads, positions, **kw)
    monkeypatch.setattr(attend_mod, "gather_rows", bad)
    assert _fails([_bf_all])


def test_mutation_window_off_by_one(monkeypatch):
    orig = vis_mod.visible_positions

    def bad(T, mask_kind="causal", n_sink=0, window=0):
        if mask_kind == "sink_window":
            return orig(T, mask_kind, n_sink, window + 1)
        return orig(T, mask_kind, n_sink, window)
    monkeypatch.setattr(vis_mod, "visible_positions", bad)
    monkeypatch.setattr(oracle, "visible_positions", bad)
    monkeypatch.setattr(attend_mod, "visible_positions", bad)
    assert _fails([tp.test_window_and_sink_sets, _bf_all])


def test_mutation_paged_row_swapped(monkeypatch):
    monkeypatch.setattr(attend_mod, "paged_nhd_offset",
                        lambda page, r, h, x, P, H, D: ((page * P + (P - 1 - r)) * H + h) * D + x)
    assert _fails([_bf_all])


def test_mutation_merge_wrong_frame(monkeypatch):
    def bad(a, b):
        if not a.valid:
            return b
        if not b.valid:
            return a
        m = max(a.m, b.m)
        return state_mod.State(True, m, a.l + b.l, a.u + b.u)   # forgot alpha/beta
    monkeypatch.setattr(state_mod, "merge_state", bad)
    monkeypatch.setattr(oracle, "merge_state", bad)
    monkeypatch.setattr(attend_mod, "merge_state", bad)
    assert _fails([tp.test_worked_three_split_trace_bit_exact,
                   lambda: tm.test_partition_invariance(0)])


def test_mutation_empty_split_not_identity(monkeypatch):
    def bad(scores, values, allowed=None):
        scores = np.asarray(scores, dtype=np.float64)
        values = np.asarray(values, dtype=np.float64)
        if values.ndim == 1:
            values = values[:, None]
        if allowed is not None:
            scores, values = scores[np.asarray(allowed)], values[np.asarray(allowed)]
        if scores.size == 0:
            return state_mod.State(True, 0.0, 1.0, np.zeros(values.shape[1]))  # fake mass
        m = float(scores.max())
        w = np.exp(scores - m)
        return state_mod.State(True, m, float(w.sum()), w @ values)
    monkeypatch.setattr(oracle, "summarize_allowed", bad)
    monkeypatch.setattr(attend_mod, "summarize_allowed", bad)
    assert _fails([tp.test_worked_three_split_trace_bit_exact,
                   lambda: tm.test_partition_invariance(1)])


def test_mutation_int8_scale_axis(monkeypatch):
    """K scale indexed by token instead of by 128-token group."""
    orig = attend_mod.gather_rows

    def bad(prob, buf, b, h_kv, positions, **kw):
        if prob.kv_format != "i8":
            return orig(prob, buf, b, h_kv, positions, **kw)
        K, V, offs, reg = orig(prob, buf, b, h_kv, positions, **kw)
        pos = np.asarray(positions)
        q = reg == 0
        G = prob.k_group
        gi = np.minimum(pos[q], buf["k_scale"].shape[1] - 1)
        wrong = oracle.decode_f16(buf["k_scale"][b, gi, h_kv, :])
        right = oracle.decode_f16(buf["k_scale"][b, pos[q] // G, h_kv, :])
        K[q] = K[q] / right * wrong
        return K, V, offs, reg
    monkeypatch.setattr(attend_mod, "gather_rows", bad)
    assert _fails([lambda: t8.test_int8_oracle_equals_decoded_reference(("causal", 0, 0))])


def test_mutation_empty_request_reads_a_row(monkeypatch):
    """A length-0 request that still reads position 0 (loop bound rounded up)."""
    def bad(T, mask_kind="causal", n_sink=0, window=0):
        return vis_mod.visible_positions(max(int(T), 1), mask_kind, n_sink, window)
    monkeypatch.setattr(attend_mod, "visible_positions", bad)
    assert _fails([tm.test_empty_and_all_masked_rows])


quant_mod = importlib.import_module("oracle.quant")


def _kivi_pins():
    from tests import test_kivi_append as tk
    fns = [lambda c=c: tk.test_closure_counts_follow_the_pages_rule(c) for c in tk._golden()["cases"]]
    fns += [lambda: tk.test_sequential_appends_equal_the_static_writer(128, 128, 300),
            lambda: tk.test_sequential_appends_equal_the_static_writer(32, 128, 300)]
    return fns


def test_mutation_kivi_closes_at_residual_instead_of_above(monkeypatch):
    orig = quant_mod.quantized_count

    def bad(T, policy, k_group, residual_len):
        if policy == "groups":
            return k_group * max(0, -(-(int(T) - residual_len + 1) // k_group))
        return orig(T, policy, k_group, residual_len)
    monkeypatch.setattr(quant_mod, "quantized_count", bad)
    from tests import test_kivi_append as tk
    monkeypatch.setattr(tk, "quantized_count", bad)
    assert _fails(_kivi_pins())


def test_mutation_kivi_append_v_scale_per_channel(monkeypatch):
    orig = quant_mod.quantize_symmetric

    def bad(x, axis, *a, **k):
        # V (one scale per token, over the last axis) quantized with one scale
        # per channel over the tokens instead, the scales then spread over the
        # per-token slots
        if axis == 2:
            c, s = orig(x, 0, *a, **k)
            return c, np.resize(s, np.asarray(x).shape[:2]).astype(s.dtype)
        return orig(x, axis, *a, **k)
    monkeypatch.setattr(quant_mod, "quantize_symmetric", bad)
    from tests import test_kivi_append as tk
    assert _fails([lambda: tk.test_sequential_appends_equal_the_static_writer(32, 128, 300),
                   tk.test_input_writer_matches_oracle_writer_under_groups_policy,
                   lambda: t8.test_writers_agree_byte_for_byte([300, 128, 5])])


def test_mutation_fp16_scale_rounded_toward_zero(monkeypatch):
    # committing the scale by truncation instead of rounding to nearest
    def bad(v):
        v = np.asarray(v, dtype=np.float64)
        _, e = np.frexp(v)
        spacing = np.ldexp(1.0, np.maximum(e - 11, -24))
        return np.floor(v / spacing) * spacing
    monkeypatch.setattr(quant_mod, "fp16_round", bad)
    assert _fails([t8.test_fp16_commit_matches_ieee_binary16])
