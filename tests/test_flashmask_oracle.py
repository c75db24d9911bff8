"""Pins of the FlashMask column-interval mask program (M4.5 §0x06A-§0x06F) as
the oracle applies it to the decode row."""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth
from oracle import flashmask as fm
from tests.conftest import GOLDEN


def test_worked_column_half_open():
    with open(os.path.join(GOLDEN, "flashmask_column.json")) as f:
        fx = json.load(f)
    iv = fx["UT"] + fx["LT"]
    hidden = [q for q in range(12) if fm.masked(q, iv)]
    assert hidden == fx["masked_rows"]
    assert all(not fm.masked(q, iv) for q in fx["visible_rows_between"])


def test_summary_is_blockwise_min_max():
    g = synth.rng(3)
    iv = g.integers(0, 50, size=(37, 4)).astype(np.int32)
    s = fm.block_summary(iv, 16)
    assert s.shape == (3, 8)
    for J in range(3):
        blk = iv[J * 16:(J + 1) * 16]
        for v in range(4):
            assert s[J, 2 * v] == min(blk[:, v]) and s[J, 2 * v + 1] == max(blk[:, v])


@pytest.mark.parametrize("seed", range(4))
def test_tile_classifier_is_safe(seed):
    """SKIP never for a tile with a visible cell, FULL never for a tile with a
    hidden cell (§0x06D), over random intervals and query rows."""
    g = synth.rng(seed)
    seen = set()
    for _ in range(400):
        iv = np.sort(g.integers(0, 40, size=(16, 2, 2)), axis=2).reshape(16, 4)
        if g.random() < 0.3:
            iv[:, 0:2] = [g.integers(0, 10), g.integers(25, 40)]          # one covering run
        s = fm.block_summary(iv, 16)[0]
        q0 = int(g.integers(0, 40))
        q1 = q0 + 1
        cls = fm.classify_tile(q0, q1, s)
        seen.add(cls)
        hid = [fm.masked(q0, iv[j]) for j in range(16)]
        if cls == "SKIP":
            assert all(hid)
        if cls == "FULL":
            assert not any(hid)
    assert seen == {"SKIP", "FULL", "PARTIAL"}


def test_flashmask_attention_matches_dense_masked_softmax():
    """Skipping hidden columns is exact (§0x06F): the oracle equals a dense
    pure-Python softmax over all T columns with hidden scores at -inf."""
    lens = [40, 1, 33]
    w = synth.make_contiguous(16, 3, 4, 2, 8, lens, dtype="f32", kv_capacity=48)
    iv = synth.flashmask_intervals(2, lens, 48, block=4)
    w.problem.mask_kind = "flashmask"
    w.buffers["mask_intervals"] = iv
    O, L = oracle.attend(w.problem, w.buffers)
    q, k, v = (w.buffers[x].astype(np.float64) for x in ("q", "k", "v"))
    for b, T in enumerate(lens):
        for hq in range(4):
            h = hq // 2
            s = []
            for j in range(T):
                if fm.masked(T - 1, iv[b, j]):
                    s.append(-math.inf)
                else:
                    s.append(math.fsum(q[b, hq, x] * k[b, j, h, x] for x in range(8)) / math.sqrt(8))
            m = max(s)
            if m == -math.inf:
                assert np.all(O[b, hq] == 0) and L[b, hq] == -math.inf
                continue
            e = [math.exp(t - m) if t > -math.inf else 0.0 for t in s]
            den = math.fsum(e)
            for x in range(8):
                ref = math.fsum(e[j] * v[b, j, h, x] for j in range(T)) / den
                assert abs(O[b, hq, x] - ref) < 1e-12
            assert abs(L[b, hq] - (m + math.log(den))) < 1e-12


def test_generated_masks_produce_every_tile_class():
    lens = [3000, 517, 16]
    iv = synth.flashmask_intervals(1, lens, 3072)
    seen = set()
    for b, T in enumerate(lens):
        s = fm.block_summary(iv[b], 16)
        for J in range(-(-T // 16)):
            seen.add(fm.classify_tile(T - 1, T, s[J]))
    assert seen == {"SKIP", "FULL", "PARTIAL"}
