"""GPU parity for the FlashMask mask program (M4.5 §0x06A-§0x06D): library
block summaries equal the oracle's, attention equals the oracle over the
visible columns of the decode row, and the rows the timed kernel loads (its
trace instance) are the oracle's visible set plus, at most, hidden rows of
PARTIAL tiles: SKIP tiles are never read."""
import numpy as np
import pytest

import oracle
import synth
from oracle import flashmask as fm
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name(request):
    H.announce(request.node.nodeid)


def _masked(w, seed):
    p = w.problem
    L = p.max_seq_len
    w.buffers["mask_intervals"] = synth.flashmask_intervals(seed, w.buffers["seq_lens"], L)
    p.mask_kind = "flashmask"
    return w


def _ready(w, num_splits=None):
    dw = H.DeviceWorkload(w)
    plan, _ = H.plan_for(w, num_splits)
    summ = dw.summarize_mask(plan)
    ref = np.stack([fm.block_summary(w.buffers["mask_intervals"][b], 16) for b in range(w.problem.batch)])
    assert np.array_equal(summ, ref)
    return dw


@pytest.mark.parametrize("S", [None, 3, 9])
def test_flashmask_contiguous(S):
    lens = [3000, 517, 16, 1, 0, 2222]
    w = _masked(synth.make_contiguous(61, len(lens), 32, 8, 128, lens, kv_capacity=3008), 1)
    dw = _ready(w, S)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    O, L, _ = H.forward(w, num_splits=S, dw=dw)
    H.check_rows(O, L, Or, Lr, 2e-3)
    O, L, _ = H.run(w, num_splits=S, dw=dw)
    H.check_rows(O, L, Or, Lr, 2e-3)


def test_flashmask_paged_and_trace():
    lens = [1500, 33, 700]
    w = _masked(synth.make_paged(62, len(lens), 8, 2, 128, lens, page_size=16), 2)
    dw = _ready(w)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    O, L, _ = H.forward(w, dw=dw)
    H.check_rows(O, L, Or, Lr, 2e-3)
    _trace_rows_fm(w, dw, 4)


def test_flashmask_trace_contiguous():
    lens = [2000, 100, 3]
    w = _masked(synth.make_contiguous(63, len(lens), 8, 2, 128, lens, kv_capacity=2000), 3)
    dw = _ready(w, 3)
    _trace_rows_fm(w, dw, 3)
    _trace_rows_fm(w, dw, 3, forward=True)


def test_flashmask_long_request_tile_numbering():
    """A request of more than 4096 tiles: the non-SKIP numbering spans several
    passes of the prefix scan and many entries per wave."""
    lens = [70001, 4099]
    w = _masked(synth.make_contiguous(65, len(lens), 8, 2, 128, lens, kv_capacity=70016), 4)
    dw = _ready(w)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    O, L, _ = H.forward(w, dw=dw)
    H.check_rows(O, L, Or, Lr, 2e-3)
    _trace_rows_fm(w, dw, None)


def test_flashmask_everything_hidden():
    lens = [400, 64]
    w = synth.make_contiguous(64, 2, 8, 2, 128, lens, kv_capacity=400)
    iv = np.zeros((2, 400, 4), np.int32)
    iv[:, :, 0], iv[:, :, 1] = 0, 1 << 30          # UT covers every query row
    iv[:, :, 2], iv[:, :, 3] = 1 << 30, 1 << 30
    w.buffers["mask_intervals"] = iv
    w.problem.mask_kind = "flashmask"
    dw = _ready(w)
    O, L, _ = H.forward(w, dw=dw)
    assert np.all(O == 0) and not np.signbit(O).any() and np.all(np.isneginf(L))


def _trace_rows_fm(w, dw, S, forward=False):
    """The timed kernel's trace instance loads every visible column once and
    hidden columns only inside PARTIAL tiles (never a SKIP tile)."""
    summ = [fm.block_summary(w.buffers["mask_intervals"][b], 16) for b in range(w.problem.batch)]
    lens = w.buffers["seq_lens"]

    def partial(b, pos):
        q = int(lens[b]) - 1
        return pos < lens[b] and fm.classify_tile(q, q + 1, summ[b][pos // 16]) == "PARTIAL"
    tr, plan, O, L = H.trace(w, num_splits=S, dw=dw, forward=forward)
    H.check_trace(w, tr, fm_partial=partial)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    H.check_rows(O, L, Or, Lr, 2e-3)