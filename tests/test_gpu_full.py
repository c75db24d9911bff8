"""Every config at its full size, on the launches the bench times: all output
rows against the oracle for seeds 0, 1 and 2, and the rows the timed kernels
load (their trace instances) against the oracle's visible rows for every
(b, h_kv): exact offsets, each row once, int8 scale rows included
("M4.5 - Decode Attention Kernels, Mask Programs, and Backend Boundaries",
sections 0x04F and 0x04H).  Each case prints its max |dO| and max |dLSE|."""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

TOL = {1: 1e-5, 2: 2e-3, 3: 2e-3, 4: 2e-3}


def _check(cfg, seed, what, O, L, Or, Lr):
    if cfg == 5:
        H.check_rows(O, L, Or, Lr, 0.0, rtol=1e-2)
    else:
        H.check_rows(O, L, Or, Lr, TOL[cfg])
    e, le = H.errors(O, L, Or, Lr)
    H.announce(f"cfg{cfg} seed {seed} {what}: max|dO| = {e:.3e} (max|O_ref| = "
               f"{float(np.max(np.abs(Or))):.3g}), max|dLSE| = {le:.3e}")


@pytest.mark.parametrize("cfg", [1, 2, 4, 5])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_full_forward_all_rows(cfg, seed):
    H.announce(f"full cfg{cfg} seed {seed}")
    w = synth.config(cfg, seed)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    dw = H.DeviceWorkload(w)
    O, L, plan = H.forward(w, dw=dw)
    _check(cfg, seed, f"forward S={plan.num_splits}", O, L, Or, Lr)
    O, L, plan = H.run(w, dw=dw)
    _check(cfg, seed, f"run+combine S={plan.num_splits}", O, L, Or, Lr)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_cfg3_all_rows_fixed_splits_and_partition(seed):
    H.announce(f"full cfg3 seed {seed}")
    w = synth.config(3, seed)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    dw = H.DeviceWorkload(w)
    O, L, plan = H.run(w, dw=dw)
    _check(3, seed, f"fixed splits S={plan.num_splits}", O, L, Or, Lr)
    O, L, _ = H.run(w, dw=dw, partition=0)
    _check(3, seed, "balanced partition", O, L, Or, Lr)
    assert np.all(np.isfinite(O))      # poisoned tails and spare pages never reached


@pytest.mark.parametrize("cfg", [1, 2, 4, 5])
def test_full_trace_forward(cfg):
    H.announce(f"full trace cfg{cfg}")
    w = synth.config(cfg, 0)
    Or, Lr, ref = oracle.attend(w.problem, w.buffers, with_trace=True)
    tr, plan, O, L = H.trace(w, forward=True)
    rows = H.check_trace(w, tr, ref=ref)
    _check(cfg, 0, f"trace instance, {rows} rows", O, L, Or, Lr)
    if cfg == 5:
        assert rows == 16 * 8 * 4100


def test_cfg3_full_trace_fixed_splits_and_partition():
    H.announce("full trace cfg3")
    w = synth.config(3, 0)
    Or, Lr, ref = oracle.attend(w.problem, w.buffers, with_trace=True)
    dw = H.DeviceWorkload(w)
    for part in (None, 0):
        tr, plan, O, L = H.trace(w, dw=dw, partition=part)
        rows = H.check_trace(w, tr, ref=ref)
        assert rows == 8 * int(np.sum(w.buffers["seq_lens"]))
        _check(3, 0, f"trace instance ({'partition' if part is not None else 'fixed'}), {rows} rows",
               O, L, Or, Lr)


def test_cfg5_larger_grid_instance():
    """Config 5 at S = 6 (768 workgroups, 3 per CU) runs the int8 kernel's
    168-VGPR instance (separate sink phase) instead of the auto plan's; every
    row and every load against the oracle."""
    H.announce("full cfg5 S=6")
    w = synth.config(5, 0)
    Or, Lr, ref = oracle.attend(w.problem, w.buffers, with_trace=True)
    dw = H.DeviceWorkload(w)
    O, L, plan = H.forward(w, num_splits=6, dw=dw)
    assert plan.num_splits == 6
    _check(5, 0, "forward S=6", O, L, Or, Lr)
    tr, plan, O, L = H.trace(w, num_splits=6, dw=dw, forward=True)
    assert H.check_trace(w, tr, ref=ref) == 16 * 8 * 4100
    _check(5, 0, "trace instance S=6", O, L, Or, Lr)
