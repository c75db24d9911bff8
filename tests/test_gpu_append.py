"""GPU streaming append (decode_attn_append) against the oracle's append model
(M8.6 §0x06B): byte-exact codes, scales and residual rows, then attention over
the appended cache against the oracle."""
import numpy as np
import pytest

import kv_cache_amd as ka
import oracle
import synth
from oracle.quant import kivi_append, kivi_state_from_parts, kivi_state_parts, quantized_count
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu
G = 128


@pytest.fixture(autouse=True)
def _name(request):
    H.announce(request.node.nodeid)


def _cache(seed, lens, cap, Hq=8, Hkv=2, D=128, values=None, g=G, R=None):
    w = synth.make_int8(seed, len(lens), Hq, Hkv, D, lens, kv_capacity=cap, residual_policy="groups",
                        values=values, k_group=g, residual_len=g if R is None else R)
    w.problem.max_seq_len = cap
    return w


def _parts(buf, b, T, G=G, R=None):
    n_q = quantized_count(T, "groups", G, G if R is None else R)
    return dict(n_q=n_q, k_codes=buf["k"][b, :n_q], k_scale=buf["k_scale"][b, :n_q // G],
                v_codes=buf["v"][b, :n_q], v_scale=buf["v_scale"][b, :n_q],
                k_resid_bits=buf["k_resid"][b, :T - n_q], v_resid_bits=buf["v_resid"][b, :T - n_q])


def _apply_parts(buf, b, parts, G=G):
    n_q = parts["n_q"]
    r = parts["k_resid_bits"].shape[0]
    buf["k"][b, :n_q] = parts["k_codes"]
    buf["v"][b, :n_q] = parts["v_codes"]
    buf["k_scale"][b, :n_q // G] = parts["k_scale"]
    buf["v_scale"][b, :n_q] = parts["v_scale"]
    buf["k_resid"][b, :r] = parts["k_resid_bits"]
    buf["v_resid"][b, :r] = parts["v_resid_bits"]


def _gpu_append(plan, dev, k_new, v_new, lens):
    t = H.torch()
    status = t.zeros(len(lens), dtype=t.int32, device="cuda")
    sl = t.tensor(np.asarray(lens, np.int32), device="cuda")
    kn, vn = H.to_dev(k_new), H.to_dev(v_new)
    ka.decode_attn_append(plan, kn, vn, dev["k"], dev["v"], dev["k_scale"], dev["v_scale"],
                          dev["k_resid"], dev["v_resid"], sl, status,
                          t.cuda.current_stream().cuda_stream)
    t.cuda.synchronize()
    return status.cpu().numpy()


def _host(dev, like):
    out = {}
    for k in ("k", "v", "k_scale", "v_scale", "k_resid", "v_resid"):
        out[k] = dev[k].cpu().numpy().view(like[k].dtype).reshape(like[k].shape)
    return out


def test_append_steps_across_group_closure_byte_exact_and_attention():
    lens = [0, 1, 126, 127, 128, 129, 255, 256, 300]
    cap = 512
    w = _cache(31, lens, cap)
    _, plan, _, _ = ka.decode_attn_plan(ka.problem_from(w.problem))
    dw = H.DeviceWorkload(w)
    ref = {k: w.buffers[k].copy() for k in ("k", "v", "k_scale", "v_scale", "k_resid", "v_resid")}
    cur = list(lens)
    for step in range(3):
        k_new, v_new = synth.append_rows(100 + step, len(lens), 2, 128)
        status = _gpu_append(plan, dw.dev, k_new, v_new, cur)
        assert not status.any()
        for b, T in enumerate(cur):
            st = kivi_state_from_parts(_parts(ref, b, T), G)
            _apply_parts(ref, b, kivi_state_parts(kivi_append(st, k_new[b], v_new[b], G, G)))
        cur = [T + 1 for T in cur]
        got = _host(dw.dev, ref)
        for b, T in enumerate(cur):
            e, g_ = _parts(ref, b, T), _parts(got, b, T)
            for key in ("k_codes", "v_codes", "k_resid_bits", "v_resid_bits"):
                assert np.array_equal(e[key], g_[key]), (step, b, key)
            for key in ("k_scale", "v_scale"):
                assert np.array_equal(e[key].view(np.uint16), g_[key].view(np.uint16)), (step, b, key)
    # attention over the appended cache: GPU buffers vs the oracle's appended bytes
    w.buffers.update(ref)
    w.buffers["seq_lens"] = np.asarray(cur, np.int32)
    dw.dev["seq_lens"] = H.to_dev(w.buffers["seq_lens"])
    O, L, _ = H.forward(w, dw=dw)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    H.check_rows(O, L, Or, Lr, 0.0, rtol=1e-2)


@pytest.mark.parametrize("D,g", [(64, 128), (128, 256), (128, 32), (64, 256), (64, 16)])
def test_append_closure_other_head_dims_and_groups(D, g):
    # the closure's layouts for other head sizes and group lengths (rows per
    # thread from one to sixteen, partial sweeps): appends across a closure,
    # byte-exact against the oracle's append model
    lens = [g - 1, g, 2 * g, 0, 3 * g + 5]
    cap = 4 * g
    w = _cache(41 + D + g, lens, cap, D=D, g=g)
    _, plan, _, _ = ka.decode_attn_plan(ka.problem_from(w.problem))
    dw = H.DeviceWorkload(w)
    ref = {k: w.buffers[k].copy() for k in ("k", "v", "k_scale", "v_scale", "k_resid", "v_resid")}
    cur = list(lens)
    for step in range(2):
        k_new, v_new = synth.append_rows(300 + step, len(lens), 2, D)
        status = _gpu_append(plan, dw.dev, k_new, v_new, cur)
        assert not status.any()
        for b, T in enumerate(cur):
            st = kivi_state_from_parts(_parts(ref, b, T, g), g)
            _apply_parts(ref, b, kivi_state_parts(kivi_append(st, k_new[b], v_new[b], g, g)), g)
        cur = [T + 1 for T in cur]
        got = _host(dw.dev, ref)
        for b, T in enumerate(cur):
            e, g_ = _parts(ref, b, T, g), _parts(got, b, T, g)
            for key in ("k_codes", "v_codes", "k_resid_bits", "v_resid_bits"):
                assert np.array_equal(e[key], g_[key]), (step, b, key)
            for key in ("k_scale", "v_scale"):
                assert np.array_equal(e[key].view(np.uint16), g_[key].view(np.uint16)), (step, b, key)


@pytest.mark.parametrize("D,g,R", [(128, 32, 128), (64, 16, 48), (128, 64, 96), (128, 128, 256),
                                   (64, 256, 300)])
def test_append_residual_longer_than_group(D, g, R):
    # G < R (the page's teaching state closes 32-token groups behind a
    # 128-token residual): a closure takes the oldest G residual rows and the
    # other R - G move down; byte-exact against the oracle's append model over
    # several appends, then attention over the appended cache
    lens = [R - 1, R, R + 1, R + g, 0, 2 * g + R - 2, 3 * g + R + 5]
    cap = 4 * g + R + 16
    w = _cache(51 + D + g + R, lens, cap, D=D, g=g, R=R)
    _, plan, _, _ = ka.decode_attn_plan(ka.problem_from(w.problem))
    dw = H.DeviceWorkload(w)
    ref = {k: w.buffers[k].copy() for k in ("k", "v", "k_scale", "v_scale", "k_resid", "v_resid")}
    cur = list(lens)
    for step in range(3):
        k_new, v_new = synth.append_rows(400 + step, len(lens), 2, D)
        status = _gpu_append(plan, dw.dev, k_new, v_new, cur)
        assert not status.any()
        for b, T in enumerate(cur):
            st = kivi_state_from_parts(_parts(ref, b, T, g, R), g)
            _apply_parts(ref, b, kivi_state_parts(kivi_append(st, k_new[b], v_new[b], g, R)), g)
        cur = [T + 1 for T in cur]
        got = _host(dw.dev, ref)
        for b, T in enumerate(cur):
            e, g_ = _parts(ref, b, T, g, R), _parts(got, b, T, g, R)
            assert e["n_q"] == g_["n_q"]
            for key in ("k_codes", "v_codes", "k_resid_bits", "v_resid_bits"):
                assert np.array_equal(e[key], g_[key]), (step, b, key)
            for key in ("k_scale", "v_scale"):
                assert np.array_equal(e[key].view(np.uint16), g_[key].view(np.uint16)), (step, b, key)
    w.buffers.update(ref)
    w.buffers["seq_lens"] = np.asarray(cur, np.int32)
    dw.dev["seq_lens"] = H.to_dev(w.buffers["seq_lens"])
    O, L, _ = H.forward(w, dw=dw)
    Or, Lr = oracle.attend(w.problem, w.buffers)
    H.check_rows(O, L, Or, Lr, 0.0, rtol=1e-2)


def test_append_no_room_and_bad_scale_write_nothing():
    lens = [128, 128, 511]
    cap = 512
    g = synth.rng(7)
    kf = g.standard_normal((3, cap, 2, 128), dtype=np.float32)
    vf = g.standard_normal((3, cap, 2, 128), dtype=np.float32)
    vf[1, 5, 0, :] = 1e-30          # request 1: a residual V row whose scale underflows fp16
    w = _cache(32, lens, cap, values=(kf, vf))
    _, plan, _, _ = ka.decode_attn_plan(ka.problem_from(w.problem))
    dw = H.DeviceWorkload(w)
    before = _host(dw.dev, w.buffers)
    k_new, v_new = synth.append_rows(200, 3, 2, 128)
    lens_now = [128, 128, 512]      # request 2 is at max_seq_len: no room
    status = _gpu_append(plan, dw.dev, k_new, v_new, lens_now)
    assert status[0] == 0
    assert status[1] == ka.DA_APPEND_BAD_SCALE
    assert status[2] == ka.DA_APPEND_NO_ROOM
    after = _host(dw.dev, w.buffers)

    def raw(x):                         # bytes, so NaN slots compare equal
        return np.ascontiguousarray(x).view(np.uint8)

    for key in before:
        # request 2 (no room) and head 0 of request 1 (bad scale) are untouched
        assert np.array_equal(raw(before[key][2]), raw(after[key][2])), key
        assert np.array_equal(raw(before[key][1, :, 0]), raw(after[key][1, :, 0])), key
    # head 1 of request 1 closed its group normally
    assert not np.array_equal(raw(before["k_scale"][1, 0, 1]), raw(after["k_scale"][1, 0, 1]))   # group 0, head 1
