"""Host-side tests of the C ABI (no GPU needed): the library loads, exports
every function include/mok.h declares, sizes and layouts are consistent, and
every argument error is caught on the host before anything touches a device."""
import ctypes
import os
import re

import pytest

import mixture_experts_layer_30_amd as mok

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "mok.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mok_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(mok.EXPORTS), names
    L = mok.lib()
    for n in names:
        assert hasattr(L, n), n
        assert ctypes.cast(getattr(L, n), ctypes.c_void_p).value


def test_version_and_status_strings():
    assert mok.version() == 100
    assert mok.status_string(0) == "ok"
    for s in (-1, -2, -3, -4):
        assert mok.status_string(s) and mok.status_string(s) != "unknown status"
    assert mok.status_string(7) == "unknown status"


def P(T=256, H=256, I=512, E=8, k=2, dtype=0):
    return mok.make_problem(T, H, I, E, k, dtype)


def test_buffer_sizes_and_layout():
    ws, sb, cb = mok.buffer_sizes(P())
    R = 512
    assert cb >= R * 2 * 256 + R * 4 * 512
    assert ws >= R * 2 * 256 * 4          # backward keeps four [R][H]-sized buffers
    L = mok.schedule_layout(P())
    assert L.total == sb
    offs = [L.status, L.counts, L.offsets, L.perm, L.dest, L.n_fwd_tiles, L.fwd_tiles,
            L.mb_tile_start, L.n_bwd_tiles, L.bwd_tiles]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert L.perm - L.offsets >= 4 * 9 and L.dest - L.perm >= 4 * R
    # default minibatch: round_up(max(4*S*H/I, S*65536/I), 256) capped at R
    assert L.minibatch_rows == 512 and L.n_minibatches == 1 and L.ring_slots == 1


def test_default_minibatch_rule_large_shapes():
    # T=16384, H=4096, I=1536: 4*256*4096/1536 = 2731 (pages' form) and
    # 256*65536/1536 = 10923 (two waves of 256x256 gate|up tiles) -> 11008 rows
    L = mok.schedule_layout(mok.make_problem(16384, 4096, 1536, 128, 8))
    assert L.minibatch_rows == 11008 and L.n_minibatches == 12 and L.ring_slots == 4
    L = mok.schedule_layout(mok.make_problem(16384, 7168, 2048, 32, 4))   # max(3584, 8192)
    assert L.minibatch_rows == 8192 and L.n_minibatches == 8
    L = mok.schedule_layout(mok.make_problem(4096, 2048, 768, 64, 8), mok.make_config(num_cus=128))
    assert L.minibatch_rows == 11008                                      # max(1366, 10923)
    # the pages' bound 4*S*H/I wins once H > 16384
    L = mok.schedule_layout(mok.make_problem(65536, 32768, 256, 8, 1), mok.make_config(num_cus=16))
    assert L.minibatch_rows == 8192                                        # max(8192, 4096)
    L = mok.schedule_layout(mok.make_problem(100, 256, 256, 4, 2),
                            mok.make_config(minibatch_rows=64, ring_slots=9))
    assert L.minibatch_rows == 64 and L.n_minibatches == 4 and L.ring_slots == 4


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), mok.MOK_ERR_INVALID_ARG),
    (dict(k=0), mok.MOK_ERR_INVALID_ARG),
    (dict(k=9), mok.MOK_ERR_INVALID_ARG),
    (dict(E=0), mok.MOK_ERR_INVALID_ARG),
    (dict(H=200), mok.MOK_ERR_UNSUPPORTED),
    (dict(I=96), mok.MOK_ERR_UNSUPPORTED),
    (dict(E=513, k=2), mok.MOK_ERR_UNSUPPORTED),
    (dict(dtype=5), mok.MOK_ERR_INVALID_ARG),
    (dict(T=1 << 29, k=8, E=8), mok.MOK_ERR_UNSUPPORTED),
])
def test_invalid_problems_rejected(kw, status):
    with pytest.raises(mok.MokError) as ei:
        mok.buffer_sizes(P(**kw))
    assert ei.value.status == status


@pytest.mark.parametrize("cfg", [dict(minibatch_rows=-1), dict(ring_slots=-2),
                                 dict(capacity_multiplier=0.5), dict(driver=3)])
def test_invalid_configs_rejected(cfg):
    with pytest.raises(mok.MokError) as ei:
        mok.buffer_sizes(P(), mok.make_config(**cfg))
    assert ei.value.status == mok.MOK_ERR_INVALID_ARG


def test_calls_reject_bad_arguments_before_any_launch():
    L = mok.lib()
    prob = P()
    _, sb, _ = mok.buffer_sizes(prob)
    fake = ctypes.c_void_p(0x1000)
    # null pointers
    assert L.mok_build_schedule(ctypes.byref(prob), None, None, fake, sb, None) == mok.MOK_ERR_INVALID_ARG
    assert L.mok_build_schedule(ctypes.byref(prob), None, fake, None, sb, None) == mok.MOK_ERR_INVALID_ARG
    # schedule buffer too small
    assert L.mok_build_schedule(ctypes.byref(prob), None, fake, fake, sb - 1, None) == mok.MOK_ERR_BUFFER_TOO_SMALL
    w = mok.Weights(0x1000, 0x1000, 0x1000, None, None, None)
    ws, _, _ = mok.buffer_sizes(prob)
    assert L.mok_forward(ctypes.byref(prob), None, fake, fake, fake, ctypes.byref(w), fake, None,
                         fake, ws - 1, None) == mok.MOK_ERR_BUFFER_TOO_SMALL
    w0 = mok.Weights(0x1000, None, 0x1000, None, None, None)
    assert L.mok_forward(ctypes.byref(prob), None, fake, fake, fake, ctypes.byref(w0), fake, None,
                         fake, ws, None) == mok.MOK_ERR_INVALID_ARG
    assert prob.T > 0                        # y is required when there are tokens
    assert L.mok_forward(ctypes.byref(prob), None, fake, fake, fake, ctypes.byref(w), None, None,
                         fake, ws, None) == mok.MOK_ERR_INVALID_ARG
    # MXFP8 forward needs scales; its backward needs the transposed weight copies
    pm = P(dtype=mok.MOK_MXFP8)
    wsm, _, cbm = mok.buffer_sizes(pm)
    _, _, cb = mok.buffer_sizes(prob)
    assert 0 < cbm == cb                     # obuf and a, b in both formats (x is read in place)
    assert L.mok_forward(ctypes.byref(pm), None, fake, fake, fake, ctypes.byref(w), fake, None,
                         fake, wsm, None) == mok.MOK_ERR_INVALID_ARG
    # the backward needs the forward's context when there are tokens
    assert L.mok_backward(ctypes.byref(prob), None, fake, None, fake, fake, ctypes.byref(w), fake,
                          fake, fake, fake, fake, fake, fake, ws, None) == mok.MOK_ERR_INVALID_ARG
    wm = mok.Weights(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    assert L.mok_backward(ctypes.byref(pm), None, fake, fake, fake, fake, ctypes.byref(wm), fake,
                          fake, fake, fake, fake, fake, fake, wsm, None) == mok.MOK_ERR_INVALID_ARG
    # single-launch forward: the schedule's and the forward's checks
    assert L.mok_forward_fused(ctypes.byref(prob), None, None, fake, sb, fake, fake, ctypes.byref(w), fake, None,
                               fake, ws, None) == mok.MOK_ERR_INVALID_ARG          # no topk_ids
    assert L.mok_forward_fused(ctypes.byref(prob), None, fake, None, sb, fake, fake, ctypes.byref(w), fake, None,
                               fake, ws, None) == mok.MOK_ERR_INVALID_ARG          # no schedule
    assert L.mok_forward_fused(ctypes.byref(prob), None, fake, fake, sb - 1, fake, fake, ctypes.byref(w), fake,
                               None, fake, ws, None) == mok.MOK_ERR_BUFFER_TOO_SMALL
    assert L.mok_forward_fused(ctypes.byref(prob), None, fake, fake, sb, fake, fake, ctypes.byref(w), fake, None,
                               fake, ws - 1, None) == mok.MOK_ERR_BUFFER_TOO_SMALL
    assert L.mok_forward_fused(ctypes.byref(prob), None, fake, fake, sb, fake, fake, ctypes.byref(w0), fake, None,
                               fake, ws, None) == mok.MOK_ERR_INVALID_ARG          # missing w_up
    assert L.mok_forward_fused(ctypes.byref(pm), None, fake, fake, sb, fake, fake, ctypes.byref(w), fake, None,
                               fake, wsm, None) == mok.MOK_ERR_INVALID_ARG         # MXFP8 without scales
    # quantize: K must be a multiple of 32
    assert L.mok_mxfp8_quantize(fake, 4, 48, fake, fake, None) == mok.MOK_ERR_INVALID_ARG
    assert L.mok_mxfp8_quantize(fake, -1, 64, fake, fake, None) == mok.MOK_ERR_INVALID_ARG
    assert L.mok_mxfp8_quantize(None, 4, 64, fake, fake, None) == mok.MOK_ERR_INVALID_ARG


def test_router_calls_reject_bad_arguments():
    L = mok.lib()
    fake = ctypes.c_void_p(0x1000)
    prob = P()
    assert L.mok_router_forward(ctypes.byref(prob), None, fake, None, fake, fake, None) == mok.MOK_ERR_INVALID_ARG
    assert L.mok_router_forward(ctypes.byref(prob), fake, fake, None, fake, None, None) == mok.MOK_ERR_INVALID_ARG
    assert L.mok_router_forward(None, fake, fake, None, fake, fake, None) == mok.MOK_ERR_INVALID_ARG
    # at most 64 experts per token (one wavefront's lanes hold the picks)
    assert L.mok_router_forward(ctypes.byref(mok.make_problem(16, 256, 128, 128, 65)), fake, fake, None, fake,
                                fake, None) == mok.MOK_ERR_UNSUPPORTED
    args = [fake] * 9
    assert L.mok_router_backward(ctypes.byref(prob), None, None, *args[:8], None) == mok.MOK_ERR_INVALID_ARG
    for i in range(9):
        a = list(args)
        a[i] = None
        assert L.mok_router_backward(ctypes.byref(prob), None, *a, None) == mok.MOK_ERR_INVALID_ARG, i


def test_transposed_quantize_and_probe_reject_bad_arguments():
    L = mok.lib()
    fake = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1008)                 # not 16-byte aligned
    Q = L.mok_mxfp8_quantize_transposed
    E = mok.MOK_ERR_INVALID_ARG
    assert Q(fake, 2, 48, 64, fake, fake, 64, 0, None) == E          # rows not a multiple of 32
    assert Q(fake, 2, 64, 60, fake, fake, 64, 0, None) == E          # cols not a multiple of 8
    assert Q(fake, 2, 64, 64, fake, fake, 96, 16, None) == E         # col0 not a multiple of 32
    assert Q(fake, 2, 64, 64, fake, fake, 80, 0, None) == E          # ld not a multiple of 32
    assert Q(fake, 2, 64, 64, fake, fake, 64, 32, None) == E         # col0 + rows > ld
    assert Q(fake, -1, 64, 64, fake, fake, 64, 0, None) == E
    assert Q(None, 2, 64, 64, fake, fake, 64, 0, None) == E
    assert Q(fake, 2, 64, 64, fake, None, 64, 0, None) == E
    assert Q(odd, 2, 64, 64, fake, fake, 64, 0, None) == E
    assert Q(fake, 2, 64, 64, odd, fake, 64, 0, None) == E
    assert Q(fake, 70000, 64, 64, fake, fake, 64, 0, None) == mok.MOK_ERR_UNSUPPORTED
    assert Q(None, 0, 64, 64, None, None, 64, 0, None) == mok.MOK_OK  # empty: nothing to do
    P_ = L.mok_probe_mfma
    assert P_(2, 4, 4, fake, None) == E
    assert P_(0, -1, 4, fake, None) == E
    assert P_(1, 4, 4, None, None) == E
