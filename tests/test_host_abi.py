"""CPU tests of the C-ABI library: it loads, exports every symbol the header
declares, and its host-side integer work (slot map, window plan, argument
validation) matches the oracle bit for bit.  No kernel is launched here:
every call below is rejected or answered on the host before any launch."""
import ctypes
import itertools
import os
import re
import subprocess

import numpy as np
import pytest

import causal_video_diffusion_amd as cvd
from causal_video_diffusion_amd import _binding as B
from causal_video_diffusion_amd import workload as wl
import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from causal_video_diffusion_amd import build
        build.build()
    return B.load()


def _header_symbols():
    """Functions declared by every header under include/."""
    syms = set()
    inc = os.path.join(ROOT, "include")
    for name in sorted(os.listdir(inc)):
        if name.endswith(".h"):
            txt = re.sub(r"/\*.*?\*/", "", open(os.path.join(inc, name)).read(), flags=re.S)
            syms |= set(re.findall(r"\b(ust_[a-z0-9_]+)\s*\(", txt))
    return sorted(syms)


def test_exports_every_declared_symbol(lib):
    syms = _header_symbols()
    assert len(syms) == 19
    assert sorted(B.EXPORTS) == syms
    for s in syms:
        assert hasattr(lib, s), s


def _geom(w):
    return cvd.geom(*w.geom_tuple())


def test_slot_of_frame_bit_exact(lib):
    for n_slots, n_sink in [(9, 1), (7, 1), (21, 3), (15, 3), (21, 0), (5, 4), (40, 7)]:
        ring = B.Kv(None, None, n_slots, n_sink)
        got = [B.ust_slot_of_frame(ring, f) for f in range(1000)]
        assert got == [O.slot_of_frame(f, n_slots, n_sink) for f in range(1000)]
    assert B.ust_slot_of_frame(B.Kv(None, None, 3, 3), 0) == -1
    assert B.ust_slot_of_frame(B.Kv(None, None, 8, 1), -1) == -1


def test_window_plan_bit_exact_exhaustive(lib):
    g = _geom(wl.TINY)
    n = 0
    for n_slots in range(4, 16):
        for n_sink in range(0, 4):
            if n_sink >= n_slots:
                continue
            ring = B.Kv(None, None, n_slots, n_sink)
            for n_recent in (-1, 0, 1, 2, 3, 6, 9):
                for f0 in range(0, 45):
                    try:
                        want = O.window_slots(f0, 3, n_sink, n_recent, n_slots)
                    except ValueError:
                        want = None
                    if want is not None and len(want[0]) > B.UST_MAX_WINDOW_FRAMES:
                        want = None
                    if want is None:
                        with pytest.raises(cvd.UstError) as e:
                            B.ust_window_plan(g, ring, f0, n_recent)
                        assert e.value.name == "UST_E_RANGE"
                    else:
                        assert B.ust_window_plan(g, ring, f0, n_recent) == \
                            (list(want[0]), list(want[1]))
                    n += 1
    assert n > 5000


def test_window_plan_long_horizon(lib):
    """Streaming far past one clip with a 15-slot ring, 3 sinks, 9 recent."""
    g = _geom(wl.WAN_720P)
    ring = B.Kv(None, None, 15, 3)
    for f0 in range(0, 1000, 3):
        assert B.ust_window_plan(g, ring, f0, 9) == \
            tuple(list(v) for v in O.window_slots(f0, 3, 3, 9, 15))


def test_window_plan_workloads(lib):
    for w in (wl.TINY, wl.TINY_WRAP, wl.WAN_FULL, wl.WAN_WINDOW, wl.WAN_720P):
        g = _geom(w)
        ring = B.Kv(None, None, w.n_slots, w.n_sink)
        for c in range(w.n_chunks):
            assert B.ust_window_plan(g, ring, 3 * c, w.n_recent) == \
                tuple(list(v) for v in O.window_slots(3 * c, 3, w.n_sink, w.n_recent,
                                                      w.n_slots))


def test_window_plan_errors(lib):
    g = _geom(wl.WAN_WINDOW)
    ring = B.Kv(None, None, 21, 3)
    with pytest.raises(cvd.UstError, match="UST_E_RANGE"):
        B.ust_window_plan(g, ring, -3, 6)
    with pytest.raises(cvd.UstError, match="UST_E_RANGE"):
        B.ust_window_plan(g, ring, 3, -2)
    with pytest.raises(cvd.UstError, match="UST_E_SHAPE"):
        B.ust_window_plan(g, ring, 15, 6, cap=4)
    # a ring too small for the window
    with pytest.raises(cvd.UstError, match="UST_E_RANGE"):
        B.ust_window_plan(g, B.Kv(None, None, 10, 3), 15, 6)
    # a window longer than the maximum
    big = B.Kv(None, None, 400, 0)
    with pytest.raises(cvd.UstError, match="UST_E_RANGE"):
        B.ust_window_plan(g, big, 200, -1)
    # exactly at the maximum (2 sinks + 123 recent + 3 current = 128 frames)
    # is accepted, one frame more is not
    ring130 = B.Kv(None, None, 130, 2)
    frames, slots = B.ust_window_plan(g, ring130, 126, 123)
    assert len(frames) == B.UST_MAX_WINDOW_FRAMES == 128
    assert frames == [0, 1] + list(range(3, 129))
    with pytest.raises(cvd.UstError, match="UST_E_RANGE"):
        B.ust_window_plan(g, B.Kv(None, None, 131, 2), 127, 124)


def test_window_plan_far_frames(lib):
    """Frames near the top of the 32-bit range: a chunk whose last frame
    would pass 2^31 - 1 is rejected (no overflow), and a window far along a
    stream is planned by visiting only its own frames (this returns at once;
    a walk from frame 0 would take 2^31 steps)."""
    g = _geom(wl.WAN_WINDOW)
    ring = B.Kv(None, None, 21, 3)
    top = 2 ** 31 - 1
    for f0 in (top, top - 1):
        with pytest.raises(cvd.UstError, match="UST_E_RANGE"):
            B.ust_window_plan(g, ring, f0, 6)
    f0 = top - 2                       # the chunk's last frame is exactly 2^31 - 1
    frames, slots = B.ust_window_plan(g, ring, f0, 6)
    assert frames == [0, 1, 2] + list(range(f0 - 6, f0 + 3))
    assert slots == [O.slot_of_frame(f, 21, 3) for f in frames]
    # every prior frame: the ring cannot hold them, which is found at once
    with pytest.raises(cvd.UstError, match="UST_E_RANGE"):
        B.ust_window_plan(g, ring, f0, -1)
    # a recent count reaching past frame 0 takes every prior frame once
    frames, _ = B.ust_window_plan(g, B.Kv(None, None, 400, 3), 30, top)
    assert frames == list(range(33))


def _raw(lib, name, *args):
    st = getattr(lib, name)(*args)
    return B.STATUS[st], lib.ust_last_error().decode()


def test_compute_entry_points_reject_bad_arguments(lib):
    """Validation happens before any launch, so these return without a GPU."""
    w = wl.WAN_WINDOW
    g = _geom(w)
    fake = 0x10000          # aligned, never dereferenced: every call below fails validation
    ring = B.Kv(fake, fake, 21, 3)
    gp, rp = ctypes.byref(g), ctypes.byref(ring)
    # NULL pointers
    assert _raw(lib, "ust_kv_append", gp, rp, None, fake, fake, fake, 0, 21, 0, None)[0] == "UST_E_NULL"
    assert _raw(lib, "ust_window_attn", gp, rp, fake, fake, fake, 0, 21, 0, 6, 0.0, None, None,
                None)[0] == "UST_E_NULL"
    assert _raw(lib, "ust_rope_table_build", gp, 0, 21, 1e4, None, fake, None)[0] == "UST_E_NULL"
    assert _raw(lib, "ust_lowrank_proj", fake, fake, fake, None, None, fake, 8, 8, 8, 8,
                None)[0] == "UST_E_NULL"
    assert _raw(lib, "ust_lowrank_proj_static", None, fake, fake, None, fake, 8, 8, 8, 8,
                None)[0] == "UST_E_NULL"
    # the static scratch holds at most UST_LOWRANK_STATIC_MAX_ELEMS elements of T
    big_m = B.UST_LOWRANK_STATIC_MAX_ELEMS // 64 + 8
    st, msg = _raw(lib, "ust_lowrank_proj_static", fake, fake, fake, None, fake, big_m, 64, 64,
                   64, None)
    assert st == "UST_E_RANGE" and "static scratch" in msg
    # the decoder convolution
    assert _raw(lib, "ust_conv3d_causal", None, fake, None, fake, 2, 3, 4, 16, 128,
                None)[0] == "UST_E_NULL"
    assert _raw(lib, "ust_conv3d_causal", fake, fake, None, fake, 0, 3, 4, 16, 128,
                None)[0] == "UST_E_SHAPE"
    assert _raw(lib, "ust_conv3d_causal", fake, fake, None, fake, 2, 3, 4, 48, 128,
                None)[0] == "UST_E_UNSUPPORTED"
    assert _raw(lib, "ust_conv3d_causal", fake, fake, None, fake, 2, 3, 4, 24, 128,
                None)[0] == "UST_E_UNSUPPORTED"
    assert _raw(lib, "ust_conv3d_causal", fake, fake, None, fake, 2, 3, 4, 16, 100,
                None)[0] == "UST_E_UNSUPPORTED"
    assert _raw(lib, "ust_conv3d_causal", fake, fake + 8, None, fake, 2, 3, 4, 16, 128,
                None)[0] == "UST_E_ALIGN"
    assert _raw(lib, "ust_conv3d_causal", fake, fake, None, fake, 2048, 1024, 1024, 16, 128,
                None)[0] == "UST_E_SHAPE"
    # the streaming form: x holds T + 2 frames
    assert _raw(lib, "ust_conv3d_causal_stream", None, fake, None, fake, 2, 3, 4, 16, 128,
                None)[0] == "UST_E_NULL"
    assert _raw(lib, "ust_conv3d_causal_stream", fake, fake, None, fake, 2, 3, 4, 24, 128,
                None)[0] == "UST_E_UNSUPPORTED"
    # 63 x 512 x 1024 x 32 elements fit under 2^30, the 65 frames of x do not
    assert _raw(lib, "ust_conv3d_causal_stream", fake, fake, None, fake, 63, 512, 1024, 32, 32,
                None)[0] == "UST_E_SHAPE"
    # frames outside the table
    assert _raw(lib, "ust_kv_append", gp, rp, fake, fake, fake, fake, 0, 21, 19, None)[0] == "UST_E_RANGE"
    assert _raw(lib, "ust_window_attn", gp, rp, fake, fake, fake, 0, 21, 21, 6, 0.0, fake, None,
                None)[0] == "UST_E_RANGE"
    # misaligned
    assert _raw(lib, "ust_kv_append", gp, rp, fake + 2, fake, fake, fake, 0, 21, 0, None)[0] == "UST_E_ALIGN"
    assert _raw(lib, "ust_lowrank_proj", fake, fake, None, None, None, fake, 8, 12, 8, 8,
                None)[0] == "UST_E_ALIGN"
    # shapes
    assert _raw(lib, "ust_lowrank_proj", fake, fake, None, None, None, fake, 8, 16, 8, 16,
                None)[0] == "UST_E_SHAPE"
    assert _raw(lib, "ust_lowrank_proj", fake, fake, None, None, None, fake, 0, 16, 8, 8,
                None)[0] == "UST_E_SHAPE"
    assert _raw(lib, "ust_rope_table_build", gp, 0, 0, 1e4, fake, fake, None)[0] == "UST_E_SHAPE"
    assert _raw(lib, "ust_rope_table_build", gp, 0, 4, -1.0, fake, fake, None)[0] == "UST_E_RANGE"
    # unsupported head size and token count
    g2 = cvd.geom(30, 52, 12, 96, 16, 16, 16, 3)
    assert _raw(lib, "ust_kv_append", ctypes.byref(g2), rp, fake, fake, fake, fake, 0, 21, 0,
                None)[0] == "UST_E_UNSUPPORTED"
    g3 = cvd.geom(3, 5, 12, 128, 22, 21, 21, 3)
    assert _raw(lib, "ust_kv_append", ctypes.byref(g3), rp, fake, fake, fake, fake, 0, 21, 0,
                None)[0] == "UST_E_UNSUPPORTED"
    # pair split that does not add up
    g4 = cvd.geom(30, 52, 12, 128, 22, 21, 20, 3)
    assert _raw(lib, "ust_kv_append", ctypes.byref(g4), rp, fake, fake, fake, fake, 0, 21, 0,
                None)[0] == "UST_E_SHAPE"
    # ring that cannot hold a chunk
    small = B.Kv(fake, fake, 4, 3)
    assert _raw(lib, "ust_kv_append", gp, ctypes.byref(small), fake, fake, fake, fake, 0, 21, 6,
                None)[0] == "UST_E_RANGE"
    # a window frame already overwritten
    ring10 = B.Kv(fake, fake, 10, 3)
    st, msg = _raw(lib, "ust_window_attn", gp, ctypes.byref(ring10), fake, fake, fake, 0, 21, 15,
                   6, 0.0, fake, None, None)
    assert st == "UST_E_RANGE" and "no longer in the ring" in msg


def test_table_first_frame_rejects_bad_arguments(lib):
    """A table holds the frames tab_first_frame .. tab_first_frame + n_tab_frames
    - 1: the chunk's frames must all lie there, in every consumer; the builder
    rejects a negative first frame and frames past INT32_MAX.  Every call here
    fails in validation, before any launch."""
    w = wl.WAN_WINDOW
    g = _geom(w)
    fake = 0x10000
    ring = B.Kv(fake, fake, 21, 3)
    gp, rp = ctypes.byref(g), ctypes.byref(ring)
    imax = 2 ** 31 - 1
    assert _raw(lib, "ust_rope_table_build", gp, -1, 3, 1e4, fake, fake, None)[0] == "UST_E_RANGE"
    st, msg = _raw(lib, "ust_rope_table_build", gp, imax - 1, 3, 1e4, fake, fake, None)
    assert st == "UST_E_RANGE" and "INT32_MAX" in msg
    kv = lambda t0, n_tab, f0: _raw(lib, "ust_kv_append", gp, rp, fake, fake, fake, fake, t0,
                                    n_tab, f0, None)
    assert kv(-1, 21, 0)[0] == "UST_E_RANGE"
    assert kv(3, 3, 0)[0] == "UST_E_RANGE"                 # chunk before the table
    assert kv(100000, 2, 100000)[0] == "UST_E_RANGE"       # last chunk frame past the table
    st, msg = kv(100000, 3, 100001)
    assert st == "UST_E_RANGE" and "100000..100002" in msg
    # frames near INT32_MAX: 64-bit bounds, no wrap
    assert kv(imax - 2, 3, imax - 1)[0] == "UST_E_RANGE"
    att = lambda t0, n_tab, f0: _raw(lib, "ust_window_attn", gp, rp, fake, fake, fake, t0, n_tab,
                                     f0, 6, 0.0, fake, None, None)
    assert att(-3, 21, 0)[0] == "UST_E_RANGE"
    assert att(16, 3, 15)[0] == "UST_E_RANGE"
    assert att(15, 2, 15)[0] == "UST_E_RANGE"
    need = lib.ust_window_attn_work_bytes(gp, 256)
    assert _raw(lib, "ust_window_attn_split", gp, rp, fake, fake, fake, 18, 3, 15, 6, 0.0, fake,
                None, fake, need, 256, None)[0] == "UST_E_RANGE"
    assert _raw(lib, "ust_qkv_append", gp, rp, fake, fake, 1536, fake, fake, 9, 3, 6, fake,
                None)[0] == "UST_E_RANGE"


def test_window_attn_split_rejects_bad_arguments(lib):
    """The key-split variant validates like ust_window_attn, then its workspace;
    every call here fails before a launch."""
    w = wl.WAN_WINDOW
    g = _geom(w)
    fake = 0x10000
    ring = B.Kv(fake, fake, 21, 3)
    gp, rp = ctypes.byref(g), ctypes.byref(ring)
    need = lib.ust_window_attn_work_bytes(gp, 256)
    args = (gp, rp, fake, fake, fake, 0, 21, 15, 6, 0.0, fake, None)
    # the same validation as the unsplit call comes first
    assert _raw(lib, "ust_window_attn_split", gp, rp, fake, fake, fake, 0, 21, 21, 6, 0.0, fake,
                None, fake, need, 256, None)[0] == "UST_E_RANGE"
    assert _raw(lib, "ust_window_attn_split", gp, rp, fake, fake, fake, 0, 21, 15, 6, 0.0, None,
                None, fake, need, 256, None)[0] == "UST_E_NULL"
    # then the workspace
    assert _raw(lib, "ust_window_attn_split", *args, None, need, 256, None)[0] == "UST_E_NULL"
    assert _raw(lib, "ust_window_attn_split", *args, fake + 4, need, 256, None)[0] == "UST_E_ALIGN"
    st, msg = _raw(lib, "ust_window_attn_split", *args, fake, need - 1, 256, None)
    assert st == "UST_E_SHAPE" and "needed" in msg
    assert _raw(lib, "ust_window_attn_split", *args, fake, need, 1 << 17, None)[0] == "UST_E_SHAPE"


def test_qkv_append_rejects_bad_arguments(lib):
    """The fused projection validates like ust_kv_append, then hidden; every
    call here fails before a launch."""
    w = wl.WAN_WINDOW
    g = _geom(w)
    fake = 0x10000
    ring = B.Kv(fake, fake, 21, 3)
    gp, rp = ctypes.byref(g), ctypes.byref(ring)
    call = lambda x, wq, hidden, n_tab, f0, q: _raw(lib, "ust_qkv_append", gp, rp, x, wq, hidden,
                                                     fake, fake, 0, n_tab, f0, q, None)
    assert call(None, fake, 1536, 21, 0, fake)[0] == "UST_E_NULL"
    assert call(fake, fake, 1536, 21, 0, None)[0] == "UST_E_NULL"
    assert call(fake + 8, fake, 1536, 21, 0, fake)[0] == "UST_E_ALIGN"
    assert call(fake, fake, 0, 21, 0, fake)[0] == "UST_E_SHAPE"
    assert call(fake, fake, 1560, 21, 0, fake)[0] == "UST_E_UNSUPPORTED"   # 1560 % 64 = 24
    assert call(fake, fake, 1536, 21, 19, fake)[0] == "UST_E_RANGE"     # frames 19..21
    small = B.Kv(fake, fake, 4, 3)
    assert _raw(lib, "ust_qkv_append", gp, ctypes.byref(small), fake, fake, 1536, fake, fake, 0,
                21, 6, fake, None)[0] == "UST_E_RANGE"


def test_lowrank_proj_v_append_rejects_bad_arguments(lib):
    """The value projection into the ring validates the geometry, the ring
    and its operands before any launch; misaligned v_new is still rejected
    by ust_kv_append (NULL v_new is the keys-only form)."""
    w = wl.WAN_WINDOW
    g = _geom(w)
    fake = 0x10000
    ring = B.Kv(fake, fake, 21, 3)
    gp, rp = ctypes.byref(g), ctypes.byref(ring)
    call = lambda x, t, hidden, rank, f0, rr=rp: _raw(lib, "ust_lowrank_proj_v_append", gp, rr, x,
                                                     fake, fake, t, hidden, rank, None, None,
                                                     None, 0, 0, f0, None)
    # with the keys: k_new, table, table range
    callk = lambda k, cs, t0, n_tab, f0: _raw(lib, "ust_lowrank_proj_v_append", gp, rp, fake, fake,
                                              fake, fake, 1536, 512, k, cs, fake, t0, n_tab, f0,
                                              None)
    assert callk(fake, None, 0, 21, 0)[0] == "UST_E_NULL"
    assert callk(fake + 8, fake, 0, 21, 0)[0] == "UST_E_ALIGN"
    assert callk(fake, fake + 4, 0, 21, 0)[0] == "UST_E_ALIGN"
    assert callk(fake, fake, 0, 21, 19)[0] == "UST_E_RANGE"        # frames 19..21
    assert callk(fake, fake, 9, 3, 6)[0] == "UST_E_RANGE"          # chunk before the table
    assert callk(fake, fake, -1, 21, 0)[0] == "UST_E_RANGE"
    assert call(None, fake, 1536, 512, 0)[0] == "UST_E_NULL"
    assert call(fake, None, 1536, 512, 0)[0] == "UST_E_NULL"
    assert call(fake + 8, fake, 1536, 512, 0)[0] == "UST_E_ALIGN"
    assert call(fake, fake, 0, 512, 0)[0] == "UST_E_SHAPE"
    assert call(fake, fake, 1536, -64, 0)[0] == "UST_E_SHAPE"
    assert call(fake, fake, 1540, 512, 0)[0] == "UST_E_ALIGN"          # hidden % 8
    assert call(fake, fake, 1536, 520, 0)[0] == "UST_E_UNSUPPORTED"    # rank % 64
    assert call(fake, fake, 1536, 512, -3)[0] == "UST_E_RANGE"
    small = B.Kv(fake, fake, 4, 3)
    assert call(fake, fake, 1536, 512, 6, ctypes.byref(small))[0] == "UST_E_RANGE"
    assert _raw(lib, "ust_kv_append", gp, rp, fake, fake + 2, fake, fake, 0, 21, 0,
                None)[0] == "UST_E_ALIGN"


def test_flow_step_rejects_bad_arguments(lib):
    """Each call fails in validation, before any launch (no GPU needed)."""
    fake = 0x10000
    call = lambda x, v, nz, s, sn, x0, xn, n: _raw(lib, "ust_flow_step", x, v, nz, s, sn, x0,
                                                 xn, n, None)
    assert call(None, fake, fake, 0.5, 0.25, None, fake, 8)[0] == "UST_E_NULL"
    assert call(fake, None, fake, 0.5, 0.25, None, fake, 8)[0] == "UST_E_NULL"
    assert call(fake, fake, fake, 0.5, 0.25, None, None, 8)[0] == "UST_E_NULL"
    assert call(fake, fake, None, 0.5, 0.25, None, fake, 8)[0] == "UST_E_NULL"   # noise needed
    assert call(fake, fake, fake, 0.5, 0.25, None, fake, -1)[0] == "UST_E_SHAPE"
    assert call(fake, fake, fake, 1.5, 0.25, None, fake, 8)[0] == "UST_E_RANGE"
    assert call(fake, fake, fake, 0.5, -0.1, None, fake, 8)[0] == "UST_E_RANGE"
    assert call(fake, fake, fake, float("nan"), 0.0, None, fake, 8)[0] == "UST_E_RANGE"
    assert call(fake + 4, fake, fake, 0.5, 0.25, None, fake, 8)[0] == "UST_E_ALIGN"
    assert call(fake, fake, fake, 0.5, 0.25, fake + 8, fake, 8)[0] == "UST_E_ALIGN"
    assert call(fake, fake, None, 0.5, 0.0, None, fake, 0)[0] == "UST_OK"   # nothing to do


def test_sigma_schedule_matches_oracle_and_table4(lib):
    """The library's levels and labels against the oracle (same closed form in
    fp64, to rounding) and Table 4's printed fractions; argument errors."""
    raw = [1000, 750, 500, 250, 0]
    sig, lab = B.ust_sigma_schedule(raw)
    ref = O.shifted_sigma(raw)
    assert np.allclose(sig, ref, rtol=1e-15, atol=0)
    assert np.allclose(lab, O.dit_label(ref), rtol=1e-15, atol=0)
    assert sig[:4] == [1.0, 15 / 16, pytest.approx(5 / 6, rel=1e-15), 5 / 8] and sig[4] == 0.0
    arr = (ctypes.c_int32 * 2)(1000, 1001)
    out = (ctypes.c_double * 2)()
    assert _raw(lib, "ust_sigma_schedule", arr, 2, 5.0, 1000, out, None)[0] == "UST_E_RANGE"
    assert _raw(lib, "ust_sigma_schedule", arr, 1, 0.0, 1000, out, None)[0] == "UST_E_RANGE"
    assert _raw(lib, "ust_sigma_schedule", None, 1, 5.0, 1000, out, None)[0] == "UST_E_NULL"
    assert _raw(lib, "ust_sigma_schedule", arr, -1, 5.0, 1000, out, None)[0] == "UST_E_SHAPE"


def test_window_attn_work_bytes(lib):
    """2 partial outputs (256 rows x (D values + 1 log-sum-exp), fp32) per workgroup."""
    for w in (wl.WAN_WINDOW, wl.TINY):
        g = _geom(w)
        for n in (1, 7, 256, 1000):
            assert lib.ust_window_attn_work_bytes(ctypes.byref(g), n) == \
                2 * n * 256 * (w.head_dim + 1) * 4
    g = _geom(wl.WAN_WINDOW)
    assert lib.ust_window_attn_work_bytes(ctypes.byref(g), 1 << 17) == 0
    bad = cvd.geom(30, 52, 12, 96, 16, 16, 16, 3)
    assert lib.ust_window_attn_work_bytes(ctypes.byref(bad), 256) == 0


def _schedule_cases():
    """(units, key tiles per unit, requested workgroups): the parity-test and
    bench shapes, plus every small combination, so that units split over 1..many
    workgroups and workgroups span 1..many units, with ragged boundaries."""
    cases = [(228, 293, 256), (228, 293, 1), (228, 293, 228), (228, 293, 512),
             (228, 293, 65536), (1, 3, 256), (1, 1, 256), (2, 1, 3), (19, 3, 256),
             (19, 3, 5), (12, 500, 256), (38, 48, 256), (1000, 7, 256), (256, 10, 256),
             (512, 10, 256), (300, 293, 256), (24, 293, 304),
             # whole-unit rounds followed by a small key-split rest
             (516, 844, 256), (257, 1, 256), (300, 2, 256), (4, 1, 3), (513, 3, 256),
             (1000, 1, 999), (600, 5, 256)]
    for u, t, g in itertools.product(range(1, 13), range(1, 13), (1, 2, 3, 5, 7, 16, 64, 1000)):
        cases.append((u, t, g))
    # the GPU tests' shapes: units x key tiles of every chunk, at their workgroup counts
    shapes = [(1, (2, 3)), (2, (24, 48)), (4, (2, 4, 5)), (24, (5, 10, 15, 20)),
              (228, (74, 147, 220, 293, 366, 439, 512)), (516, (169, 338, 507, 675, 844))]
    for u, tiles in shapes:
        for t in tiles:
            for g in (1, 2, 5, 7, 37, 256, 304):
                cases.append((u, t, g))
    return cases


def test_split_schedule_covers_every_tile_once(tmp_path):
    """The key-split schedule (attn_schedule.h, shared by the attention and merge
    kernels), run on the CPU: exact coverage, in-range key tiles and partial slots,
    and a merge that reads exactly the slots the segments wrote."""
    from causal_video_diffusion_amd import build
    exe = tmp_path / "attn_schedule_check"
    src = os.path.join(ROOT, "tests", "attn_schedule_check.cpp")
    subprocess.run([build.hipcc(), "-O1", "-std=c++17", f"--offload-arch={build.ARCH}", src,
                    "-o", str(exe)], check=True, capture_output=True)
    cases = _schedule_cases()
    inp = "".join(f"{u} {t} {g}\n" for u, t, g in cases)
    r = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == f"ok {len(cases)}", r.stdout


def test_gemm_tile_order_covers_every_tile_once(tmp_path):
    """The pipelined GEMM's tile order (gemm_order.h, shared with the kernel),
    run on the CPU: every tile once, a contiguous run of tiles per XCD, the
    row-major order exactly when the grid fits one round or W fits one L2,
    and compact blocks per XCD in the grouped order; and the positions of
    the extra (key-append) workgroups past the tiles: each once, in
    contiguous per-XCD runs."""
    from causal_video_diffusion_amd import build
    exe = tmp_path / "gemm_order_check"
    src = os.path.join(ROOT, "tests", "gemm_order_check.cpp")
    subprocess.run([build.hipcc(), "-O1", "-std=c++17", f"--offload-arch={build.ARCH}", src,
                    "-o", str(exe)], check=True, capture_output=True)
    cases = []
    # the path's products (fused Q/K/V 19 x 36 with 14.2 MB of W, the projections,
    # 720p), then grids around one round and the L2 size, and ragged last groups
    for nbm, nbn, wb in [(19, 36, 4608 * 1536 * 2), (19, 12, 1536 * 1536 * 2),
                         (37, 4, 512 * 1536 * 2), (19, 12, 1536 * 512 * 2),
                         (57, 12, 1536 * 256 * 2), (25, 72, 2304 * 1536 * 2)]:
        cases.append((nbm, nbn, wb))
    for nbm in (1, 2, 3, 4, 5, 7, 8, 9, 16, 17, 18, 19, 33, 64, 65):
        for nbn in (1, 2, 3, 8, 12, 13, 36, 40, 72):
            for wb in (1 << 20, (4 << 20), (4 << 20) + 2, 16 << 20):
                cases.append((nbm, nbn, wb))
    inp = "".join(f"{m} {n} {w}\n" for m, n, w in cases)
    r = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, timeout=120)
    # then the extra workgroups' order: 9 range starts x (70 small + 4 large) sizes
    n_ranges = 9 * (70 + 4)
    assert r.returncode == 0 and r.stdout.strip() == f"ok {len(cases) + n_ranges}", r.stdout


def test_status_strings(lib):
    for k, v in B.STATUS.items():
        assert lib.ust_status_str(k).decode() == v
    assert lib.ust_v_row_len(1560) == 1600 and lib.ust_v_row_len(64) == 64
    assert lib.ust_v_row_len(3600) == 3648 and lib.ust_v_row_len(0) == -1
