"""Pins of the CPU oracle against what the paper and mathematics fix.

None of these restates the oracle's formula: each compares it with a closed
form, an invariant, a library special case, a printed value (tests/golden/) or
a brute-force computation by another route (oracle/brute.py).
"""
import math
import os

import numpy as np
import pytest
import torch

from causal_video_diffusion_amd import workload as wl
import oracle as O
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                yield line


# ---------------------------------------------------------------- bf16 input rounding

def test_bf16_rounding_matches_torch():
    rs = np.random.default_rng(1)
    x = np.concatenate([rs.standard_normal(20000).astype(np.float32),
                        (rs.standard_normal(2000) * 1e30).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, -3.5, 65504.0], np.float32)])
    ours = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_oracle_rne_bf16_matches_input_rounding():
    rs = np.random.default_rng(2)
    x = rs.standard_normal(50000).astype(np.float32)
    # ties: values exactly halfway between two bfloat16 neighbours
    ties = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(2.0 + 2.0 ** -7)],
                    np.float32)
    x = np.concatenate([x, ties])
    a = O.rne_bf16(x.astype(np.float64))
    b = wl.bf16_bits_to_f64(wl.f32_to_bf16_bits(x))
    assert np.array_equal(a, b)
    # ties go to the even neighbour
    assert O.rne_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert O.rne_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6


# ---------------------------------------------------------------- RoPE

@pytest.mark.parametrize("w", [wl.TINY, wl.WAN_WINDOW], ids=lambda w: w.name)
def test_rope_preserves_norm(w):
    cos, sin = O.rope_table(w.n_tab_frames, w.grid_h, w.grid_w, w.pairs, w.theta)
    rs = np.random.default_rng(3)
    u = rs.standard_normal((w.n_tab_frames, w.grid_h, w.grid_w, w.head_dim))
    r = O.rope_apply(u, cos, sin)
    n0 = np.linalg.norm(u, axis=-1)
    n1 = np.linalg.norm(r, axis=-1)
    assert np.max(np.abs(n1 - n0) / n0) < 1e-14


@pytest.mark.parametrize("w", [wl.TINY, wl.WAN_WINDOW], ids=lambda w: w.name)
def test_rope_scores_depend_only_on_offset(w):
    """<R(P1) q, R(P2) k> = <R(P1+d) q, R(P2+d) k> for every 3-D shift d."""
    cos, sin = O.rope_table(w.n_tab_frames, w.grid_h, w.grid_w, w.pairs, w.theta)
    rs = np.random.default_rng(4)
    dims = (w.n_tab_frames, w.grid_h, w.grid_w)
    for _ in range(200):
        q = rs.standard_normal(w.head_dim)
        k = rs.standard_normal(w.head_dim)
        p1 = [rs.integers(0, n) for n in dims]
        p2 = [rs.integers(0, n) for n in dims]
        lo = [-min(a, b) for a, b in zip(p1, p2)]
        hi = [n - 1 - max(a, b) for n, a, b in zip(dims, p1, p2)]
        d = [rs.integers(l, h + 1) for l, h in zip(lo, hi)]
        s1 = O.rope_apply(q, cos[tuple(p1)], sin[tuple(p1)]) @ \
            O.rope_apply(k, cos[tuple(p2)], sin[tuple(p2)])
        p1s = tuple(a + b for a, b in zip(p1, d))
        p2s = tuple(a + b for a, b in zip(p2, d))
        s2 = O.rope_apply(q, cos[p1s], sin[p1s]) @ O.rope_apply(k, cos[p2s], sin[p2s])
        assert abs(s1 - s2) <= 1e-12 * max(1.0, abs(s1))


def test_rope_identity_at_origin():
    for w in (wl.TINY, wl.WAN_WINDOW, wl.WAN_720P):
        cos, sin = O.rope_table(2, w.grid_h, w.grid_w, w.pairs, w.theta)
        assert np.all(cos[0, 0, 0] == 1.0) and np.all(sin[0, 0, 0] == 0.0)
        u = np.random.default_rng(5).standard_normal(w.head_dim)
        assert np.array_equal(O.rope_apply(u, cos[0, 0, 0], sin[0, 0, 0]), u)


def test_rope_closed_form_angles():
    n = 0
    for line in _golden_lines("rope_angles.txt"):
        vals, _ = line.split(";")
        pt, ph, pw, f, y, x, p, ang = vals.split()
        pairs = (int(pt), int(ph), int(pw))
        f, y, x, p, ang = int(f), int(y), int(x), int(p), float(ang)
        cos, sin = O.rope_table(f + 1, y + 1, x + 1, pairs, 10000.0)
        assert abs(cos[f, y, x, p] - math.cos(ang)) < 1e-15, line
        assert abs(sin[f, y, x, p] - math.sin(ang)) < 1e-15, line
        n += 1
    assert n == 11


def test_rope_axis_separation():
    """Frame pairs change only with the frame, row pairs only with the row,
    column pairs only with the column."""
    w = wl.WAN_WINDOW
    cos, _ = O.rope_table(4, 5, 6, w.pairs, w.theta)
    pt, ph, _ = w.pairs
    t, h, c = cos[..., :pt], cos[..., pt:pt + ph], cos[..., pt + ph:]
    assert np.all(t == t[:, :1, :1]) and np.all(h == h[:1, :, :1]) \
        and np.all(c == c[:1, :1, :])


def test_rope_matches_complex_brute_force():
    w = wl.TINY
    cos, sin = O.rope_table(w.n_tab_frames, w.grid_h, w.grid_w, w.pairs, w.theta)
    rs = np.random.default_rng(6)
    for f in range(w.n_tab_frames):
        for y in range(w.grid_h):
            for x in range(w.grid_w):
                u = rs.standard_normal(w.head_dim)
                a = O.rope_apply(u, cos[f, y, x], sin[f, y, x])
                b = brute.rope_rotate(list(u), f, y, x, w.pairs, w.theta)
                assert np.max(np.abs(a - np.array(b))) < 1e-13


def test_rope_table_from_a_later_frame():
    """A table that starts at frame F holds, bit for bit, the rows the table
    from frame 0 holds for those frames.  Far past any clip (F ~ 10^6) the
    first temporal pair (frequency theta^0 = 1) turns by the frame index
    itself, and every rotation agrees with the complex brute force."""
    w = wl.TINY
    full_c, full_s = O.rope_table(12, w.grid_h, w.grid_w, w.pairs, w.theta)
    c, s = O.rope_table(3, w.grid_h, w.grid_w, w.pairs, w.theta, first_frame=7)
    assert np.array_equal(c, full_c[7:10]) and np.array_equal(s, full_s[7:10])
    F = 1_000_003
    c, s = O.rope_table(3, w.grid_h, w.grid_w, w.pairs, w.theta, first_frame=F)
    for i in range(3):
        assert abs(c[i, 1, 2, 0] - math.cos(F + i)) < 1e-15
        assert abs(s[i, 1, 2, 0] - math.sin(F + i)) < 1e-15
    rs = np.random.default_rng(61)
    for _ in range(40):
        i, y, x = rs.integers(0, 3), rs.integers(0, w.grid_h), rs.integers(0, w.grid_w)
        u = rs.standard_normal(w.head_dim)
        a = O.rope_apply(u, c[i, y, x], s[i, y, x])
        b = brute.rope_rotate(list(u), F + int(i), int(y), int(x), w.pairs, w.theta)
        assert np.max(np.abs(a - np.array(b))) < 1e-12


def test_stream_shifted_far_keeps_attention():
    """Scores under RoPE depend only on position offsets.  With no sink
    frames, three chunks appended 10^6 frames into a stream, each with a
    table that starts at its own first frame, give the last chunk the
    attention output of the same three chunks at the start of the stream.
    A table row taken for the wrong frame (an offset dropped in the append
    or in the attention) breaks the equality or the indexing."""
    w = wl.TINY
    n_slots, n_sink, n_recent = 9, 0, 6
    rs = np.random.default_rng(62)
    n = 3 * w.T
    ks = [rs.standard_normal((n, w.n_heads, w.head_dim)) for _ in range(3)]
    vs = [rs.standard_normal((n, w.n_heads, w.head_dim)) for _ in range(3)]
    q = rs.standard_normal((n, w.n_heads, w.head_dim))
    outs = []
    for base in (0, 999_999):
        cache = O.KVCache(n_slots, w.n_heads, w.T, w.head_dim)
        for c in range(3):
            f0 = base + 3 * c
            cos, sin = O.rope_table(3, w.grid_h, w.grid_w, w.pairs, w.theta, first_frame=f0)
            O.kv_append(cache, ks[c], vs[c], cos, sin, f0, 3, w.grid_h, w.grid_w, n_slots,
                        n_sink, tab_first=f0)
        outs.append(O.window_attn(cache, q, cos, sin, base + 6, 3, w.grid_h, w.grid_w,
                                  n_slots, n_sink, n_recent, tab_first=base + 6))
    (o0, l0), (o1, l1) = outs
    assert np.max(np.abs(o0 - o1)) < 1e-8 and np.max(np.abs(l0 - l1)) < 1e-8
    # and the shift is not a no-op: the far stream's keys differ from the near ones
    cache_far = O.KVCache(n_slots, w.n_heads, w.T, w.head_dim)
    cos, sin = O.rope_table(3, w.grid_h, w.grid_w, w.pairs, w.theta, first_frame=999_999)
    O.kv_append(cache_far, ks[0], vs[0], cos, sin, 999_999, 3, w.grid_h, w.grid_w, n_slots,
                n_sink, tab_first=999_999)
    cache_near = O.KVCache(n_slots, w.n_heads, w.T, w.head_dim)
    cos, sin = O.rope_table(3, w.grid_h, w.grid_w, w.pairs, w.theta)
    O.kv_append(cache_near, ks[0], vs[0], cos, sin, 0, 3, w.grid_h, w.grid_w, n_slots, n_sink)
    s_far = O.slot_of_frame(999_999, n_slots, n_sink)
    assert np.max(np.abs(cache_far.k[s_far] - cache_near.k[0])) > 1e-2


# ---------------------------------------------------------------- slots and window

@pytest.mark.parametrize("n_slots,n_sink", [(9, 1), (7, 1), (21, 3), (15, 3),
                                            (21, 0), (5, 2), (12, 0), (30, 7)])
def test_slot_map_matches_ring_simulation(n_slots, n_sink):
    sim = brute.ring_simulation(1000, n_slots, n_sink)
    assert [O.slot_of_frame(f, n_slots, n_sink) for f in range(1000)] == sim


def test_slot_map_identity_when_ring_holds_clip():
    for n_sink in (0, 1, 3):
        assert [O.slot_of_frame(f, 21, n_sink) for f in range(21)] == list(range(21))


def test_window_counts_golden():
    table = {w.name: w for w in (wl.TINY, wl.WAN_FULL, wl.WAN_WINDOW, wl.WAN_720P)}
    seen = 0
    for line in _golden_lines("window_counts.txt"):
        if line.startswith("tiny_last_window"):
            frames = [int(v) for v in line.split()[1:]]
            assert O.window_frames(6, 3, 1, 3) == frames
            continue
        vals, keys = line.split(";")
        name, n_sink, n_recent, T, *counts = vals.split()
        w = table[name]
        assert (int(n_sink), int(n_recent), int(T)) == (w.n_sink, w.n_recent, w.T)
        got = []
        for c in range(len(counts)):
            frames, slots = O.window_slots(3 * c, 3, w.n_sink, w.n_recent, w.n_slots)
            assert len(set(slots)) == len(slots)
            got.append(len(frames))
        assert got == [int(v) for v in counts], name
        assert got[-1] * w.T == int(keys)
        seen += 1
    assert seen == 4


def test_window_membership_matches_brute():
    for n_sink in range(0, 4):
        for n_recent in (-1, 0, 1, 3, 6, 9):
            for f0 in range(0, 40, 3):
                got = O.window_frames(f0, 3, n_sink, n_recent)
                want = [f for f in range(f0 + 3)
                        if brute.in_window(f, f0, 3, n_sink, n_recent)]
                assert got == want
                assert got == sorted(set(got))


def test_full_window_equals_all_prior_frames():
    for f0 in range(0, 60, 3):
        for n_recent in (f0, f0 + 5, -1):
            assert O.window_frames(f0, 3, 2, n_recent) == list(range(f0 + 3))


def test_window_resident_iff_no_frame_overwritten():
    """window_slots succeeds exactly when simulating the ring shows every
    window frame still in its slot after the chunk is written."""
    for n_slots in range(2, 14):
        for n_sink in range(0, min(3, n_slots - 1) + 1):
            if n_slots <= n_sink:
                continue
            sim = brute.ring_simulation(60, n_slots, n_sink)
            for n_recent in (-1, 0, 1, 2, 4, 6):
                for f0 in range(0, 54, 3):
                    last = f0 + 2
                    holder = {}
                    for g in range(last + 1):
                        holder[sim[g]] = g
                    frames = O.window_frames(f0, 3, n_sink, n_recent)
                    ok = all(holder[sim[f]] == f for f in frames)
                    if ok:
                        fr, sl = O.window_slots(f0, 3, n_sink, n_recent, n_slots)
                        assert sl == [sim[f] for f in fr]
                    else:
                        with pytest.raises(ValueError):
                            O.window_slots(f0, 3, n_sink, n_recent, n_slots)


# ---------------------------------------------------------------- KV append

def _tiny_chunks(w, n_chunks):
    ks = [wl.bf16_bits_to_f64(wl.chunk_tokens(w, wl.TAG_K, c)) for c in range(n_chunks)]
    vs = [wl.bf16_bits_to_f64(wl.chunk_tokens(w, wl.TAG_V, c)) for c in range(n_chunks)]
    qs = [wl.bf16_bits_to_f64(wl.chunk_tokens(w, wl.TAG_Q, c)) for c in range(n_chunks)]
    return qs, ks, vs


@pytest.mark.parametrize("w", [wl.TINY, wl.TINY_WRAP], ids=lambda w: w.name)
def test_kv_append_matches_brute(w):
    cos, sin = O.rope_table(w.n_tab_frames, w.grid_h, w.grid_w, w.pairs, w.theta)
    _, ks, vs = _tiny_chunks(w, w.n_chunks)
    cache = O.KVCache(w.n_slots, w.n_heads, w.T, w.head_dim)
    written = set()
    for c in range(w.n_chunks):
        before_k = cache.k.copy()
        O.kv_append(cache, ks[c], vs[c], cos, sin, 3 * c, 3, w.grid_h, w.grid_w,
                    w.n_slots, w.n_sink)
        sim = brute.ring_simulation(3 * c + 3, w.n_slots, w.n_sink)
        new_slots = {sim[f] for f in range(3 * c, 3 * c + 3)}
        for s in range(w.n_slots):
            if s not in new_slots:      # untouched slots keep their bits
                assert np.array_equal(cache.k[s], before_k[s], equal_nan=True)
        for i in range(3):
            f = 3 * c + i
            s = sim[f]
            for t in range(w.T):
                for h in range(w.n_heads):
                    want = brute.rope_rotate(list(ks[c][i * w.T + t, h]), f,
                                             t // w.grid_w, t % w.grid_w,
                                             w.pairs, w.theta)
                    assert np.max(np.abs(cache.k[s, h, t] - want)) < 1e-13
                    assert np.array_equal(cache.v[s, h, t], vs[c][i * w.T + t, h])
        written |= new_slots
    untouched = [s for s in range(w.n_slots) if s not in written]
    assert all(np.isnan(cache.k[s]).all() for s in untouched)


# ---------------------------------------------------------------- attention

def _run_tiny(w, n_chunks=None, poison=False):
    """Append every chunk and attend with each; returns [(O, lse)] per chunk."""
    n_chunks = n_chunks or w.n_chunks
    cos, sin = O.rope_table(w.n_tab_frames, w.grid_h, w.grid_w, w.pairs, w.theta)
    qs, ks, vs = _tiny_chunks(w, n_chunks)
    cache = O.KVCache(w.n_slots, w.n_heads, w.T, w.head_dim,
                      fill=np.nan if poison else 0.0)
    res = []
    for c in range(n_chunks):
        O.kv_append(cache, ks[c], vs[c], cos, sin, 3 * c, 3, w.grid_h, w.grid_w,
                    w.n_slots, w.n_sink)
        if poison:
            _, slots = O.window_slots(3 * c, 3, w.n_sink, w.n_recent, w.n_slots)
            for s in range(w.n_slots):
                if s not in slots:
                    cache.k[s] = np.nan
                    cache.v[s] = np.nan
        res.append(O.window_attn(cache, qs[c], cos, sin, 3 * c, 3, w.grid_h,
                                 w.grid_w, w.n_slots, w.n_sink, w.n_recent))
    return res, (qs, ks, vs)


@pytest.mark.parametrize("w", [wl.TINY, wl.TINY_WRAP], ids=lambda w: w.name)
def test_attention_matches_brute(w):
    res, (qs, ks, vs) = _run_tiny(w)
    k_frames, v_frames = {}, {}
    for c in range(w.n_chunks):
        for i in range(3):
            k_frames[3 * c + i] = ks[c][i * w.T:(i + 1) * w.T].tolist()
            v_frames[3 * c + i] = vs[c][i * w.T:(i + 1) * w.T].tolist()
        # brute force sees only the frames written so far
        kf = {f: k_frames[f] for f in range(3 * c + 3)}
        vf = {f: v_frames[f] for f in range(3 * c + 3)}
        o_b, lse_b = brute.window_attention(qs[c].tolist(), kf, vf, 3 * c, 3,
                                            w.grid_h, w.grid_w, w.n_sink,
                                            w.n_recent, w.pairs, w.theta, 0)
        o, lse = res[c]
        assert np.max(np.abs(o[:, 0] - np.array(o_b))) < 1e-12
        assert np.max(np.abs(lse[0] - np.array(lse_b))) < 1e-12


def test_attention_ring_layout_does_not_change_result():
    a, _ = _run_tiny(wl.TINY)
    b, _ = _run_tiny(wl.TINY_WRAP)
    for (oa, la), (ob, lb) in zip(a, b):
        assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_attention_nan_outside_window_is_invisible():
    a, _ = _run_tiny(wl.TINY_WRAP)
    b, _ = _run_tiny(wl.TINY_WRAP, poison=True)
    for (oa, la), (ob, lb) in zip(a, b):
        assert np.isfinite(ob).all()
        assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def _small_geom_cache(w, rs, frames_written, v_const=None, k_zero=False):
    cos, sin = O.rope_table(w.n_tab_frames, w.grid_h, w.grid_w, w.pairs, w.theta)
    cache = O.KVCache(w.n_slots, w.n_heads, w.T, w.head_dim)
    for c in range(frames_written // 3):
        k = np.zeros((w.n_q, w.n_heads, w.head_dim)) if k_zero else \
            rs.standard_normal((w.n_q, w.n_heads, w.head_dim))
        v = np.full((w.n_q, w.n_heads, w.head_dim), v_const) if v_const is not None \
            else rs.standard_normal((w.n_q, w.n_heads, w.head_dim))
        O.kv_append(cache, k, v, cos, sin, 3 * c, 3, w.grid_h, w.grid_w,
                    w.n_slots, w.n_sink)
    return cache, cos, sin


SMALL = wl.WAN_WINDOW.replace(name="small", grid_h=3, grid_w=5, n_heads=2,
                              head_dim=128, n_slots=12, n_sink=3, n_recent=6,
                              n_tab_frames=18)


def test_attention_v_one_gives_one():
    rs = np.random.default_rng(7)
    cache, cos, sin = _small_geom_cache(SMALL, rs, 18, v_const=1.0)
    q = rs.standard_normal((SMALL.n_q, 2, 128)) * 4.0
    o, _ = O.window_attn(cache, q, cos, sin, 15, 3, 3, 5, 12, 3, 6)
    assert np.max(np.abs(o - 1.0)) < 1e-12


def test_attention_k_zero_closed_form():
    """K = 0: every score is 0, so O is the mean of the window values and
    lse = ln(number of keys)."""
    rs = np.random.default_rng(8)
    cache, cos, sin = _small_geom_cache(SMALL, rs, 18, k_zero=True)
    q = rs.standard_normal((SMALL.n_q, 2, 128))
    o, lse = O.window_attn(cache, q, cos, sin, 15, 3, 3, 5, 12, 3, 6)
    frames, slots = O.window_slots(15, 3, 3, 6, 12)
    n_keys = len(frames) * SMALL.T
    assert n_keys == 12 * 15
    for h in range(2):
        mean = cache.v[slots, h].reshape(-1, 128).mean(axis=0)
        assert np.max(np.abs(o[:, h] - mean[None, :])) < 1e-13
    assert np.max(np.abs(lse - math.log(n_keys))) < 1e-13


def test_attention_matches_sdpa_on_gathered_window():
    rs = np.random.default_rng(9)
    w = SMALL
    cache, cos, sin = _small_geom_cache(w, rs, 18)
    q = rs.standard_normal((w.n_q, 2, 128))
    o, _ = O.window_attn(cache, q, cos, sin, 15, 3, 3, 5, 12, 3, 6)
    frames, slots = O.window_slots(15, 3, 3, 6, 12)
    f, y, x = O.chunk_positions(15, 3, 3, 5)
    qr = O.rope_apply(q, cos[f, y, x][:, None, :], sin[f, y, x][:, None, :])
    for h in range(2):
        K = torch.from_numpy(cache.k[slots, h].reshape(-1, 128))
        V = torch.from_numpy(cache.v[slots, h].reshape(-1, 128))
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qr[:, h])[None], K[None], V[None])[0].numpy()
        assert np.max(np.abs(o[:, h] - ref)) < 1e-12


def test_full_window_equals_block_causal_attention():
    """With every prior frame in the window, windowed attention equals full
    chunk-causal attention over all frames written so far, built with an
    explicit (query frame, key frame) mask."""
    rs = np.random.default_rng(10)
    w = SMALL.replace(n_slots=18, n_sink=0, n_recent=-1)
    cos, sin = O.rope_table(18, w.grid_h, w.grid_w, w.pairs, w.theta)
    cache = O.KVCache(18, 2, w.T, 128)
    all_k, all_v, frame_of = [], [], []
    for c in range(6):
        k = rs.standard_normal((w.n_q, 2, 128))
        v = rs.standard_normal((w.n_q, 2, 128))
        O.kv_append(cache, k, v, cos, sin, 3 * c, 3, w.grid_h, w.grid_w, 18, 0)
        f, y, x = O.chunk_positions(3 * c, 3, w.grid_h, w.grid_w)
        all_k.append(O.rope_apply(k, cos[f, y, x][:, None], sin[f, y, x][:, None]))
        all_v.append(v)
        frame_of.append(f)
    K = np.concatenate(all_k)
    V = np.concatenate(all_v)
    kf = np.concatenate(frame_of)
    for c in (2, 5):
        q = rs.standard_normal((w.n_q, 2, 128))
        o, _ = O.window_attn(cache, q, cos, sin, 3 * c, 3, w.grid_h, w.grid_w,
                             18, 0, -1)
        f, y, x = O.chunk_positions(3 * c, 3, w.grid_h, w.grid_w)
        qr = O.rope_apply(q, cos[f, y, x][:, None], sin[f, y, x][:, None])
        # chunk-causal mask: a query of chunk c sees keys of chunks <= c
        mask = torch.from_numpy((kf[None, :] // 3) <= (f[:, None] // 3))
        for h in range(2):
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(qr[:, h])[None], torch.from_numpy(K[:, h])[None],
                torch.from_numpy(V[:, h])[None], attn_mask=mask[None])[0].numpy()
            assert np.max(np.abs(o[:, h] - ref)) < 1e-12


# ---------------------------------------------------------------- low rank

def test_full_rank_factors_reproduce_dense_projection():
    w = wl.TINY
    A, B = wl.svd_factors_f64(w, wl.TAG_WV, 64)
    W = wl.dense_weight_f64(w, wl.TAG_WV)
    assert np.max(np.abs(A @ B - W)) < 1e-12
    x = wl.bf16_bits_to_f64(wl.activations(w, 0))
    assert np.max(np.abs(O.lowrank_proj(x, A, B) - x @ W)) < 1e-12


@pytest.mark.parametrize("w,r", [(wl.TINY, 16), (wl.WAN_WINDOW, 512)],
                         ids=["tiny", "wan_window"])
def test_factors_eckart_young(w, r):
    """||W - A_r B_r||_F^2 equals the sum of the discarded squared singular
    values, taken from the eigenvalues of W^T W (another route)."""
    A, B = wl.svd_factors_f64(w, wl.TAG_WO, r)
    W = wl.dense_weight_f64(w, wl.TAG_WO)
    ev = np.sort(np.linalg.eigvalsh(W.T @ W))[::-1]
    err = np.sum((W - A @ B) ** 2)
    assert abs(err - ev[r:].sum()) <= 1e-10 * ev[r:].sum()


def test_lowrank_associative_and_brute():
    w = wl.TINY
    rs = np.random.default_rng(11)
    x = rs.standard_normal((9, 64))
    a = rs.standard_normal((64, 16))
    b = rs.standard_normal((16, 40))
    bias = rs.standard_normal(40)
    y = O.lowrank_proj(x, a, b, bias)
    assert np.max(np.abs(y - (x @ (a @ b) + bias))) < 1e-12
    yb = np.array(brute.matmul(brute.matmul(x.tolist(), a.tolist()), b.tolist())) + bias
    assert np.max(np.abs(y - yb)) < 1e-12
    y1 = O.lowrank_proj(x, a)
    assert np.max(np.abs(y1 - np.array(brute.matmul(x.tolist(), a.tolist())))) < 1e-12


# ---------------------------------------------------------------- clip schedule

def test_clip_schedule_forward_counts():
    n = 0
    for line in _golden_lines("clip_forwards.txt"):
        name, chunks, first, later, clean, total, frames = line.split()
        sched = O.clip_schedule(int(chunks), int(first), int(later), clean == "1")
        assert len(sched) == int(total), name
        assert 3 * (max(c for c, _, _ in sched) + 1) == int(frames)
        for c in range(int(chunks)):
            fw = [s for s in sched if s[0] == c]
            assert fw[-1][2] and not any(s[2] for s in fw[:-1])
        n += 1
    assert n == 2


# ---------------------------------------------------------------- sampler

def test_sigma_schedule_table4():
    """Levels and labels as Table 4 prints them (levels as exact fractions,
    labels to the printed digits), from both the oracle and the scalar
    version written by another algebraic route."""
    n = 0
    for line in _golden_lines("sigma_schedule.txt"):
        name, raw, num, den, label = line.split()
        sigma = int(num) / int(den)
        if raw != "-":
            assert abs(float(O.shifted_sigma(int(raw))) - sigma) < 1e-15, name
            assert abs(brute.shifted_sigma(int(raw)) - sigma) < 1e-15, name
            printed = float(label)
            assert abs(float(O.dit_label(sigma)) - printed) <= 0.05 + 1e-12, name
        else:
            assert float(label) == 0.0          # the clean-cache forward's label
        n += 1
    assert n == 6
    # the 2-step schedule is a subset of the printed levels
    assert np.allclose(O.shifted_sigma(O.RAW_STEPS_2), [1.0, 5.0 / 6.0], rtol=0, atol=1e-15)


def _clean_sigma(name):
    for line in _golden_lines("sigma_schedule.txt"):
        f = line.split()
        if f[0] == name:
            return int(f[2]) / int(f[3])
    raise KeyError(name)


def test_sampler_forward_counts_table3():
    """Running the sampler over a clip's seven chunks makes Table 3's forward
    counts: 35 for Self Forcing (four steps per chunk), 23 for UnStep (two per
    later chunk); each chunk ends with the label-0 clean-cache forward."""
    rows = {l.split()[0]: l.split() for l in _golden_lines("clip_forwards.txt")}
    for name, later, s_star in (("self_forcing", O.RAW_STEPS_4, _clean_sigma("clean_sf")),
                                ("unstep", O.RAW_STEPS_2, _clean_sigma("clean_unstep"))):
        _, chunks, first, later_n, _, total, _ = rows[name]
        assert len(later) == int(later_n) and len(O.RAW_STEPS_4) == int(first)
        calls = []
        dit = lambda x, t: (calls.append(t), np.zeros_like(x))[1]
        for c in range(int(chunks)):
            steps = O.RAW_STEPS_4 if c == 0 else later
            before = len(calls)
            O.sample_chunk(dit, np.ones(4), [np.zeros(4)] * len(steps), steps, s_star)
            assert calls[-1] == 0.0 and 0.0 not in calls[before:-1]
        assert len(calls) == int(total), name


def test_sampler_recovers_clean_latent_from_exact_velocity():
    """A model that returns the exact velocity of the latent it is given
    (v = eps - x0 for x = (1 - s) x0 + s eps) makes every step's estimate the
    clean latent, so each chunk comes out as x0 after any schedule, at both
    clean-cache levels; and the levels it sees are Table 4's, in order."""
    rs = np.random.default_rng(3)
    x0 = rs.standard_normal(50)
    for steps, s_star in ((O.RAW_STEPS_4, 0.0), (O.RAW_STEPS_4, 0.02), (O.RAW_STEPS_2, 0.02)):
        levels = [float(s) for s in O.shifted_sigma(steps)] + [s_star]
        seen = []

        def exact(x, t, _lv=levels, _seen=seen):
            s = _lv[len(_seen)]
            _seen.append(s)
            return np.zeros_like(x) if s == 0 else (x - x0) / s

        noises = [rs.standard_normal(50) for _ in steps]
        out, lv, labels = O.sample_chunk(exact, rs.standard_normal(50), noises, steps, s_star)
        assert np.max(np.abs(out - x0)) < 1e-12
        assert lv == levels and labels == [1000.0 * s for s in levels[:-1]] + [0.0]


def test_flow_step_level_endpoints():
    """Table 4's endpoints: level 1 is pure noise and level 0 the clean
    latent, so renoising to 1 gives the draw itself and to 0 the estimate;
    at level 0 the estimate is the latent whatever the velocity."""
    rs = np.random.default_rng(4)
    x, v, eps = (rs.standard_normal(33) for _ in range(3))
    x0, xn = O.flow_step(x, v, eps, 0.625, 1.0)
    assert np.array_equal(xn, eps)
    x0b, xn0 = O.flow_step(x, v, None, 0.625, 0.0)
    assert np.array_equal(x0b, x0) and np.array_equal(xn0, x0)
    assert np.array_equal(O.flow_step(x, v, eps, 0.0, 0.0)[0], x)


def test_sampler_matches_scalar_brute_force():
    """Oracle against the scalar sampler (another route for the mapping and
    the renoising) with a fixed, input-independent velocity per forward."""
    rs = np.random.default_rng(5)
    n = 9
    for steps, s_star in ((O.RAW_STEPS_4, 0.0), (O.RAW_STEPS_2, 0.02), ((1000, 750), 0.02)):
        vs = [rs.standard_normal(n) for _ in range(len(steps) + 1)]
        x_init = rs.standard_normal(n)
        noises = [rs.standard_normal(n) for _ in steps]
        it1, it2 = iter(vs), iter(vs)
        a, la, ta = O.sample_chunk(lambda x, t: next(it1), x_init, noises, steps, s_star)
        b, lb, tb = brute.sample_chunk(lambda x, t: next(it2).tolist(), x_init.tolist(),
                                       [z.tolist() for z in noises], steps, s_star)
        assert np.max(np.abs(a - np.array(b))) < 1e-12
        assert np.allclose(la, lb, rtol=0, atol=1e-15) and np.allclose(ta, tb, rtol=0, atol=1e-12)


# ------------------------------------------------------------------ decoder convolution

def _conv_inputs(T, H, W, Ci, Co, seed):
    rs = np.random.default_rng(seed)
    return rs.standard_normal((T, H, W, Ci)), rs.standard_normal((Co, 3, 3, 3, Ci)), \
        rs.standard_normal(Co)


def test_conv3d_matches_scalar_brute_force():
    """The causal 3-D convolution against scalar loops over the input
    positions each output reads (Ci != Co, so transposed weights show)."""
    x, w, b = _conv_inputs(4, 3, 5, 3, 2, 0)
    got = O.conv3d_causal(x, w, b)
    ref = np.array(brute.conv3d_causal(x.tolist(), w.tolist(), b.tolist()))
    assert np.max(np.abs(got - ref)) < 1e-12


def test_conv3d_delta_kernels_copy_and_shift():
    """A kernel that is the identity at one tap copies the input shifted by
    that tap: the current frame's centre copies it exactly; two frames back
    delays it by two frames with zeros before (causal, no future frame
    read); a corner tap shifts it in space with zeros at the border."""
    T, H, W, C = 5, 4, 6, 3
    x = np.random.default_rng(1).standard_normal((T, H, W, C))

    def delta(dt, dy, dx):
        w = np.zeros((C, 3, 3, 3, C))
        w[:, dt, dy, dx, :] = np.eye(C)
        return w
    assert np.array_equal(O.conv3d_causal(x, delta(2, 1, 1)), x)
    want = np.zeros_like(x)
    want[2:] = x[:-2]
    assert np.array_equal(O.conv3d_causal(x, delta(0, 1, 1)), want)
    # tap (dt, dy, dx) = (2, 0, 2): out[t, y, x] = x[t, y - 1, x + 1]
    want = np.zeros_like(x)
    want[:, 1:, :-1] = x[:, :-1, 1:]
    assert np.array_equal(O.conv3d_causal(x, delta(2, 0, 2)), want)
    # bias only
    b = np.arange(C, dtype=np.float64)
    assert np.array_equal(O.conv3d_causal(x, np.zeros((C, 3, 3, 3, C)), b),
                          np.broadcast_to(b, x.shape))


def test_conv3d_is_causal_in_time():
    """Changing frames t0 and later leaves every earlier output frame as it was."""
    x, w, b = _conv_inputs(6, 3, 4, 4, 5, 2)
    y1 = O.conv3d_causal(x, w, b)
    x2 = x.copy()
    x2[3:] = np.random.default_rng(3).standard_normal(x2[3:].shape)
    y2 = O.conv3d_causal(x2, w, b)
    assert np.array_equal(y1[:3], y2[:3])
    assert not np.allclose(y1[3:], y2[3:])


def test_conv3d_equals_torch_conv3d_on_padded_input():
    """A library special case: torch's conv3d (fp64, CPU) over the input padded
    with two zero frames in front and one zero row / column on each side."""
    import torch
    import torch.nn.functional as F
    x, w, b = _conv_inputs(5, 6, 7, 8, 16, 4)
    xt = torch.from_numpy(x).permute(3, 0, 1, 2)[None]           # [1][Ci][T][H][W]
    xt = F.pad(xt, (1, 1, 1, 1, 2, 0))                            # W, H, then T (front only)
    wt = torch.from_numpy(w).permute(0, 4, 1, 2, 3)               # [Co][Ci][3][3][3]
    ref = F.conv3d(xt, wt, torch.from_numpy(b))[0].permute(1, 2, 3, 0).numpy()
    assert np.max(np.abs(O.conv3d_causal(x, w, b) - ref)) < 1e-11


def test_conv3d_history_is_the_clip_before_the_chunk():
    """Decoding chunk by chunk with the previous chunk's last two input
    frames as history reproduces the whole clip (chunks of three frames,
    zero history for the first), and the history path equals the scalar
    brute force run over history and chunk together, keeping the outputs of
    the chunk's own frames."""
    x, w, b = _conv_inputs(9, 3, 4, 5, 6, 5)
    whole = O.conv3d_causal(x, w, b)
    parts = []
    for c in range(3):
        hist = np.zeros((2,) + x.shape[1:])
        lo = 3 * c - 2
        for k in range(2):
            if lo + k >= 0:
                hist[k] = x[lo + k]
        parts.append(O.conv3d_causal(x[3 * c:3 * c + 3], w, b, history=hist))
    assert np.max(np.abs(np.concatenate(parts) - whole)) < 1e-12
    # zero history is no history
    assert np.array_equal(O.conv3d_causal(x, w, b, history=np.zeros((2,) + x.shape[1:])),
                          O.conv3d_causal(x, w, b))
    # random history against brute force over [history, chunk]
    hist = np.random.default_rng(6).standard_normal((2,) + x.shape[1:])
    xs = x[:3]
    got = O.conv3d_causal(xs, w, b, history=hist)
    ext = np.concatenate([hist, xs])
    ref = np.array(brute.conv3d_causal(ext.tolist(), w.tolist(), b.tolist()))[2:]
    assert np.max(np.abs(got - ref)) < 1e-12
