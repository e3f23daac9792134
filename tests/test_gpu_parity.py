"""GPU parity: the HIP path (through the C ABI) against the CPU fp64 oracle on
the same seeded bf16 inputs.

Bar: bit-exact for slot indexing, window plans, value copies and untouched
slots; keys within one bf16 ulp; bf16 outputs within max-abs 2e-2 and
relative-L2 1e-2 of the fp64 oracle; the fp32 RoPE table within one fp32
ulp.  Small geometries are compared element by element; the full-size
workloads in full for the steady-state chunk the benchmark times and on
sampled query rows elsewhere (attention rows are independent, so a sampled
row is exact for that row).
"""
import math

import numpy as np
import pytest
import torch

import causal_video_diffusion_amd as cvd
from causal_video_diffusion_amd import _binding as B
from causal_video_diffusion_amd import path as P
from causal_video_diffusion_amd import workload as wl
import oracle as O

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
REL_L2 = 1e-2
NAN_BITS = 0x7FC1          # a quiet-NaN sentinel for untouched memory


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load()


def _g(w):
    return cvd.geom(*w.geom_tuple())


def _f64(bits):
    return wl.bf16_bits_to_f64(bits)


def assert_close(got, ref, what, max_abs=MAX_ABS, rel_l2=REL_L2):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, what
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    d = got - ref
    ma = float(np.max(np.abs(d)))
    rl = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))
    print(f"  {what}: max_abs={ma:.3e} rel_l2={rl:.3e}", flush=True)
    assert ma <= max_abs and rl <= rel_l2, f"{what}: max_abs {ma:.3e}, rel_l2 {rl:.3e}"


def _bf16_ulp(x):
    _, e = np.frexp(np.asarray(x, np.float64))
    return np.ldexp(1.0, e - 8)


def _sample_rows(n, k=192, seed=0):
    """First, last (ragged tail) and random rows."""
    if n <= k:
        return np.arange(n)
    rs = np.random.default_rng(seed)
    mid = rs.choice(np.arange(64, n - 64), size=k - 128, replace=False)
    return np.unique(np.concatenate([np.arange(64), mid, np.arange(n - 64, n)]))


# ------------------------------------------------------------------ RoPE table

@pytest.mark.parametrize("name", ["tiny", "mid", "wan_window", "wan_720p"])
def test_rope_table(name):
    w = wl.ALL[name]
    print(f"[rope_table {name}]", flush=True)
    t = P.RopeTable(_g(w), w.n_tab_frames, w.theta)
    torch.cuda.synchronize()
    c_ref, s_ref = O.rope_table(w.n_tab_frames, w.grid_h, w.grid_w, w.pairs, w.theta)
    for got, ref in ((t.cos, c_ref), (t.sin, s_ref)):
        g = got.cpu().numpy().astype(np.float64)
        ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(g - ref) <= ulp + 1e-300)


@pytest.mark.parametrize("first", [9, 1_000_002, 2 ** 31 - 3])
def test_rope_table_from_a_later_frame(first):
    """A chunk's own table (3 frames from `first`, up to the last int32
    frame) against the oracle's, within one fp32 ulp."""
    w = wl.WAN_WINDOW
    print(f"[rope_table from frame {first}]", flush=True)
    t = P.RopeTable(_g(w), 3, w.theta, first_frame=first)
    torch.cuda.synchronize()
    c_ref, s_ref = O.rope_table(3, w.grid_h, w.grid_w, w.pairs, w.theta, first_frame=first)
    for got, ref in ((t.cos, c_ref), (t.sin, s_ref)):
        g = got.cpu().numpy().astype(np.float64)
        ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(g - ref) <= ulp + 1e-300)


# ------------------------------------------------------------------ KV append

def _append_all(w, n_chunks=None, tokens=None):
    """Append every chunk on the GPU and in the oracle; yields per chunk."""
    g = _g(w)
    table = P.RopeTable(g, w.n_tab_frames, w.theta)
    ring = P.Ring(g, w.n_slots, w.n_sink, fill_bits=NAN_BITS)
    cos, sin = O.rope_table(w.n_tab_frames, w.grid_h, w.grid_w, w.pairs, w.theta)
    cache = O.KVCache(w.n_slots, w.n_heads, w.T, w.head_dim)
    for c in range(n_chunks or w.n_chunks):
        kb = wl.chunk_tokens(w, wl.TAG_K, c)
        vb = wl.chunk_tokens(w, wl.TAG_V, c)
        B.ust_kv_append(g, ring.abi, P.to_device_bf16(kb), P.to_device_bf16(vb),
                        table.cos, table.sin, w.n_tab_frames, 3 * c)
        O.kv_append(cache, _f64(kb), _f64(vb), cos, sin, 3 * c, 3, w.grid_h,
                    w.grid_w, w.n_slots, w.n_sink)
        yield c, g, table, ring, cache, (cos, sin), kb, vb


@pytest.mark.parametrize("name", ["tiny", "tiny_wrap", "mid", "mid64", "wan_720p"])
def test_kv_append(name):
    w = wl.ALL[name]
    print(f"[kv_append {name}]", flush=True)
    written = {}
    kin = {}
    for c, g, table, ring, cache, _, kb, vb in _append_all(w):
        for i in range(3):
            written[O.slot_of_frame(3 * c + i, w.n_slots, w.n_sink)] = 3 * c + i
            kin[3 * c + i] = _f64(kb[i * w.T:(i + 1) * w.T]).transpose(1, 0, 2)
        torch.cuda.synchronize()
        gk = ring.host_k()
        gv_raw = P.from_device_bf16(ring.v)
        gv = ring.host_v_natural()
        for s in range(w.n_slots):
            if s not in written:        # untouched slots keep the sentinel, bit for bit
                assert np.all(gk[s] == NAN_BITS) and np.all(gv_raw[s] == NAN_BITS)
                continue
            # The rotation runs in fp32 from fp32 coefficients, then rounds to
            # bf16: the error is one bf16 ulp of the result plus the fp32
            # rounding of the rotation, ~2^-23 (|a| + |b|) for the pair (a, b)
            # (visible when a rotated pair nearly cancels).
            ref_k = cache.k[s]
            got_k = _f64(gk[s])
            src = kin[written[s]]
            pair = np.abs(src[..., 0::2]) + np.abs(src[..., 1::2])
            fp32_err = np.repeat(pair, 2, axis=-1) * 2.0 ** -21
            assert np.all(np.abs(got_k - ref_k) <= _bf16_ulp(ref_k) + fp32_err), f"slot {s} keys"
            assert_close(got_k, ref_k, f"slot {s} keys")
            # values are a bit copy of the appended bf16 values
            f = written[s]
            cc, i = divmod(f, 3)
            src = wl.chunk_tokens(w, wl.TAG_V, cc)[i * w.T:(i + 1) * w.T]
            assert np.array_equal(gv[s], src.transpose(1, 0, 2)), f"slot {s} values"
        # the padding past T in every transposed value row is never written
        assert np.all(gv_raw[..., w.T:] == NAN_BITS)


# ------------------------------------------------------------------ attention

def _attn_gpu(g, w, ring, table, qb, c, n_recent=None, lse=True, n_wg=None, f0=None):
    """ust_window_attn, or ust_window_attn_split over n_wg workgroups (0: one
    per compute unit) with a NaN-filled workspace, so that a merge reading a
    partial result nobody wrote shows up as NaN.  The chunk starts at frame
    f0 (default 3 c)."""
    q = P.to_device_bf16(qb)
    out = torch.empty_like(q)
    l = torch.empty((w.n_heads, w.n_q), dtype=torch.float32, device="cuda") if lse else None
    nr = w.n_recent if n_recent is None else n_recent
    f0 = 3 * c if f0 is None else f0
    if n_wg is None:
        B.ust_window_attn(g, ring.abi, q, table.cos, table.sin, table.n_frames, f0,
                          nr, 0.0, out, l, tab_first_frame=table.first_frame)
    else:
        nbytes = B.ust_window_attn_work_bytes(g, n_wg)
        assert nbytes > 0 and nbytes % 4 == 0
        work = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
        B.ust_window_attn_split(g, ring.abi, q, table.cos, table.sin, table.n_frames, f0,
                                nr, 0.0, out, l, work, n_wg, tab_first_frame=table.first_frame)
    torch.cuda.synchronize()
    return P.from_device_bf16(out), (l.cpu().numpy() if lse else None)


def _attn_case(name, full_chunks=(), rows_per_chunk=192, n_wg=None, w=None, chunks=None,
               q_mult=1.0):
    """Attention of every chunk (or of `chunks`) after its append, against the
    oracle on all rows of small chunks and of `full_chunks`, on sampled rows
    otherwise.  q_mult scales the queries (a power of two keeps them exact in
    bf16) to make the softmax peaky."""
    w = wl.ALL[name] if w is None else w
    for c, g, table, ring, cache, (cos, sin), kb, vb in _append_all(w):
        if chunks is not None and c not in chunks:
            continue
        qb = wl.chunk_tokens(w, wl.TAG_Q, c)
        if q_mult != 1.0:
            qb = wl.f32_to_bf16_bits((_f64(qb) * q_mult).astype(np.float32))
        rows = np.arange(w.n_q) if (c in full_chunks or w.n_q <= 512) else \
            _sample_rows(w.n_q, rows_per_chunk, seed=c)
        mode = "" if n_wg is None else f" split over {n_wg or 'all CUs'}"
        print(f"[attn {name}{mode} chunk {c}: {len(rows)} rows]", flush=True)
        o_gpu, lse_gpu = _attn_gpu(g, w, ring, table, qb, c, n_wg=n_wg)
        o_ref, lse_ref = O.window_attn(cache, _f64(qb), cos, sin, 3 * c, 3, w.grid_h,
                                       w.grid_w, w.n_slots, w.n_sink, w.n_recent,
                                       rows=rows)
        # The bar's absolute part is for outputs of unit scale (the workloads'
        # outputs stay well below 1).  Peaky queries give outputs up to ~3.4,
        # where one bf16 ulp is 2^-6 and the bf16 rounding of each rotated
        # query element (2^-9 relative) moves scores of ~15 by ~0.03: the
        # absolute part then scales with the largest output.
        o_scale = max(1.0, float(np.max(np.abs(o_ref)))) if q_mult != 1.0 else 1.0
        assert_close(_f64(o_gpu[rows]), o_ref, f"{name} chunk {c} O", max_abs=MAX_ABS * o_scale)
        assert_close(lse_gpu[:, rows], lse_ref, f"{name} chunk {c} lse", max_abs=2e-2 * q_mult,
                     rel_l2=1e-3)


@pytest.mark.parametrize("name", ["tiny", "tiny_wrap", "mid", "mid64"])
def test_window_attn_full_compare(name):
    _attn_case(name)


def test_window_attn_wan_window():
    # chunk 5 is the steady-state chunk the benchmark times: compared in full
    _attn_case("wan_window", full_chunks=(5,))


def test_window_attn_wan_window_peaky():
    # queries x4: scores four times wider, so the softmax is far from uniform
    # (a stress input beside the random-weight workload); chunk 5 in full.
    # A CPU model of the kernel's roundings (bf16 rotated query, bf16 cached
    # key, bf16 probabilities, bf16 output) puts max-abs near 3e-2 here, at
    # outputs up to 3.4: the absolute bar is scaled by the largest output
    _attn_case("wan_window", full_chunks=(5,), chunks=(5,), q_mult=4.0)


def test_window_attn_wan_full_cache():
    # the last chunk (32760 keys, every prior frame) in full, the others sampled
    _attn_case("wan_full", full_chunks=(6,))


def test_window_attn_wan_720p():
    _attn_case("wan_720p")


# The key-split schedule: every unit (head, 256-query tile) may be divided
# between workgroups and merged afterwards.  n_wg = 0 is one workgroup per
# compute unit (the benchmark's launch); the small counts make units span
# several workgroups and workgroups span several units, with boundaries
# inside frames and inside the ragged last key tile.
@pytest.mark.parametrize("n_wg", [0, 1, 2, 5, 37])
@pytest.mark.parametrize("name", ["tiny", "tiny_wrap", "mid", "mid64"])
def test_window_attn_split_full_compare(name, n_wg):
    _attn_case(name, n_wg=n_wg)


def test_window_attn_split_wan_window():
    _attn_case("wan_window", full_chunks=(5,), n_wg=0)


# Head size 64 at full size: the Wan frame grid and window with 24 heads of
# 64 (hidden 1536), so the D = 64 tiles straddle 1560-token frames over a
# 12-frame window, on sampled rows of every chunk, both schedules.
WAN_WINDOW_D64 = wl.WAN_WINDOW.replace(name="wan_window_d64", n_heads=24, head_dim=64,
                                       pairs=(12, 10, 10))


@pytest.mark.parametrize("n_wg", [None, 0])
def test_window_attn_d64_wan_grid(n_wg):
    _attn_case("wan_window_d64", n_wg=n_wg, rows_per_chunk=160, w=WAN_WINDOW_D64)


def test_window_attn_split_wan_720p():
    # 516 units: with one workgroup per CU each workgroup spans two or three units
    _attn_case("wan_720p", n_wg=0)


def test_window_attn_split_matches_unsplit():
    """Where no unit is split (n_wg = units: one each; units / 2: two whole
    units per workgroup, run one after the other) the split kernel does the
    unsplit arithmetic exactly: bit-identical outputs.  Where units are split,
    each part starts its own reference max, so the bf16 probabilities round
    differently (both schedules stay within the oracle bar, tested above);
    the log-sum-exp uses no bf16 step and agrees to fp32 rounding."""
    w = wl.MID
    units = -(-w.n_q // 256) * w.n_heads
    for c, g, table, ring, cache, _, kb, vb in _append_all(w):
        qb = wl.chunk_tokens(w, wl.TAG_Q, c)
        o1, l1 = _attn_gpu(g, w, ring, table, qb, c)
        for n_wg in (units, units // 2):
            o2, l2 = _attn_gpu(g, w, ring, table, qb, c, n_wg=n_wg)
            assert np.array_equal(o1, o2) and np.array_equal(l1, l2), f"chunk {c} n_wg {n_wg}"
        for n_wg in (0, 3):
            _, l2 = _attn_gpu(g, w, ring, table, qb, c, n_wg=n_wg)
            assert np.allclose(l1, l2, rtol=1e-5, atol=1e-5), \
                f"chunk {c} n_wg {n_wg}: lse max diff {np.abs(l1 - l2).max():.3e}"


def test_window_edge_cases():
    """n_recent = 0 (sinks + chunk), n_recent past the start (= full causal),
    no sinks, and the chunk-0 window (only the chunk itself)."""
    base = wl.MID
    for w in (base.replace(n_recent=0), base.replace(n_recent=30, n_slots=18),
              base.replace(n_sink=0, n_slots=9), base.replace(n_recent=-1, n_slots=18)):
        print(f"[edge n_sink={w.n_sink} n_recent={w.n_recent} n_slots={w.n_slots}]", flush=True)
        for c, g, table, ring, cache, (cos, sin), kb, vb in _append_all(w):
            qb = wl.chunk_tokens(w, wl.TAG_Q, c)
            o_gpu, _ = _attn_gpu(g, w, ring, table, qb, c, lse=False)
            o_ref, _ = O.window_attn(cache, _f64(qb), cos, sin, 3 * c, 3, w.grid_h,
                                     w.grid_w, w.n_slots, w.n_sink, w.n_recent)
            assert_close(_f64(o_gpu), o_ref, f"edge chunk {c}")


@pytest.mark.parametrize("head_dim,pairs", [(64, (12, 10, 10)), (128, (22, 21, 21))])
def test_window_attn_longest_window_short_frames(head_dim, pairs):
    """The longest window the library accepts (128 frames: 2 sinks, 123
    recent, 3 current) over 24-token frames, so every 64-key tile spans three
    or four frames and every tile load takes the per-lane frame lookup; the
    ring (130 slots) has wrapped.  Chunk 20 (the whole history, 63 frames)
    and chunk 42 (exactly 128 frames) are compared row by row."""
    w = wl.TINY.replace(name=f"longwin{head_dim}", wid=20 + head_dim // 64, n_heads=2,
                        head_dim=head_dim, pairs=pairs, n_chunks=43, n_slots=130,
                        n_sink=2, n_recent=123, n_tab_frames=129)
    for c, g, table, ring, cache, (cos, sin), kb, vb in _append_all(w):
        if c not in (20, 42):
            continue
        frames, _ = B.ust_window_plan(g, ring.abi, 3 * c, w.n_recent)
        assert len(frames) == (63 if c == 20 else 128)
        print(f"[longest window D={head_dim} chunk {c}: {len(frames)} frames]", flush=True)
        qb = wl.chunk_tokens(w, wl.TAG_Q, c)
        o_ref, lse_ref = O.window_attn(cache, _f64(qb), cos, sin, 3 * c, 3, w.grid_h,
                                       w.grid_w, w.n_slots, w.n_sink, w.n_recent)
        for n_wg in (None, 0, 7):
            o_gpu, lse_gpu = _attn_gpu(g, w, ring, table, qb, c, n_wg=n_wg)
            assert_close(_f64(o_gpu), o_ref, f"longest window chunk {c} n_wg {n_wg} O")
            assert_close(lse_gpu, lse_ref, f"longest window chunk {c} n_wg {n_wg} lse",
                         max_abs=2e-2, rel_l2=1e-3)


def test_streaming_far_past_one_clip():
    """A stream of 40 chunks (frames 0-119) through a 12-slot ring (3 pinned
    sinks + 9 cycling slots, so the cycling part wraps 13 times) with a RoPE
    table over all 120 frames: the window keeps the 3 sink frames and the 6
    most recent ones at any length, and keys keep their absolute positions.
    Chunks 10, 25 and 39 are compared in full, on both schedules."""
    w = wl.MID.replace(name="mid_stream", wid=30, n_chunks=40, n_tab_frames=120)
    for c, g, table, ring, cache, (cos, sin), kb, vb in _append_all(w):
        if c not in (10, 25, 39):
            continue
        frames, slots = B.ust_window_plan(g, ring.abi, 3 * c, w.n_recent)
        assert frames == [0, 1, 2] + list(range(3 * c - 6, 3 * c + 3))
        assert slots == [0, 1, 2] + [3 + (f - 3) % 9 for f in range(3 * c - 6, 3 * c + 3)]
        qb = wl.chunk_tokens(w, wl.TAG_Q, c)
        o_ref, lse_ref = O.window_attn(cache, _f64(qb), cos, sin, 3 * c, 3, w.grid_h,
                                       w.grid_w, w.n_slots, w.n_sink, w.n_recent)
        for n_wg in (None, 0):
            print(f"[stream chunk {c} (frames {3 * c}-{3 * c + 2}) n_wg {n_wg}]", flush=True)
            o_gpu, lse_gpu = _attn_gpu(g, w, ring, table, qb, c, n_wg=n_wg)
            assert_close(_f64(o_gpu), o_ref, f"stream chunk {c} O")
            assert_close(lse_gpu, lse_ref, f"stream chunk {c} lse", max_abs=2e-2, rel_l2=1e-3)


def test_stream_with_chunk_tables_equals_full_table():
    """A stream of 8 chunks through a 12-slot ring, once with one table over
    all 24 frames and once with a 3-frame table rebuilt in place for each
    chunk: ring, outputs and log-sum-exps agree bit for bit, for the append,
    both attention schedules and the fused projection's epilogue."""
    w = wl.MID.replace(name="mid_tables", wid=31, n_chunks=8, n_tab_frames=24)
    g = _g(w)
    full = P.RopeTable(g, w.n_tab_frames, w.theta)
    own = P.RopeTable(g, 3, w.theta)
    rings = [P.Ring(g, w.n_slots, w.n_sink, fill_bits=NAN_BITS) for _ in range(2)]
    rs = np.random.default_rng(71)
    hidden = 256
    w_qkv = P.to_device_bf16(wl.f32_to_bf16_bits(
        rs.standard_normal((3 * w.n_heads * w.head_dim, hidden)) * hidden ** -0.5))
    for c in range(w.n_chunks):
        own.rebuild(3 * c)
        kb = P.to_device_bf16(wl.chunk_tokens(w, wl.TAG_K, c))
        vb = P.to_device_bf16(wl.chunk_tokens(w, wl.TAG_V, c))
        qb = wl.chunk_tokens(w, wl.TAG_Q, c)
        res = []
        for ring, table in zip(rings, (full, own)):
            B.ust_kv_append(g, ring.abi, kb, vb, table.cos, table.sin, table.n_frames, 3 * c,
                            tab_first_frame=table.first_frame)
            outs = [_attn_gpu(g, w, ring, table, qb, c, n_wg=n_wg) for n_wg in (None, 0)]
            res.append((P.from_device_bf16(ring.k), P.from_device_bf16(ring.v), outs))
        print(f"[chunk tables: chunk {c}]", flush=True)
        (k1, v1, o1), (k2, v2, o2) = res
        assert np.array_equal(k1, k2) and np.array_equal(v1, v2), f"chunk {c} ring"
        for (a, la), (b, lb) in zip(o1, o2):
            assert np.array_equal(a, b) and np.array_equal(la, lb), f"chunk {c} attention"
    # the fused projection's epilogue rotates K with the same rows
    x = P.to_device_bf16(wl.f32_to_bf16_bits(rs.standard_normal((w.n_q, hidden))))
    c = w.n_chunks - 1
    qs = []
    for ring, table in zip(rings, (full, own)):
        q_out = torch.empty((w.n_q, w.n_heads * w.head_dim), dtype=torch.bfloat16, device="cuda")
        B.ust_qkv_append(g, ring.abi, x, w_qkv, hidden, table.cos, table.sin, table.n_frames,
                         3 * c, q_out, tab_first_frame=table.first_frame)
        qs.append(q_out)
    torch.cuda.synchronize()
    assert torch.equal(qs[0].view(torch.int16), qs[1].view(torch.int16))
    for a, b in ((rings[0].k, rings[1].k), (rings[0].v, rings[1].v)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_stream_a_million_frames_in():
    """A stream a million frames in, with a table of the chunk's own three
    frames for each chunk: the sink chunk (frames 0-2, its own table from
    frame 0) and the chunks at frames F-6, F-3 and F (F = 1,000,002), then
    the attention of the chunk at F on both schedules, against the oracle
    fed the same tables, in full."""
    w = wl.MID
    g = _g(w)
    F = 1_000_002
    ring = P.Ring(g, w.n_slots, w.n_sink, fill_bits=NAN_BITS)
    table = P.RopeTable(g, 3, w.theta)
    cache = O.KVCache(w.n_slots, w.n_heads, w.T, w.head_dim)
    for c, f0 in enumerate((0, F - 6, F - 3, F)):
        table.rebuild(f0)
        cos, sin = O.rope_table(3, w.grid_h, w.grid_w, w.pairs, w.theta, first_frame=f0)
        kb = wl.chunk_tokens(w, wl.TAG_K, c)
        vb = wl.chunk_tokens(w, wl.TAG_V, c)
        B.ust_kv_append(g, ring.abi, P.to_device_bf16(kb), P.to_device_bf16(vb), table.cos,
                        table.sin, 3, f0, tab_first_frame=f0)
        O.kv_append(cache, _f64(kb), _f64(vb), cos, sin, f0, 3, w.grid_h, w.grid_w,
                    w.n_slots, w.n_sink, tab_first=f0)
    frames, slots = B.ust_window_plan(g, ring.abi, F, w.n_recent)
    assert frames == [0, 1, 2] + list(range(F - 6, F + 3))
    assert slots == [O.slot_of_frame(f, w.n_slots, w.n_sink) for f in frames]
    qb = wl.chunk_tokens(w, wl.TAG_Q, 3)
    o_ref, lse_ref = O.window_attn(cache, _f64(qb), cos, sin, F, 3, w.grid_h, w.grid_w,
                                   w.n_slots, w.n_sink, w.n_recent, tab_first=F)
    for n_wg in (None, 0):
        print(f"[stream at frame {F} n_wg {n_wg}]", flush=True)
        o_gpu, lse_gpu = _attn_gpu(g, w, ring, table, qb, 3, n_wg=n_wg, f0=F)
        assert_close(_f64(o_gpu), o_ref, f"frame {F} O")
        assert_close(lse_gpu, lse_ref, f"frame {F} lse", max_abs=2e-2, rel_l2=1e-3)


def test_nan_outside_window_and_determinism():
    """Poisoning every slot outside the window (and the value padding) with NaN
    leaves the output bit-identical; two runs agree bit for bit.  Both
    schedules (the split one over 5 workgroups)."""
    w = wl.MID
    for c, g, table, ring, cache, _, kb, vb in _append_all(w):
        qb = wl.chunk_tokens(w, wl.TAG_Q, c)
        o1, l1 = _attn_gpu(g, w, ring, table, qb, c)
        o2, l2 = _attn_gpu(g, w, ring, table, qb, c)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
        s1, sl1 = _attn_gpu(g, w, ring, table, qb, c, n_wg=5)
        s2, sl2 = _attn_gpu(g, w, ring, table, qb, c, n_wg=5)
        assert np.array_equal(s1, s2) and np.array_equal(sl1, sl2)
        _, slots = O.window_slots(3 * c, 3, w.n_sink, w.n_recent, w.n_slots)
        keep_k = ring.k[slots].clone()
        keep_v = ring.v[slots].clone()
        ring.fill(NAN_BITS)
        ring.k[slots] = keep_k
        ring.v[slots] = keep_v
        ring.v[..., w.T:].view(torch.int16).fill_(NAN_BITS)
        o3, l3 = _attn_gpu(g, w, ring, table, qb, c)
        assert np.array_equal(o1, o3) and np.array_equal(l1, l3), f"chunk {c}"
        s3, sl3 = _attn_gpu(g, w, ring, table, qb, c, n_wg=5)
        assert np.array_equal(s1, s3) and np.array_equal(sl1, sl3), f"chunk {c} split"
        if c == 3:
            break


def test_window_attn_scores_far_above_the_first_tile():
    """Keys of chunks 0, 1, 2, 3 scaled by 1, 4, 16, 64 (powers of two: exact
    in bf16), so that along the window later tiles score far above the
    reference max set on the first one: by up to ~2^4 (large probabilities,
    no rescale), ~2^6 (a running sum past 2^64: rescale with finite values)
    and ~2^8 (exp2 overflows to infinity: rescale from the raw scores).
    Both schedules, so segments also start inside the scaled chunks.

    Scores this large are only as exact as the bf16 query fragments (each
    rotated, scaled query element is rounded to bf16: relative error at most
    2^-8, bf16 having 8 significant bits), so the checks are ones that
    rounding cannot disturb:
    - every window value row of a head is the same row v, so O = v whatever
      the weights: the kernel's sum bf16(p) v / sum p (fp32) is within
      2^-8 |v| of v, less than one bf16 ulp of v, so the bf16 output is
      within one ulp of v (and finite: no infinity or NaN from an overflowed
      tile leaks through);
    - the log-sum-exp, which counts every tile's mass against its reference,
      moves with the scores by at most the largest score error,
      2^-8 sum_d |q_d k_d| scale (1% added for the fp32 rotation and
      accumulation): that bound, per query row."""
    w = wl.MID
    g = _g(w)
    table = P.RopeTable(g, w.n_tab_frames, w.theta)
    ring = P.Ring(g, w.n_slots, w.n_sink, fill_bits=NAN_BITS)
    cos, sin = O.rope_table(w.n_tab_frames, w.grid_h, w.grid_w, w.pairs, w.theta)
    cache = O.KVCache(w.n_slots, w.n_heads, w.T, w.head_dim)
    scale = 1.0 / math.sqrt(w.head_dim)
    vrow = wl.chunk_tokens(w, wl.TAG_V, 0)[:1]                 # [1][H][D]
    vb = np.repeat(vrow, w.n_q, axis=0)
    v = _f64(vrow)[0]                                          # [H][D]
    for c, e in enumerate((0, 2, 4, 6)):
        kb = wl.f32_to_bf16_bits((_f64(wl.chunk_tokens(w, wl.TAG_K, c)) * 2.0 ** e).astype(np.float32))
        B.ust_kv_append(g, ring.abi, P.to_device_bf16(kb), P.to_device_bf16(vb),
                        table.cos, table.sin, w.n_tab_frames, 3 * c)
        O.kv_append(cache, _f64(kb), _f64(vb), cos, sin, 3 * c, 3, w.grid_h,
                    w.grid_w, w.n_slots, w.n_sink)
        qb = wl.chunk_tokens(w, wl.TAG_Q, c)
        o_ref, lse_ref = O.window_attn(cache, _f64(qb), cos, sin, 3 * c, 3, w.grid_h,
                                       w.grid_w, w.n_slots, w.n_sink, w.n_recent)
        f, y, x = O.chunk_positions(3 * c, 3, w.grid_h, w.grid_w)
        qr = np.abs(O.rope_apply(_f64(qb), cos[f, y, x][:, None, :], sin[f, y, x][:, None, :]))
        _, slots = O.window_slots(3 * c, 3, w.n_sink, w.n_recent, w.n_slots)
        bound = np.empty((w.n_heads, w.n_q))
        for h in range(w.n_heads):
            kabs = np.abs(cache.k[slots][:, h].reshape(-1, w.head_dim))
            bound[h] = 1.01 * 2.0 ** -8 * scale * (qr[:, h] @ kabs.T).max(axis=1)
        for n_wg in (None, 5, 37):
            print(f"[scaled keys chunk {c} (x{2 ** e}) n_wg {n_wg}]", flush=True)
            o_gpu, lse_gpu = _attn_gpu(g, w, ring, table, qb, c, n_wg=n_wg)
            o = _f64(o_gpu)
            assert_close(o, o_ref, f"scaled chunk {c} O")
            assert np.all(np.abs(o - v) <= _bf16_ulp(v)), f"chunk {c}: O more than one ulp from v"
            err = np.abs(lse_gpu - lse_ref)
            print(f"  lse: max err {err.max():.3e}, max err / bound {(err / bound).max():.3f}",
                  flush=True)
            assert np.all(err <= bound + 1e-4 * (1 + np.abs(lse_ref))), f"chunk {c} lse"


# Dimensions 38..43 are the frame-axis pairs 19..21 (of 22 at head size 128),
# whose frequencies are at most 10^4^(-19/22) ~ 3.5e-4 rad per frame: the
# RoPE of a vector living there depends on the frame only, and turns it by
# less than 0.007 rad over the table (so its cosine part rounds to the same
# bf16 value in every frame).
_BIG = slice(38, 44)


def _with_big_part(bits, coef):
    """Zero dimensions 38..43 and put `coef` in their even elements (the first
    element of each of those three rotation pairs)."""
    x = _f64(bits).copy()
    x[..., _BIG] = 0.0
    x[..., _BIG.start:_BIG.stop:2] = coef
    return wl.f32_to_bf16_bits(x.astype(np.float32))


@pytest.mark.parametrize("where,offset", [("current", 20.0), ("current", 48.0),
                                          ("current", 100.0), ("recent", 48.0),
                                          ("recent", 100.0), ("sink", -100.0)])
def test_window_attn_rescale_path_random_values(where, offset):
    """The lazy-rescale path against the oracle element by element, with
    distinct random value rows.  Every query carries gamma = 16 on the three
    frame-axis pairs 19..21, and the keys of one chunk carry beta there
    (others 0), so that chunk's keys score `offset` (natural units) above
    the rest, and all keys of a frame get the same offset to fp32 rounding:
    their frame-axis RoPE is the same, and the bf16 rounding of a query's
    large part shifts them all alike.  Inside the chunk the weights follow
    the random parts, as accurate as in the plain workload.
      current, 20: probabilities up to 2^29 against the first tile's
        reference; no rescale;
      current / recent, 48: running sums past 2^64: a rescale with finite
        values, the tile redone (recent: mid-window, later tiles fall far
        below the new reference);
      current / recent, 100: exp2 overflows to infinity: the rescale from
        the raw scores;
      sink, -100: the window's first tile (the sink frames) scores ~144
        below every later key (log2 units), so its reference is ~144 below
        the scores that follow.
    Chunk 5 of the mid workload (window: sinks 0-2, recent 9-14, current
    15-17), on both schedules (the split one over 5, 37 and all
    workgroups, so segments also start inside the offset chunk).  The
    log-sum-exp carries the bf16 rounding of the queries' large part, so
    it is held to that bound, per row."""
    w = wl.MID
    c_att = 5
    big_chunk = {"current": 5, "recent": 3, "sink": 0}[where]
    gamma = 16.0
    scale = 1.0 / math.sqrt(w.head_dim)
    beta = float(wl.bf16_bits_to_f64(wl.f32_to_bf16_bits(
        np.array([offset / (3 * gamma * scale)], np.float32)))[0])
    g = _g(w)
    table = P.RopeTable(g, w.n_tab_frames, w.theta)
    ring = P.Ring(g, w.n_slots, w.n_sink, fill_bits=NAN_BITS)
    cos, sin = O.rope_table(w.n_tab_frames, w.grid_h, w.grid_w, w.pairs, w.theta)
    cache = O.KVCache(w.n_slots, w.n_heads, w.T, w.head_dim)
    for c in range(c_att + 1):
        kb = _with_big_part(wl.chunk_tokens(w, wl.TAG_K, c), beta if c == big_chunk else 0.0)
        vb = wl.chunk_tokens(w, wl.TAG_V, c)
        B.ust_kv_append(g, ring.abi, P.to_device_bf16(kb), P.to_device_bf16(vb),
                        table.cos, table.sin, w.n_tab_frames, 3 * c)
        O.kv_append(cache, _f64(kb), _f64(vb), cos, sin, 3 * c, 3, w.grid_h,
                    w.grid_w, w.n_slots, w.n_sink)
    qb = _with_big_part(wl.chunk_tokens(w, wl.TAG_Q, c_att), gamma)
    o_ref, lse_ref = O.window_attn(cache, _f64(qb), cos, sin, 3 * c_att, 3, w.grid_h,
                                   w.grid_w, w.n_slots, w.n_sink, w.n_recent)
    # lse bound: each rotated, scaled query element is rounded to bf16
    # (relative error <= 2^-9), so a score moves by at most
    # 2^-9 scale sum_d |q'_d k_d|; 2^-8 and 1% cover the fp32 rotation
    f, y, x = O.chunk_positions(3 * c_att, 3, w.grid_h, w.grid_w)
    qr = np.abs(O.rope_apply(_f64(qb), cos[f, y, x][:, None, :], sin[f, y, x][:, None, :]))
    _, slots = O.window_slots(3 * c_att, 3, w.n_sink, w.n_recent, w.n_slots)
    bound = np.empty((w.n_heads, w.n_q))
    for h in range(w.n_heads):
        kabs = np.abs(cache.k[slots][:, h].reshape(-1, w.head_dim))
        bound[h] = 1.01 * 2.0 ** -8 * scale * (qr[:, h] @ kabs.T).max(axis=1)
    for n_wg in (None, 0, 5, 37):
        print(f"[rescale path: {where} chunk offset {offset:+g}, n_wg {n_wg}]", flush=True)
        o_gpu, lse_gpu = _attn_gpu(g, w, ring, table, qb, c_att, n_wg=n_wg)
        assert_close(_f64(o_gpu), o_ref, f"rescale {where} {offset:+g} n_wg {n_wg} O")
        err = np.abs(lse_gpu - lse_ref)
        assert np.all(err <= bound + 1e-4 * (1 + np.abs(lse_ref))), \
            f"lse: max err {err.max():.3e}, max err / bound {(err / bound).max():.3f}"


def test_v_one_gives_one_and_k_zero_gives_mean():
    w = wl.MID
    g = _g(w)
    table = P.RopeTable(g, w.n_tab_frames, w.theta)
    ring = P.Ring(g, w.n_slots, w.n_sink, fill_bits=NAN_BITS)
    ones = np.full((w.n_q, w.n_heads, w.head_dim), 0x3F80, np.uint16)
    zeros = np.zeros((w.n_q, w.n_heads, w.head_dim), np.uint16)
    for c in range(4):
        kb = wl.chunk_tokens(w, wl.TAG_K, c)
        B.ust_kv_append(g, ring.abi, P.to_device_bf16(kb), P.to_device_bf16(ones),
                        table.cos, table.sin, w.n_tab_frames, 3 * c)
    qb = wl.chunk_tokens(w, wl.TAG_Q, 3)
    q4 = wl.f32_to_bf16_bits((_f64(qb) * 4).astype(np.float32))   # peaky scores
    o, _ = _attn_gpu(g, w, ring, table, q4, 3)
    assert np.max(np.abs(_f64(o) - 1.0)) <= 2 ** -7
    # K = 0: uniform weights, O = mean of the window's values, lse = ln(keys)
    ring2 = P.Ring(g, w.n_slots, w.n_sink, fill_bits=NAN_BITS)
    vs = []
    for c in range(4):
        vb = wl.chunk_tokens(w, wl.TAG_V, c)
        vs.append(_f64(vb))
        B.ust_kv_append(g, ring2.abi, P.to_device_bf16(zeros), P.to_device_bf16(vb),
                        table.cos, table.sin, w.n_tab_frames, 3 * c)
    o, lse = _attn_gpu(g, w, ring2, table, qb, 3)
    frames, _ = O.window_slots(9, 3, w.n_sink, w.n_recent, w.n_slots)
    allv = np.concatenate(vs)                      # frames 0..11, [n][H][D]
    sel = np.concatenate([allv[f * w.T:(f + 1) * w.T] for f in frames])
    mean = sel.mean(axis=0)                        # [H][D]
    assert_close(_f64(o), np.broadcast_to(mean, o.shape), "K=0 mean", max_abs=1e-2)
    assert np.max(np.abs(lse - math.log(len(frames) * w.T))) < 1e-4


# ------------------------------------------------------------------ sampler
# One step in fp32: x0 = x - sigma v (one rounding), x_next = fp32(1 - s')
# x0 rounded, then + s' eps in one fma; the oracle is fp64 with the same fp32
# levels.  Each rounding is at most 2^-24 relative, so per element
# |error| <= 2^-21 (|x| + |sigma v| + |s' eps|), generously.

def _flow_bound(x, sv, se):
    return 2.0 ** -21 * (np.abs(x) + np.abs(sv) + np.abs(se)) + 1e-30


@pytest.mark.parametrize("n", [1, 3, 4, 5, 1001, 3 * 16 * 60 * 104])
def test_flow_step_matches_oracle(n):
    """Against the fp64 oracle at Table 4's levels (and the clean-cache ones),
    sizes with ragged tails up to the Wan chunk latent; the exact cases bit
    for bit; in place equal to out of place; nothing past n written."""
    print(f"[flow_step n={n}]", flush=True)
    rs = np.random.default_rng(n)
    x = (rs.standard_normal(n) * 2).astype(np.float32)
    vb = wl.f32_to_bf16_bits(rs.standard_normal(n).astype(np.float32))
    eps = rs.standard_normal(n).astype(np.float32)
    v = _f64(vb)
    xd, vd, ed = torch.from_numpy(x).cuda(), P.to_device_bf16(vb), torch.from_numpy(eps).cuda()
    for s, sn in ((1.0, 0.9375), (5 / 6, 0.625), (0.625, 0.02), (0.02, 0.0), (0.0, 0.0),
                  (0.5, 1.0)):
        s32, sn32 = float(np.float32(s)), float(np.float32(sn))
        x0 = torch.full((n + 8,), float("nan"), device="cuda")
        xn = torch.full((n + 8,), float("nan"), device="cuda")
        B.ust_flow_step(xd, vd, ed, s32, sn32, x0, xn, n)
        torch.cuda.synchronize()
        g0, gn = x0.cpu().numpy(), xn.cpu().numpy()
        assert np.isnan(g0[n:]).all() and np.isnan(gn[n:]).all(), "wrote past n"
        g0, gn = g0[:n], gn[:n]
        r0, rn = O.flow_step(x, v, eps, s32, sn32)
        assert np.all(np.abs(g0 - r0) <= _flow_bound(x, s32 * v, 0)), f"x0 {s}->{sn}"
        assert np.all(np.abs(gn - rn) <= _flow_bound(x, s32 * v, sn32 * eps)), f"x_next {s}->{sn}"
        if sn == 0.0:
            assert np.array_equal(gn, g0)
        if s == 0.0:
            assert np.array_equal(g0, x)
        if sn == 1.0:
            assert np.array_equal(gn, eps)
        # in place: the latent overwritten by its successor
        xi = xd.clone()
        B.ust_flow_step(xi, vd, ed, s32, sn32, None, xi, n)
        torch.cuda.synchronize()
        assert np.array_equal(xi.cpu().numpy(), gn), f"in place {s}->{sn}"


@pytest.mark.parametrize("name", ["tiny", "wan_window"])
def test_sample_chunk_matches_oracle(name):
    """Whole chunks of the sampler against the oracle's: Self Forcing's four
    steps with sigma* = 0, UnStep's two with sigma* = 0.02, and four with
    0.02, each with stand-in velocities drawn per forward (the same on both
    sides).  Errors add up over the forwards: per element at most
    (forwards) 2^-21 times the sum of every input's magnitude there."""
    w = wl.ALL[name]
    cases = ((P.SAMPLER_RAW_STEPS_4, 0.0), (P.SAMPLER_RAW_STEPS_2, 0.02),
             (P.SAMPLER_RAW_STEPS_4, 0.02))
    for c, (steps, s_star) in enumerate(cases):
        print(f"[sample_chunk {name} steps {steps} sigma* {s_star}]", flush=True)
        x_init = wl.latent_noise(w, c, 0)
        noises = [wl.latent_noise(w, c, i + 1) for i in range(len(steps))]
        vels = [wl.stand_in_velocity(w, c, f) for f in range(len(steps) + 1)]
        x = torch.from_numpy(x_init.copy()).cuda()
        it = iter([P.to_device_bf16(b) for b in vels])
        got, lv, lb = P.sample_chunk(lambda xx, t: next(it), x,
                                     [torch.from_numpy(z).cuda() for z in noises], steps, s_star)
        torch.cuda.synchronize()
        it2 = iter(vels)
        ref, lv2, lb2 = O.sample_chunk(lambda xx, t: _f64(next(it2)), x_init, noises, steps,
                                       s_star)
        assert np.allclose(lv, lv2, rtol=1e-15, atol=0) and np.allclose(lb, lb2, rtol=1e-15, atol=0)
        assert len(lv) == len(steps) + 1 and lb[-1] == 0.0
        mag = np.abs(x_init.astype(np.float64)) + sum(np.abs(_f64(b)) for b in vels) + \
            sum(np.abs(z.astype(np.float64)) for z in noises)
        err = np.abs(got.cpu().numpy() - ref)
        assert np.all(err <= (len(steps) + 1) * 2.0 ** -21 * mag + 1e-30), \
            f"max err {err.max():.3e}"


def test_sampler_graph_replay_matches_eager():
    """Three chunks of the UnStep sampler (4 + 1, 2 + 1, 2 + 1 flow steps)
    captured in a HIP graph (kernel nodes only) and replayed three times,
    with a reset of the latents and other eager work between replays: each
    replay equals the eager run bit for bit."""
    w = wl.WAN_WINDOW
    n = int(np.prod(wl.latent_shape(w)))
    plan = []
    for c in range(3):
        steps = P.SAMPLER_RAW_STEPS_4 if c == 0 else P.SAMPLER_RAW_STEPS_2
        lv, _ = B.ust_sigma_schedule(list(steps))
        plan += [(c, i, s, lv[i + 1] if i + 1 < len(lv) else 0.02) for i, s in enumerate(lv)]
        plan.append((c, len(lv), 0.02, 0.0))
    lat0 = [torch.from_numpy(wl.latent_noise(w, c, 0)).cuda() for c in range(3)]
    lat = [t.clone() for t in lat0]
    noise = [[torch.from_numpy(wl.latent_noise(w, c, i + 1)).cuda() for i in range(4)]
             for c in range(3)]
    vel = [[P.to_device_bf16(wl.stand_in_velocity(w, c, f)) for f in range(5)] for c in range(3)]

    def clip():
        for c, f, sg, sn in plan:
            B.ust_flow_step(lat[c], vel[c][f], noise[c][f] if sn != 0 else None, sg, sn, None,
                            lat[c], n)

    def reset():
        for t, t0 in zip(lat, lat0):
            t.copy_(t0)

    reset()
    clip()
    torch.cuda.synchronize()
    ref = [t.cpu().numpy() for t in lat]
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        clip()
    stream.wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        clip()
    for r in range(3):
        print(f"[sampler graph replay {r}]", flush=True)
        reset()
        junk = torch.randn(1 << 16, device="cuda").abs().sum()   # unrelated eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert float(junk) > 0
        for c in range(3):
            assert np.array_equal(lat[c].cpu().numpy(), ref[c]), f"replay {r} chunk {c}"


# ------------------------------------------------------------------ low rank

@pytest.mark.parametrize("name,M", [("tiny", 72), ("mid", 312), ("mid", 100),
                                    ("wan_window", 4680), ("wan_720p", 10800)])
def test_lowrank_proj(name, M):
    w = wl.ALL[name]
    print(f"[lowrank {name} M={M}]", flush=True)
    a, b = wl.svd_factors_bf16(w, wl.TAG_WV, w.rank)
    xb = wl.activations(w, 0)[:M]
    p = P.LowRank.from_bits(a, b)
    y = P.lowrank_apply(p, P.to_device_bf16(xb))
    torch.cuda.synchronize()
    ref = O.lowrank_proj(_f64(xb), _f64(a), _f64(b))
    assert_close(_f64(P.from_device_bf16(y)), ref, f"{name} lowrank M={M}")


def test_lowrank_dense_and_bias():
    w = wl.WAN_FULL
    wb = wl.dense_weight_bf16(w, wl.TAG_WV)
    xb = wl.activations(w, 0)[:1000]
    bias = wl.normal_bf16(w, (w.hidden,), 99)
    x = P.to_device_bf16(xb)
    a = P.to_device_bf16(P.output_major(wb))
    y = torch.empty((1000, w.hidden), dtype=torch.bfloat16, device="cuda")
    bd = P.to_device_bf16(bias)
    B.ust_lowrank_proj(x, a, None, bd, None, y, 1000, w.hidden, w.hidden, w.hidden)
    torch.cuda.synchronize()
    ref = O.lowrank_proj(_f64(xb), _f64(wb), None, _f64(bias))
    assert_close(_f64(P.from_device_bf16(y)), ref, "dense + bias")


@pytest.mark.parametrize("name", ["mid", "wan_window", "wan_window_d64", "wan_720p"])
def test_lowrank_proj_v_append_equals_projection_then_append(name):
    """The value projection stored straight into the ring, with the keys-only
    append, leaves the ring bit for bit as ust_lowrank_proj followed by the
    full ust_kv_append does, chunk after chunk (slots no chunk wrote and the
    rows' padding keep the NaN fill); so does the same call given the keys,
    which rotates and appends them in the first product's launch.  On the
    small shape the values are also compared with the fp64 oracle."""
    w = WAN_WINDOW_D64 if name == "wan_window_d64" else wl.ALL[name]
    g = _g(w)
    print(f"[lowrank_proj_v_append {name}]", flush=True)
    table = P.RopeTable(g, w.n_tab_frames, w.theta)
    ring_ref = P.Ring(g, w.n_slots, w.n_sink, fill_bits=NAN_BITS)
    ring = P.Ring(g, w.n_slots, w.n_sink, fill_bits=NAN_BITS)
    ring_k = P.Ring(g, w.n_slots, w.n_sink, fill_bits=NAN_BITS)
    a, b = wl.svd_factors_bf16(w, wl.TAG_WV, w.rank)
    p = P.LowRank.from_bits(a, b)
    HD = w.n_heads * w.head_dim
    t = torch.empty((w.n_q, w.rank), dtype=torch.bfloat16, device="cuda")
    v = torch.empty((w.n_q, HD), dtype=torch.bfloat16, device="cuda")
    n_chunks = min(w.n_chunks, 3)
    for c in range(n_chunks):
        xb = wl.activations(w, c)
        x = P.to_device_bf16(xb)
        k = P.to_device_bf16(wl.chunk_tokens(w, wl.TAG_K, c).reshape(w.n_q, -1))
        P.lowrank_apply(p, x, v, t)
        B.ust_kv_append(g, ring_ref.abi, k, v, table.cos, table.sin, w.n_tab_frames, 3 * c)
        B.ust_kv_append(g, ring.abi, k, None, table.cos, table.sin, w.n_tab_frames, 3 * c)
        B.ust_lowrank_proj_v_append(g, ring.abi, x, p.a, p.b, t, w.hidden, w.rank, 3 * c)
        B.ust_lowrank_proj_v_append(g, ring_k.abi, x, p.a, p.b, t, w.hidden, w.rank, 3 * c,
                                    k_new=k, cos_tab=table.cos, sin_tab=table.sin,
                                    n_tab_frames=table.n_frames)
    torch.cuda.synchronize()
    for r in (ring, ring_k):
        assert torch.equal(r.k.view(torch.int16), ring_ref.k.view(torch.int16))
        assert torch.equal(r.v.view(torch.int16), ring_ref.v.view(torch.int16))
    if name == "mid":
        c = n_chunks - 1
        ref = O.lowrank_proj(_f64(wl.activations(w, c)), _f64(a), _f64(b))
        ref = ref.reshape(3, w.T, w.n_heads, w.head_dim)
        gv = ring.host_v_natural()          # [slot][h][t][d]
        got = np.stack([gv[O.slot_of_frame(3 * c + i, w.n_slots, w.n_sink)].transpose(1, 0, 2)
                        for i in range(3)])
        assert_close(_f64(got), ref, "values in the ring")


@pytest.mark.parametrize("base,heads,hidden", [("mid", 12, 1536), ("mid", 12, 1544),
                                               ("mid", 3, 1536), ("mid64", 3, 192)])
def test_lowrank_proj_v_append_keys_other_widths(base, heads, hidden):
    """The value projection with the keys, at an input width the pipelined
    product takes (1536: the keys ride in its launch) and one it does not
    (1544, not a multiple of 64: the keys get a launch of their own, then
    the register-staged product), against the keys-only append plus the
    projection without keys: the same ring bit for bit.  With 3 heads a
    chunk has 18 key tiles (9 at head size 64 and 40 tokens per frame), so
    the last key workgroup holds two (one) of its four.  The table starts
    at the chunk's own first frame."""
    w = wl.ALL[base].replace(n_heads=heads)
    g = _g(w)
    print(f"[lowrank_proj_v_append keys: {base}, {heads} heads, hidden {hidden}]", flush=True)
    rs = np.random.default_rng(81)
    rank = 64
    HD = w.n_heads * w.head_dim
    a = P.to_device_bf16(wl.f32_to_bf16_bits(rs.standard_normal((rank, hidden)) * hidden ** -0.5))
    b = P.to_device_bf16(wl.f32_to_bf16_bits(rs.standard_normal((HD, rank)) * rank ** -0.5))
    t = torch.empty((w.n_q, rank), dtype=torch.bfloat16, device="cuda")
    rings = [P.Ring(g, w.n_slots, w.n_sink, fill_bits=NAN_BITS) for _ in range(2)]
    table = P.RopeTable(g, 3, w.theta)
    for c in range(4):
        table.rebuild(3 * c)
        x = P.to_device_bf16(wl.f32_to_bf16_bits(rs.standard_normal((w.n_q, hidden))))
        k = P.to_device_bf16(wl.chunk_tokens(w, wl.TAG_K, c).reshape(w.n_q, -1))
        B.ust_kv_append(g, rings[0].abi, k, None, table.cos, table.sin, 3, 3 * c,
                        tab_first_frame=3 * c)
        B.ust_lowrank_proj_v_append(g, rings[0].abi, x, a, b, t, hidden, rank, 3 * c)
        B.ust_lowrank_proj_v_append(g, rings[1].abi, x, a, b, t, hidden, rank, 3 * c, k_new=k,
                                    cos_tab=table.cos, sin_tab=table.sin, n_tab_frames=3,
                                    tab_first_frame=3 * c)
    torch.cuda.synchronize()
    assert torch.equal(rings[0].k.view(torch.int16), rings[1].k.view(torch.int16))
    assert torch.equal(rings[0].v.view(torch.int16), rings[1].v.view(torch.int16))
    assert not torch.equal(rings[0].k.view(torch.int16)[3],
                           torch.full_like(rings[0].k.view(torch.int16)[3], NAN_BITS))


def test_keys_only_append_leaves_values():
    """ust_kv_append with v_new NULL writes the keys of the chunk's slots and
    no value."""
    w = wl.MID
    g = _g(w)
    table = P.RopeTable(g, w.n_tab_frames, w.theta)
    ring = P.Ring(g, w.n_slots, w.n_sink, fill_bits=NAN_BITS)
    ring_full = P.Ring(g, w.n_slots, w.n_sink, fill_bits=NAN_BITS)
    k = P.to_device_bf16(wl.chunk_tokens(w, wl.TAG_K, 1).reshape(w.n_q, -1))
    v = P.to_device_bf16(wl.chunk_tokens(w, wl.TAG_V, 1).reshape(w.n_q, -1))
    B.ust_kv_append(g, ring.abi, k, None, table.cos, table.sin, w.n_tab_frames, 3)
    B.ust_kv_append(g, ring_full.abi, k, v, table.cos, table.sin, w.n_tab_frames, 3)
    torch.cuda.synchronize()
    assert torch.equal(ring.k.view(torch.int16), ring_full.k.view(torch.int16))
    assert np.all(P.from_device_bf16(ring.v) == NAN_BITS)


def test_dense_wide_product_grouped_tiles():
    """A product that needs several rounds of the chip and whose weight does
    not fit in one XCD's L2 (4680 x 1536 by 4608 outputs: 684 tiles, 14 MB of
    W) runs its tiles in groups of four row blocks; the last group holds the
    three remaining ones.  Compared in full with the fp64 oracle."""
    w = wl.WAN_WINDOW
    wb = np.concatenate([wl.dense_weight_bf16(w, t) for t in (wl.TAG_WQ, wl.TAG_WK, wl.TAG_WV)],
                        axis=1)
    xb = wl.activations(w, 1)
    bias = wl.normal_bf16(w, (wb.shape[1],), 98)
    M, K, N = xb.shape[0], wb.shape[0], wb.shape[1]
    print(f"[dense grouped {M} x {K} -> {N}]", flush=True)
    x = P.to_device_bf16(xb)
    a = P.to_device_bf16(P.output_major(wb))
    y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    B.ust_lowrank_proj(x, a, None, P.to_device_bf16(bias), None, y, M, K, N, N)
    torch.cuda.synchronize()
    ref = O.lowrank_proj(_f64(xb), _f64(wb), None, _f64(bias))
    assert_close(_f64(P.from_device_bf16(y)), ref, "dense wide product, grouped tiles")


# ------------------------------------------------------------------ layer-chunk

def test_layer_chunk_wan_window_chained():
    """V projection -> append -> attention -> O projection, chained on the
    GPU, against the same chain in fp64 (no intermediate rounding)."""
    w = wl.WAN_WINDOW
    g = _g(w)
    table = P.RopeTable(g, w.n_tab_frames, w.theta)
    ring = P.Ring(g, w.n_slots, w.n_sink, fill_bits=NAN_BITS)
    av, bv = wl.svd_factors_bf16(w, wl.TAG_WV, w.rank)
    ao, bo = wl.svd_factors_bf16(w, wl.TAG_WO, w.rank)
    wv, wo = P.LowRank.from_bits(av, bv), P.LowRank.from_bits(ao, bo)
    bufs = P.LayerBuffers.alloc(w.n_q, w.hidden, w.n_heads, w.rank, w.rank, g=g,
                                schedule="split")
    cos, sin = O.rope_table(w.n_tab_frames, w.grid_h, w.grid_w, w.pairs, w.theta)
    cache = O.KVCache(w.n_slots, w.n_heads, w.T, w.head_dim)
    for c in range(w.n_chunks):
        xb = wl.activations(w, c)
        qb = wl.chunk_tokens(w, wl.TAG_Q, c)
        kb = wl.chunk_tokens(w, wl.TAG_K, c)
        y = P.layer_chunk(g, ring, table, P.to_device_bf16(xb),
                          P.to_device_bf16(qb.reshape(w.n_q, -1)),
                          P.to_device_bf16(kb.reshape(w.n_q, -1)), wv, wo, 3 * c,
                          w.n_recent, bufs)
        torch.cuda.synchronize()
        v_ref = O.lowrank_proj(_f64(xb), _f64(av), _f64(bv)).reshape(w.n_q, w.n_heads, -1)
        O.kv_append(cache, _f64(kb), v_ref, cos, sin, 3 * c, 3, w.grid_h, w.grid_w,
                    w.n_slots, w.n_sink)
        if c < 3:
            continue
        rows = _sample_rows(w.n_q, 160, seed=10 + c)
        o_ref, _ = O.window_attn(cache, _f64(qb), cos, sin, 3 * c, 3, w.grid_h, w.grid_w,
                                 w.n_slots, w.n_sink, w.n_recent, rows=rows)
        y_ref = O.lowrank_proj(o_ref.reshape(len(rows), -1), _f64(ao), _f64(bo))
        print(f"[layer_chunk wan_window chunk {c}]", flush=True)
        assert_close(_f64(P.from_device_bf16(y))[rows], y_ref, f"chunk {c} Y")


# ------------------------------------------------------------------ the C ABI from C

def test_c_program_drives_the_library():
    """tests/c_abi_check.c (built with the library): plain C11 through
    include/ust.h alone, on the GPU -- error statuses, V = 1 gives 1, split
    and unsplit schedules agree."""
    import os
    import subprocess
    from causal_video_diffusion_amd import build
    assert os.path.exists(build.C_CHECK), "c_abi_check is built with libust.so by build()"
    print("[c_abi_check]", flush=True)
    r = subprocess.run([build.C_CHECK], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr


# ------------------------------------------------------------------ fused Q/K/V projection

def _qkv_case(w, chunks_checked, rows=None, layer=0):
    """ust_qkv_append on every chunk of w against the oracle: Q = X W_q, and
    the ring after appending K = X W_k (rotated) and V = X W_v.  Slots no
    chunk wrote keep the NaN sentinel bit for bit."""
    g = _g(w)
    table = P.RopeTable(g, w.n_tab_frames, w.theta)
    ring = P.Ring(g, w.n_slots, w.n_sink, fill_bits=NAN_BITS)
    cos, sin = O.rope_table(w.n_tab_frames, w.grid_h, w.grid_w, w.pairs, w.theta)
    cache = O.KVCache(w.n_slots, w.n_heads, w.T, w.head_dim)
    wq = wl.dense_weight_bf16(w, wl.TAG_WQ, layer)
    wk = wl.dense_weight_bf16(w, wl.TAG_WK, layer)
    wv = wl.dense_weight_bf16(w, wl.TAG_WV, layer)
    w_qkv = P.qkv_weights(wq, wk, wv)
    q = torch.empty((w.n_q, w.hidden), dtype=torch.bfloat16, device="cuda")
    written = set()
    for c in range(w.n_chunks):
        xb = wl.activations(w, c)
        B.ust_qkv_append(g, ring.abi, P.to_device_bf16(xb), w_qkv, w.hidden, table.cos,
                         table.sin, w.n_tab_frames, 3 * c, q)
        torch.cuda.synchronize()
        X = _f64(xb)
        k_ref = (X @ _f64(wk)).reshape(w.n_q, w.n_heads, w.head_dim)
        v_ref = (X @ _f64(wv)).reshape(w.n_q, w.n_heads, w.head_dim)
        O.kv_append(cache, k_ref, v_ref, cos, sin, 3 * c, 3, w.grid_h, w.grid_w, w.n_slots,
                    w.n_sink)
        for i in range(3):
            written.add(O.slot_of_frame(3 * c + i, w.n_slots, w.n_sink))
        if c not in chunks_checked:
            continue
        print(f"[qkv_append {w.name} chunk {c}]", flush=True)
        r = np.arange(w.n_q) if rows is None else rows
        q_ref = X[r] @ _f64(wq)
        assert_close(_f64(P.from_device_bf16(q))[r], q_ref, f"chunk {c} Q")
        gk = ring.host_k()
        gv = ring.host_v_natural()
        gv_raw = P.from_device_bf16(ring.v)
        for s_ in range(w.n_slots):
            if s_ not in written:
                assert np.all(gk[s_] == NAN_BITS) and np.all(gv_raw[s_] == NAN_BITS), f"slot {s_}"
                continue
            tk = (r % w.T) if rows is not None else slice(None)
            assert_close(_f64(gk[s_])[:, tk], cache.k[s_][:, tk], f"chunk {c} slot {s_} K")
            assert_close(_f64(gv[s_])[:, tk], cache.v[s_][:, tk], f"chunk {c} slot {s_} V")
        assert np.all(gv_raw[..., w.T:] == NAN_BITS)   # value row padding untouched


@pytest.mark.parametrize("name", ["tiny", "tiny_wrap", "mid", "mid64"])
def test_qkv_append_full_compare(name):
    w = wl.ALL[name]
    _qkv_case(w, chunks_checked=range(w.n_chunks))


def test_qkv_append_wan_window():
    w = wl.WAN_WINDOW
    _qkv_case(w, chunks_checked=(0, 5), rows=_sample_rows(w.n_q, 160, seed=3))


def test_qkv_append_d64_wan_grid():
    # the 64-wide-head tile (192 x 64, 4 waves) on the Wan grid: 24 heads
    w = WAN_WINDOW_D64
    _qkv_case(w, chunks_checked=(0, 5), rows=_sample_rows(w.n_q, 160, seed=4))


def test_densified_rank_1413_projection():
    """The pages' rank, 0.92 x 1536 = 1413, is above the 768 break-even, so the
    value projection runs dense with W_r = A_r B_r re-densified on the GPU
    (rank zero-padded to 1416).  W_r, and V = X W_r through the fused
    projection, against the oracle's fp64 X A_r B_r."""
    w = wl.WAN_WINDOW
    a_bits, b_bits = wl.svd_factors_bf16(w, wl.TAG_WV, 1413)
    wr_t = P.densify(a_bits, b_bits)
    torch.cuda.synchronize()
    A, Bm = _f64(a_bits), _f64(b_bits)
    assert_close(_f64(P.from_device_bf16(wr_t)), (A @ Bm).T, "W_r")
    g = _g(w)
    table = P.RopeTable(g, w.n_tab_frames, w.theta)
    ring = P.Ring(g, w.n_slots, w.n_sink, fill_bits=NAN_BITS)
    wq = wl.dense_weight_bf16(w, wl.TAG_WQ)
    wk = wl.dense_weight_bf16(w, wl.TAG_WK)
    w_qkv = P.qkv_weights(wq, wk, wr_t)
    q = torch.empty((w.n_q, w.hidden), dtype=torch.bfloat16, device="cuda")
    xb = wl.activations(w, 0)
    B.ust_qkv_append(g, ring.abi, P.to_device_bf16(xb), w_qkv, w.hidden, table.cos, table.sin,
                     w.n_tab_frames, 0, q)
    torch.cuda.synchronize()
    rows = _sample_rows(w.n_q, 256, seed=4)   # first and last 64 rows, 128 between
    v_ref = O.lowrank_proj(_f64(xb)[rows], A, Bm).reshape(len(rows), w.n_heads, w.head_dim)
    gv = ring.host_v_natural()
    for fi in range(3):
        sel = rows[(rows >= fi * w.T) & (rows < (fi + 1) * w.T)]
        assert len(sel) > 0
        got = _f64(gv[O.slot_of_frame(fi, w.n_slots, w.n_sink)])[:, sel - fi * w.T]
        ref = v_ref[np.isin(rows, sel)].transpose(1, 0, 2)
        assert_close(got, ref, f"frame {fi} V = X A_r B_r")


def test_layer_chunk_fused_mid():
    """Fused Q/K/V projection + append, attention, output projection (W_o
    re-densified from rank 48 factors) over MID's chunks, against the fp64
    chain X W_q, X W_k, X A_v B_v, attention, (O A_o) B_o."""
    w = wl.MID
    g = _g(w)
    r = 48
    table = P.RopeTable(g, w.n_tab_frames, w.theta)
    ring = P.Ring(g, w.n_slots, w.n_sink, fill_bits=NAN_BITS)
    wq = wl.dense_weight_bf16(w, wl.TAG_WQ)
    wk = wl.dense_weight_bf16(w, wl.TAG_WK)
    av, bv = wl.svd_factors_bf16(w, wl.TAG_WV, r)
    ao, bo = wl.svd_factors_bf16(w, wl.TAG_WO, r)
    w_qkv = P.qkv_weights(wq, wk, P.densify(av, bv))
    wo = P.LowRank(P.densify(ao, bo), None)
    bufs = P.LayerBuffers.alloc(w.n_q, w.hidden, w.n_heads, None, None)
    q = torch.empty((w.n_q, w.hidden), dtype=torch.bfloat16, device="cuda")
    cos, sin = O.rope_table(w.n_tab_frames, w.grid_h, w.grid_w, w.pairs, w.theta)
    cache = O.KVCache(w.n_slots, w.n_heads, w.T, w.head_dim)
    for c in range(w.n_chunks):
        xb = wl.activations(w, c)
        y = P.layer_chunk_fused(g, ring, table, P.to_device_bf16(xb), w_qkv, wo, 3 * c,
                                w.n_recent, bufs, q)
        torch.cuda.synchronize()
        X = _f64(xb)
        shape = (w.n_q, w.n_heads, w.head_dim)
        O.kv_append(cache, (X @ _f64(wk)).reshape(shape),
                    O.lowrank_proj(X, _f64(av), _f64(bv)).reshape(shape), cos, sin, 3 * c, 3,
                    w.grid_h, w.grid_w, w.n_slots, w.n_sink)
        o_ref, _ = O.window_attn(cache, (X @ _f64(wq)).reshape(shape), cos, sin, 3 * c, 3,
                                 w.grid_h, w.grid_w, w.n_slots, w.n_sink, w.n_recent)
        y_ref = O.lowrank_proj(o_ref.reshape(w.n_q, -1), _f64(ao), _f64(bo))
        print(f"[fused layer-chunk mid chunk {c}]", flush=True)
        assert_close(_f64(P.from_device_bf16(y)), y_ref, f"chunk {c} Y")


# ------------------------------------------------------------------ clip schedule

@pytest.mark.timeout(600)
def test_clip_schedule_wan_clip():
    """The 81-frame clip over 30 layers (UnStep, Table 3: 4 forwards for the
    first chunk, 2 for each later one, plus a clean-cache forward per chunk).
    Every forward of a chunk writes the chunk's frames; every layer has its
    own weights and ring and sees the same hidden states (reading).  The GPU
    runs all 23 x 30 layer-chunks; sampled (layer, forward, rows) are checked
    against the oracle, which rebuilds the cache state the sample sees: the
    clean-cache forward's keys/values for earlier chunks, the forward's own
    for the current chunk."""
    w = wl.WAN_CLIP
    g = _g(w)
    sched = P.clip_forwards(w.n_chunks, w.first_steps, w.later_steps, w.clean_pass)
    assert len(sched) == 23
    assert [f for f in sched] == O.clip_schedule(w.n_chunks, w.first_steps,
                                                 w.later_steps, w.clean_pass)
    table = P.RopeTable(g, w.n_tab_frames, w.theta)
    samples = {(0, 0), (17, 12), (29, 22), (8, 5)}      # (layer, forward index)
    print("[clip: preparing 30 layers of weights]", flush=True)
    layers = []
    for layer in range(w.layers):
        wq = wl.dense_weight_bf16(w, wl.TAG_WQ, layer)
        wk = wl.dense_weight_bf16(w, wl.TAG_WK, layer)
        av, bv = wl.svd_factors_bf16(w, wl.TAG_WV, w.rank, layer)
        ao, bo = wl.svd_factors_bf16(w, wl.TAG_WO, w.rank, layer)
        layers.append(dict(
            wq=P.LowRank(P.to_device_bf16(P.output_major(wq)), None),
            wk=P.LowRank(P.to_device_bf16(P.output_major(wk)), None),
            wv=P.LowRank.from_bits(av, bv), wo=P.LowRank.from_bits(ao, bo),
            ring=P.Ring(g, w.n_slots, w.n_sink, fill_bits=NAN_BITS),
            host=(wq, wk, av, bv, ao, bo)))
    bufs = P.LayerBuffers.alloc(w.n_q, w.hidden, w.n_heads, w.rank, w.rank, g=g)   # auto
    qbuf = torch.empty((w.n_q, w.hidden), dtype=torch.bfloat16, device="cuda")
    kbuf = torch.empty_like(qbuf)
    got = {}
    print("[clip: running 23 forwards x 30 layers]", flush=True)
    for fi, (c, s, clean) in enumerate(sched):
        x = P.to_device_bf16(wl.activations(w, c, s))
        for layer, L in enumerate(layers):
            P.lowrank_apply(L["wq"], x, qbuf)
            P.lowrank_apply(L["wk"], x, kbuf)
            y = P.layer_chunk(g, L["ring"], table, x, qbuf, kbuf, L["wv"], L["wo"], 3 * c,
                              w.n_recent, bufs)
            if (layer, fi) in samples:
                got[(layer, fi)] = P.from_device_bf16(y)
    torch.cuda.synchronize()
    cos, sin = O.rope_table(w.n_tab_frames, w.grid_h, w.grid_w, w.pairs, w.theta)
    last_forward = {c: max(i for i, f in enumerate(sched) if f[0] == c) for c in range(w.n_chunks)}
    for (layer, fi) in sorted(samples):
        c, s, clean = sched[fi]
        wq, wk, av, bv, ao, bo = (_f64(a) for a in layers[layer]["host"])
        cache = O.KVCache(w.n_slots, w.n_heads, w.T, w.head_dim)
        frames, _ = O.window_slots(3 * c, 3, w.n_sink, w.n_recent, w.n_slots)
        for cc in sorted({f // 3 for f in frames}):
            step_cc = s if cc == c else sched[last_forward[cc]][1]
            xcc = _f64(wl.activations(w, cc, step_cc))
            k = (xcc @ wk).reshape(w.n_q, w.n_heads, -1)
            v = O.lowrank_proj(xcc, av, bv).reshape(w.n_q, w.n_heads, -1)
            O.kv_append(cache, k, v, cos, sin, 3 * cc, 3, w.grid_h, w.grid_w, w.n_slots, w.n_sink)
        rows = _sample_rows(w.n_q, 128, seed=fi)
        xq = _f64(wl.activations(w, c, s))[rows]
        q = np.zeros((w.n_q, w.n_heads, w.head_dim))
        q[rows] = (xq @ wq).reshape(len(rows), w.n_heads, -1)
        o_ref, _ = O.window_attn(cache, q, cos, sin, 3 * c, 3, w.grid_h, w.grid_w, w.n_slots,
                                 w.n_sink, w.n_recent, rows=rows)
        y_ref = O.lowrank_proj(o_ref.reshape(len(rows), -1), ao, bo)
        print(f"[clip layer {layer} forward {fi} (chunk {c}, step {s}, clean {clean})]", flush=True)
        assert_close(_f64(got[(layer, fi)])[rows], y_ref, f"clip layer {layer} forward {fi}")
