"""Plain float64 reference of the per-chunk DiT self-attention path.

TEST INFRASTRUCTURE ONLY (see the package docstring): slow, obviously correct,
NumPy float64, no blocking or fusion beyond what each definition states.

The path (UnStep, abstract): a causal video DiT generates latent video chunk
by chunk; each chunk's self-attention reads a KV cache of earlier latent
frames whose temporal window is limited; positions enter through a 3-D RoPE
whose cos/sin coefficients are cached; the value and output projections are
replaced by their truncated-SVD factors.  Chunks are three latent frames, and
a clip is seven chunks (UnStep, Table 3).

Layouts used here (the oracle's own, chosen for readability):
  chunk tensors q, k_new, v_new : [chunk_frames*T][H][D]; token n is frame
      frame_start + n // T at (y, x) = divmod(n % T, grid_w)
  cache k, v                    : [n_slots][H][T][D]
  RoPE table cos, sin           : [n_frames][grid_h][grid_w][P], P = D/2;
      row i holds frame first_frame + i (0 unless a call says otherwise)

Readings of points the paper leaves open are marked READING.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "pair_axis", "rope_frequencies", "rope_table", "rope_apply",
    "chunk_positions", "slot_of_frame", "window_frames", "window_slots",
    "KVCache", "kv_append", "window_attn", "lowrank_proj", "clip_schedule",
    "RAW_STEPS_4", "RAW_STEPS_2", "shifted_sigma", "dit_label", "flow_step",
    "sample_chunk", "rne_bf16", "conv3d_causal",
]


# ------------------------------------------------------------------ 3-D RoPE
# UnStep, abstract: the runtime stack applies RoPE from precomputed cos/sin
# coefficients.
# READING: the head dimension is split into P = D/2 rotation pairs; the first
# pairs_t pairs rotate with the latent-frame index, the next pairs_h with the
# token row, the last pairs_w with the token column (the 3-D RoPE of the
# Wan-family DiT).  Each axis is a 1-D RoPE of its own: pair j of an axis with
# n_a pairs turns by position * theta**(-j/n_a).  Positions are absolute,
# 0-based; pairs are adjacent elements (2p, 2p+1).

def pair_axis(p: int, pairs: Sequence[int]) -> Tuple[int, int, int]:
    """(axis, index within the axis, pairs on that axis) of rotation pair p."""
    pt, ph, pw = pairs
    if p < pt:
        return 0, p, pt
    if p < pt + ph:
        return 1, p - pt, ph
    return 2, p - pt - ph, pw


def rope_frequencies(pairs: Sequence[int], theta: float) -> np.ndarray:
    """Angular frequency of every pair, fp64 [P]."""
    P = sum(pairs)
    out = np.empty(P)
    for p in range(P):
        _, j, n = pair_axis(p, pairs)
        out[p] = theta ** (-j / n)
    return out


def rope_table(n_frames: int, grid_h: int, grid_w: int, pairs: Sequence[int],
               theta: float, first_frame: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Cached coefficients: cos and sin of every (frame, row, col, pair) angle,
    for the frames first_frame .. first_frame + n_frames - 1 (row i holds
    frame first_frame + i; the position on the temporal axis is the absolute
    frame)."""
    P = sum(pairs)
    freq = rope_frequencies(pairs, theta)
    axis = np.array([pair_axis(p, pairs)[0] for p in range(P)])
    f = (first_frame + np.arange(n_frames, dtype=np.float64))[:, None, None, None]
    y = np.arange(grid_h, dtype=np.float64)[None, :, None, None]
    x = np.arange(grid_w, dtype=np.float64)[None, None, :, None]
    pos = np.where(axis == 0, f, np.where(axis == 1, y, x))   # broadcast to 4-D
    pos = np.broadcast_to(pos, (n_frames, grid_h, grid_w, P))
    ang = pos * freq
    return np.cos(ang), np.sin(ang)


def rope_apply(u: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate every pair (u[2p], u[2p+1]) by the angle whose cos/sin are given.

    u: [..., D]; cos, sin: broadcastable to [..., D/2]."""
    u = np.asarray(u, dtype=np.float64)
    a = u[..., 0::2]
    b = u[..., 1::2]
    out = np.empty(u.shape)
    out[..., 0::2] = a * cos - b * sin
    out[..., 1::2] = a * sin + b * cos
    return out


def chunk_positions(frame_start: int, chunk_frames: int, grid_h: int,
                    grid_w: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(frame, row, col) of every token of a chunk, in token order.

    READING: tokens are frame-major, then row-major within a frame."""
    T = grid_h * grid_w
    n = np.arange(chunk_frames * T)
    f = frame_start + n // T
    t = n % T
    return f, t // grid_w, t % grid_w


# ------------------------------------------------------------------ KV cache
# UnStep, abstract: the KV cache keeps a limited temporal window, and the
# runtime stack speeds up how the cache is indexed.
# READING: the cache holds one slot per latent frame.  The first n_sink frames
# (attention sinks, pinned) keep slots 0..n_sink-1; every later frame goes to
# a ring over the remaining n_slots - n_sink slots.

def slot_of_frame(frame: int, n_slots: int, n_sink: int) -> int:
    if frame < 0 or n_sink < 0 or n_slots <= n_sink:
        raise ValueError("bad frame or ring")
    if frame < n_sink:
        return frame
    return n_sink + (frame - n_sink) % (n_slots - n_sink)


def window_frames(frame_start: int, chunk_frames: int, n_sink: int,
                  n_recent: int) -> List[int]:
    """Latent frames one chunk attends to (UnStep, abstract: limited window).

    The prior frames that are sinks (f < n_sink) or among the n_recent most
    recent ones (n_recent = -1: all of them), each once, ascending, then the
    chunk's own frames.  READING: sink and recent sets are merged as a union;
    a sink frame inside the current chunk counts once, as current."""
    prior = [f for f in range(frame_start)
             if f < n_sink or n_recent < 0 or f >= frame_start - n_recent]
    return prior + list(range(frame_start, frame_start + chunk_frames))


def window_slots(frame_start: int, chunk_frames: int, n_sink: int,
                 n_recent: int, n_slots: int) -> Tuple[List[int], List[int]]:
    """Window frames and their slots; ValueError if a window frame has been
    overwritten by a later frame written into the same ring slot (frames are
    written in order up to frame_start + chunk_frames - 1)."""
    frames = window_frames(frame_start, chunk_frames, n_sink, n_recent)
    last = frame_start + chunk_frames - 1
    slots = []
    for f in frames:
        s = slot_of_frame(f, n_slots, n_sink)
        for g in range(f + 1, last + 1):
            if slot_of_frame(g, n_slots, n_sink) == s:
                raise ValueError(f"frame {f} was overwritten by frame {g}")
        slots.append(s)
    return frames, slots


class KVCache:
    """Keys (stored RoPE-rotated) and values per frame slot, fp64."""

    def __init__(self, n_slots: int, n_heads: int, T: int, D: int,
                 fill: float = np.nan):
        self.k = np.full((n_slots, n_heads, T, D), fill)
        self.v = np.full((n_slots, n_heads, T, D), fill)


def kv_append(cache: KVCache, k_new: np.ndarray, v_new: np.ndarray,
              cos_tab: np.ndarray, sin_tab: np.ndarray, frame_start: int,
              chunk_frames: int, grid_h: int, grid_w: int, n_slots: int,
              n_sink: int, tab_first: int = 0) -> None:
    """Write one chunk's keys (rotated at their own position) and values into
    the slots of its frames; every other slot is left as it was.  Row f -
    tab_first of the table holds frame f."""
    T = grid_h * grid_w
    k_new = np.asarray(k_new, dtype=np.float64)
    v_new = np.asarray(v_new, dtype=np.float64)
    for i in range(chunk_frames):
        f = frame_start + i
        s = slot_of_frame(f, n_slots, n_sink)
        rows = slice(i * T, (i + 1) * T)
        c = cos_tab[f - tab_first].reshape(T, -1)[:, None, :]
        sn = sin_tab[f - tab_first].reshape(T, -1)[:, None, :]
        kr = rope_apply(k_new[rows], c, sn)            # [T][H][D]
        cache.k[s] = kr.transpose(1, 0, 2)
        cache.v[s] = v_new[rows].transpose(1, 0, 2)


# ------------------------------------------------------------------ attention
# UnStep, abstract: generation is causal over chunks and the attention window
# in the KV cache is limited.  READING: every query of a chunk sees every key
# of the window (its own chunk included; no mask inside the window) and
# nothing else; scores are scaled by 1/sqrt(D).

def window_attn(cache: KVCache, q: np.ndarray, cos_tab: np.ndarray,
                sin_tab: np.ndarray, frame_start: int, chunk_frames: int,
                grid_h: int, grid_w: int, n_slots: int, n_sink: int,
                n_recent: int, scale: Optional[float] = None,
                rows: Optional[np.ndarray] = None, block: int = 1024,
                tab_first: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of the chunk's queries over the window keys.

    q: [chunk_frames*T][H][D] un-rotated; row f - tab_first of the table
    holds frame f.  Returns O [n][H][D] for the query
    rows asked for (all by default) and the natural-log sum of exponentials of
    the scaled scores, lse [H][n].  The softmax is materialised per block of
    query rows (no online rescaling)."""
    T = grid_h * grid_w
    q = np.asarray(q, dtype=np.float64)
    H, D = q.shape[1], q.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if rows is None:
        rows = np.arange(q.shape[0])
    rows = np.asarray(rows)
    frames, slots = window_slots(frame_start, chunk_frames, n_sink, n_recent,
                                 n_slots)
    f, y, x = chunk_positions(frame_start, chunk_frames, grid_h, grid_w)
    c = cos_tab[f[rows] - tab_first, y[rows], x[rows]][:, None, :]
    s = sin_tab[f[rows] - tab_first, y[rows], x[rows]][:, None, :]
    qr = rope_apply(q[rows], c, s)                     # [n][H][D]
    Kw = cache.k[slots]                                # [nf][H][T][D]
    Vw = cache.v[slots]
    out = np.empty((len(rows), H, D))
    lse = np.empty((H, len(rows)))
    for h in range(H):
        Kh = Kw[:, h].reshape(-1, D)                   # [nf*T][D]
        Vh = Vw[:, h].reshape(-1, D)
        for b0 in range(0, len(rows), block):
            b1 = min(b0 + block, len(rows))
            S = (qr[b0:b1, h] @ Kh.T) * scale
            m = S.max(axis=1, keepdims=True)
            E = np.exp(S - m)
            l = E.sum(axis=1, keepdims=True)
            out[b0:b1, h] = (E @ Vh) / l
            lse[h, b0:b1] = (m + np.log(l))[:, 0]
    return out, lse


# ------------------------------------------------------------------ low rank
# UnStep, abstract and Table 5 caption: truncated SVD of the attention value
# and output projections.  With W ~ A_r B_r (A_r: in x r, B_r: r x out) the
# projection of row vectors X is (X A_r) B_r.

def lowrank_proj(x: np.ndarray, a: np.ndarray, b: Optional[np.ndarray] = None,
                 bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Y = (X A) B (+ bias); with b None, Y = X A.  fp64."""
    y = np.asarray(x, dtype=np.float64) @ np.asarray(a, dtype=np.float64)
    if b is not None:
        y = y @ np.asarray(b, dtype=np.float64)
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)
    return y


# ------------------------------------------------------------------ schedule
# UnStep, Table 3: seven chunks of three latent frames; the first chunk takes
# four denoising steps, each later chunk two (four without UnStep), and every
# chunk one clean-cache forward; the counts include that forward.
# READING: every forward of a chunk writes the chunk's frames into the cache
# (so the chunk attends to itself); the clean-cache forward writes last, so
# later chunks see its keys and values.

def clip_schedule(n_chunks: int, first_steps: int, later_steps: int,
                  clean_pass: bool) -> List[Tuple[int, int, bool]]:
    """(chunk, forward index within the chunk, is clean-cache forward), in
    execution order."""
    out = []
    for c in range(n_chunks):
        steps = first_steps if c == 0 else later_steps
        for i in range(steps):
            out.append((c, i, False))
        if clean_pass:
            out.append((c, steps, True))
    return out


# ------------------------------------------------------------------ sampler
# UnStep, Table 4: the few-step model's four denoising levels are the raw
# timesteps 1000, 750, 500, 250 after a shift-5 mapping, giving noise levels
# sigma = 1, 15/16, 5/6, 5/8 and DiT labels t = 1000 sigma; the clean-cache
# forward runs at label 0, on the clean chunk (Self Forcing: sigma 0) or on
# the chunk renoised to sigma* = 0.02 (UnStep).  Abstract: UnStep renoises the
# generated frames to a nearly clean level and lets the clean-cache forward,
# which runs anyway, refine them.  Table 3: four denoising forwards for the
# first chunk, two for each later one, plus the clean-cache forward.
# READING (flow matching, this model family's parameterisation; the term is
# on the pages' glossary): a latent at level sigma is
# x = (1 - sigma) x0 + sigma eps, the DiT predicts the velocity
# v = eps - x0, so the denoised estimate is x0_hat = x - sigma v.
# READING: between denoising steps the estimate is renoised to the next level
# with a fresh draw, x' = (1 - sigma') x0_hat + sigma' eps'; after the last
# step, to sigma* for the clean-cache forward.
# READING: the later chunks' two steps are the raw timesteps 1000 and 500
# (every other one of the four); the pages do not say which two.
# READING: the chunk UnStep keeps is the clean-cache forward's estimate at the
# true level, x_in - sigma* v*; with sigma* = 0 (Self Forcing) that is the
# clean chunk itself, unchanged.

RAW_STEPS_4 = (1000, 750, 500, 250)
RAW_STEPS_2 = (1000, 500)


def shifted_sigma(raw, shift: float = 5.0, n_train: int = 1000) -> np.ndarray:
    """Noise level of raw timestep(s) after the shift mapping:
    sigma = shift u / (1 + (shift - 1) u), u = raw / n_train (Table 4)."""
    u = np.asarray(raw, dtype=np.float64) / n_train
    return shift * u / (1.0 + (shift - 1.0) * u)


def dit_label(sigma, n_train: int = 1000) -> np.ndarray:
    """The timestep label the DiT receives at level sigma (Table 4)."""
    return n_train * np.asarray(sigma, dtype=np.float64)


def flow_step(x: np.ndarray, v: np.ndarray, noise: Optional[np.ndarray],
              sigma: float, sigma_next: float) -> Tuple[np.ndarray, np.ndarray]:
    """One sampler step at level sigma: the denoised estimate
    x0_hat = x - sigma v, and the latent renoised to sigma_next,
    (1 - sigma_next) x0_hat + sigma_next noise (noise unused at
    sigma_next = 0).  Returns (x0_hat, x_next), fp64."""
    x = np.asarray(x, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    x0 = x - float(sigma) * v
    if sigma_next == 0:
        return x0, x0.copy()
    nz = np.asarray(noise, dtype=np.float64)
    return x0, (1.0 - float(sigma_next)) * x0 + float(sigma_next) * nz


def sample_chunk(dit, x_init: np.ndarray, noises: Sequence[np.ndarray],
                 raw_steps: Sequence[int], sigma_star: float,
                 shift: float = 5.0) -> Tuple[np.ndarray, List[float], List[float]]:
    """One chunk of the sampler: a denoising forward per raw step, then the
    clean-cache forward.  dit(x, t) returns the DiT's velocity for latent x
    at label t.  x_init is the chunk's initial noise (level sigma_0 = 1 at raw
    1000); noises[i] is the draw used to renoise after denoising step i (the
    last one renoises to sigma_star; unused when sigma_star = 0).
    Returns (the chunk kept, the levels the latent was at for each forward,
    the labels passed), so len(levels) is the chunk's forward count."""
    sig = [float(s) for s in shifted_sigma(raw_steps, shift)]
    x = np.asarray(x_init, dtype=np.float64)
    levels, labels = [], []
    for i, s in enumerate(sig):
        nxt = sig[i + 1] if i + 1 < len(sig) else float(sigma_star)
        v = dit(x, float(dit_label(s)))
        levels.append(s)
        labels.append(float(dit_label(s)))
        _, x = flow_step(x, v, noises[i] if nxt != 0 else None, s, nxt)
    # the clean-cache forward: label 0, latent at sigma_star
    v = dit(x, 0.0)
    levels.append(float(sigma_star))
    labels.append(0.0)
    x0, _ = flow_step(x, v, None, float(sigma_star), 0.0)
    return x0, levels, labels


# ------------------------------------------------------------------ rounding

def rne_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned
    as float64: the rounding every test input goes through.  The seeded
    input generator rounds float32 to bfloat16 by integer bit arithmetic;
    this is the same rounding by another route (frexp and round-half-even),
    and the pins compare the two.  Normal range only (|x| >= 2**-126);
    bfloat16 subnormals do not occur in the workloads."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                  # x = m * 2**e, 0.5 <= |m| < 1
    # bfloat16 keeps 8 significant bits: scale the mantissa to [128, 256)
    scaled = m * 256.0
    r = np.round(scaled)                # numpy rounds half to even
    out = np.ldexp(r, e - 8)
    return np.where(np.isfinite(x), out, x)


# ------------------------------------------------------------------ decoder
# UnStep, abstract: the runtime stack also speeds up VAE decoding, with an
# optimised memory layout, precision and convolution kernels; Table 3: the
# decoder turns the 1x21x16x60x104 latent into 81 frames of 832x480.  The
# decoder's architecture is not on the pages.
# READING: the decoder's convolutions are causal in time (a causal video
# model decodes frames in order): output frame t sees input frames t-2, t-1,
# t, with frames before the first taken as zero; 3x3 in space with zero
# padding, so each frame keeps its size; stride 1.
# Layout here: activations [T][H][W][C] (channels last), weights
# [Cout][3][3][3][Cin] (time, row, column offsets), bias [Cout].

def conv3d_causal(x: np.ndarray, w: np.ndarray,
                  bias: Optional[np.ndarray] = None,
                  history: Optional[np.ndarray] = None) -> np.ndarray:
    """out[t, y, x, o] = bias[o] + sum over dt, dy, dx, i of
    w[o, dt, dy, dx, i] * x[t + dt - 2, y + dy - 1, x + dx - 1, i], with x
    zero outside its rows and columns, and before frame 0 zero, or, given
    `history` [2, H, W, Ci], the two frames that precede frame 0 (the last
    input frames of the previous chunk when a clip is decoded chunk by
    chunk).  fp64; one matrix product per kernel tap over the padded input."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    T, H, W, Ci = x.shape
    Co = w.shape[0]
    assert w.shape == (Co, 3, 3, 3, Ci)
    xp = np.zeros((T + 2, H + 2, W + 2, Ci))
    xp[2:, 1:H + 1, 1:W + 1] = x
    if history is not None:
        history = np.asarray(history, dtype=np.float64)
        assert history.shape == (2, H, W, Ci)
        xp[:2, 1:H + 1, 1:W + 1] = history
    out = np.zeros((T, H, W, Co))
    for dt in range(3):
        for dy in range(3):
            for dx in range(3):
                out += xp[dt:dt + T, dy:dy + H, dx:dx + W] @ w[:, dt, dy, dx, :].T
    if bias is not None:
        out += np.asarray(bias, dtype=np.float64)
    return out
