"""Workload descriptions and seeded synthetic inputs.

This module is shared by the tests, the benchmark and the smoke check.  It
draws random numbers and converts them to bfloat16; it holds none of the
attention, RoPE, KV-cache or projection arithmetic (that lives in the HIP
library and, independently, in the CPU oracle).

Workload shapes follow the UnStep paper (arXiv 2609.32518): an 81-frame
832x480 clip whose initial latent noise is 1x21x16x60x104 (appendix Table 3),
generated as seven causal chunks of three latent frames each (Table 3), by a
Wan2.1-1.3B DiT (Table 1 caption).  With a 1x2x2 patch a latent frame is
30x52 = 1560 tokens; the DiT has hidden size 1536 = 12 heads x 128.  The
window sizes (3 sink + 6 recent frames, 3 sink + 9 recent at 720p) and the
SVD ranks (512, 256, 16) are workload parameters the paper leaves open; they
are fixed here per workload.

Seeds: every tensor is drawn from PCG64 seeded with
``SeedSequence([0, workload_id, tag, chunk, step, layer])``.  Floating values
are drawn in float32 and rounded to bfloat16 with round-to-nearest-even, and
are stored as uint16 bit patterns so that both the oracle (which widens them
exactly to float64) and the GPU see the very same values.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np

# tensor tags for the seed sequence
TAG_X = 1
TAG_Q = 2
TAG_K = 3
TAG_V = 4
TAG_WQ = 5
TAG_WK = 6
TAG_WV = 7
TAG_WO = 8
TAG_EPS = 9     # the sampler's noise draws
TAG_VEL = 10    # stand-in DiT velocities for the sampler

LATENT_CHANNELS = 16   # appendix Table 3: initial noise 1x21x16x60x104


@dataclass(frozen=True)
class Workload:
    """One workload: the geometry of a DiT self-attention layer and its cache."""

    wid: int                 # workload id, part of every seed
    name: str
    grid_h: int              # latent-frame token grid
    grid_w: int
    n_heads: int
    head_dim: int
    pairs: Tuple[int, int, int]   # RoPE pairs on the (frame, row, col) axes
    theta: float
    chunk_frames: int        # latent frames per causal chunk
    n_chunks: int            # chunks appended in order
    n_slots: int             # frame slots in the KV ring
    n_sink: int              # leading frames pinned in the ring
    n_recent: int            # recent prior frames in the window, -1 = all
    rank: Optional[int]      # SVD rank of the V/O projections, None = dense
    n_tab_frames: int        # frames covered by the RoPE table
    layers: int = 1
    first_steps: int = 1     # denoising forwards of the first chunk
    later_steps: int = 1     # denoising forwards of every later chunk
    clean_pass: bool = False # one extra clean-cache forward per chunk
    x_std: float = 1.0

    @property
    def T(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def hidden(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def n_q(self) -> int:
        return self.chunk_frames * self.T

    @property
    def w_std(self) -> float:
        return 1.0 / np.sqrt(self.hidden)

    def geom_tuple(self):
        return (self.grid_h, self.grid_w, self.n_heads, self.head_dim,
                self.pairs[0], self.pairs[1], self.pairs[2], self.chunk_frames)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


TINY = Workload(wid=0, name="tiny", grid_h=4, grid_w=6, n_heads=1, head_dim=64,
                pairs=(12, 10, 10), theta=10000.0, chunk_frames=3, n_chunks=3,
                n_slots=9, n_sink=1, n_recent=3, rank=16, n_tab_frames=9)
# same as TINY but with the smallest ring that holds the window, so slots wrap
TINY_WRAP = TINY.replace(name="tiny_wrap", n_slots=7)

WAN_FULL = Workload(wid=1, name="wan_full", grid_h=30, grid_w=52, n_heads=12,
                    head_dim=128, pairs=(22, 21, 21), theta=10000.0,
                    chunk_frames=3, n_chunks=7, n_slots=21, n_sink=0,
                    n_recent=-1, rank=None, n_tab_frames=21)

WAN_WINDOW = Workload(wid=2, name="wan_window", grid_h=30, grid_w=52, n_heads=12,
                      head_dim=128, pairs=(22, 21, 21), theta=10000.0,
                      chunk_frames=3, n_chunks=6, n_slots=21, n_sink=3,
                      n_recent=6, rank=512, n_tab_frames=21)

WAN_CLIP = Workload(wid=3, name="wan_clip", grid_h=30, grid_w=52, n_heads=12,
                    head_dim=128, pairs=(22, 21, 21), theta=10000.0,
                    chunk_frames=3, n_chunks=7, n_slots=21, n_sink=3,
                    n_recent=6, rank=512, n_tab_frames=21, layers=30,
                    first_steps=4, later_steps=2, clean_pass=True)

WAN_720P = Workload(wid=4, name="wan_720p", grid_h=45, grid_w=80, n_heads=12,
                    head_dim=128, pairs=(22, 21, 21), theta=10000.0,
                    chunk_frames=3, n_chunks=7, n_slots=15, n_sink=3,
                    n_recent=9, rank=256, n_tab_frames=21)

# Test geometries small enough for a full element-by-element oracle compare,
# yet spanning several query tiles (312 = 2*128 + 56 queries), key tiles that
# straddle frames (104 tokens/frame), a ragged last key tile, and a ring that
# wraps (12 slots, 3 sinks).
MID = Workload(wid=5, name="mid", grid_h=8, grid_w=13, n_heads=12, head_dim=128,
               pairs=(22, 21, 21), theta=10000.0, chunk_frames=3, n_chunks=6,
               n_slots=12, n_sink=3, n_recent=6, rank=64, n_tab_frames=18)
MID64 = Workload(wid=6, name="mid64", grid_h=4, grid_w=10, n_heads=4, head_dim=64,
                 pairs=(12, 10, 10), theta=10000.0, chunk_frames=3, n_chunks=5,
                 n_slots=8, n_sink=1, n_recent=4, rank=32, n_tab_frames=15)

ALL = {w.name: w for w in (TINY, TINY_WRAP, WAN_FULL, WAN_WINDOW, WAN_CLIP, WAN_720P,
                           MID, MID64)}


# ---------------------------------------------------------------- bf16 bits

def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f64(b) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) exactly to float64."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- draws

def rng(w: Workload, tag: int, chunk: int = 0, step: int = 0, layer: int = 0):
    ss = np.random.SeedSequence([0, w.wid, tag, chunk, step, layer])
    return np.random.Generator(np.random.PCG64(ss))


def normal_bf16(w: Workload, shape, tag, chunk=0, step=0, layer=0, std=1.0):
    """N(0, std^2) drawn in float32, rounded to bf16; returns uint16 bits."""
    g = rng(w, tag, chunk, step, layer)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x = (x.astype(np.float64) * std).astype(np.float32)
    return f32_to_bf16_bits(x)


def chunk_tokens(w: Workload, tag: int, chunk: int, step: int = 0, layer: int = 0):
    """A chunk's per-token head vectors, [chunk_frames*T][H][D] bf16 bits.

    Token n of the chunk is latent frame chunk*C + n // T, position
    (y, x) = divmod(n % T, grid_w) in that frame."""
    return normal_bf16(w, (w.n_q, w.n_heads, w.head_dim), tag, chunk, step, layer)


def latent_shape(w: Workload):
    """A chunk's latent: chunk_frames x 16 channels x (2 grid_h) x (2 grid_w);
    each token is a 1x2x2 patch (appendix Table 3: 21 x 16 x 60 x 104 for
    the 832x480 clip, whose frames are 30 x 52 tokens)."""
    return (w.chunk_frames, LATENT_CHANNELS, 2 * w.grid_h, 2 * w.grid_w)


def latent_noise(w: Workload, chunk: int, draw: int) -> np.ndarray:
    """A chunk's noise draw `draw` (0: its initial noise; i + 1: the draw for
    renoising after its step i), N(0, 1) in float32, flat."""
    g = rng(w, TAG_EPS, chunk, draw, 0)
    return g.standard_normal(size=int(np.prod(latent_shape(w))), dtype=np.float32)


def stand_in_velocity(w: Workload, chunk: int, forward: int) -> np.ndarray:
    """A velocity for the sampler when no DiT is run: N(0, 1) drawn in
    float32, rounded to bf16 (uint16 bits), flat, per (chunk, forward)."""
    return normal_bf16(w, (int(np.prod(latent_shape(w))),), TAG_VEL, chunk, forward, 0)


def activations(w: Workload, chunk: int, step: int = 0):
    """Hidden states X of one chunk forward, [chunk_frames*T][hidden] bf16."""
    return normal_bf16(w, (w.n_q, w.hidden), TAG_X, chunk, step, 0, std=w.x_std)


def dense_weight_f64(w: Workload, tag: int, layer: int = 0) -> np.ndarray:
    """A random projection matrix W ~ N(0, 1/hidden), applied as X @ W, in fp64."""
    g = rng(w, tag, 0, 0, layer)
    return g.standard_normal(size=(w.hidden, w.hidden)) * w.w_std


def dense_weight_bf16(w: Workload, tag: int, layer: int = 0):
    """W rounded to bf16, [in][out] bits."""
    return f32_to_bf16_bits(dense_weight_f64(w, tag, layer).astype(np.float32))


def svd_factors_f64(w: Workload, tag: int, rank: int, layer: int = 0):
    """Rank-r factors of a random projection W (in x out, fp64).

    W = U S V^T; A = U[:, :r] sqrt(S_r)  (in x r), B = sqrt(S_r) V[:, :r]^T
    (r x out).  This is the offline weight preparation of the truncated-SVD
    projections (UnStep, abstract); it is input data for the projection step,
    not part of it.  Returns (A, B) in fp64."""
    W = dense_weight_f64(w, tag, layer)
    U, S, Vt = np.linalg.svd(W)
    rs = np.sqrt(S[:rank])
    return U[:, :rank] * rs[None, :], rs[:, None] * Vt[:rank, :]


def svd_factors_bf16(w: Workload, tag: int, rank: int, layer: int = 0):
    """svd_factors_f64 rounded to bf16: (A bits [in][r], B bits [r][out])."""
    A, B = svd_factors_f64(w, tag, rank, layer)
    return (f32_to_bf16_bits(A.astype(np.float32)),
            f32_to_bf16_bits(B.astype(np.float32)))


# ---------------------------------------------------------------- decoder convolution
# The decoder runtime stack's convolution (UnStep, abstract; Table 3 fixes
# the decoder's input, 21 latent frames of 16 x 60 x 104, and its output, 81
# frames of 832 x 480).  Channel counts inside the decoder are not on the
# pages: 128 is this workload's reading.

TAG_CONV_X = 20
TAG_CONV_W = 21
TAG_CONV_B = 22


@dataclass(frozen=True)
class ConvWorkload:
    """One causal 3x3x3 convolution: input [T][H][W][ci] -> output [T][H][W][co]."""

    wid: int
    name: str
    T: int
    H: int
    W: int
    ci: int
    co: int

    @property
    def positions(self) -> int:
        return self.T * self.H * self.W

    @property
    def flops(self) -> float:
        return 2.0 * self.positions * self.co * 27 * self.ci


CONV_TINY = ConvWorkload(wid=40, name="conv_tiny", T=3, H=5, W=7, ci=16, co=128)
# a ragged last tile of positions, two blocks of output channels
CONV_MID = ConvWorkload(wid=41, name="conv_mid", T=4, H=9, W=13, ci=64, co=256)
# the decoder's first convolution: the 16-channel latent at 21 x 60 x 104
VAE_CONV_IN = ConvWorkload(wid=42, name="vae_conv_in", T=21, H=60, W=104, ci=16, co=128)
# a convolution inside the decoder at the latent resolution, 128 -> 128
VAE_CONV = ConvWorkload(wid=43, name="vae_conv", T=21, H=60, W=104, ci=128, co=128)

CONV_ALL = {c.name: c for c in (CONV_TINY, CONV_MID, VAE_CONV_IN, VAE_CONV)}


def conv_tensors(c: ConvWorkload):
    """Input x ~ N(0, 1) and weights w ~ N(0, 1/(27 ci)) as bf16 bits
    ([T][H][W][ci], [co][3][3][3][ci]), bias ~ N(0, 0.01) fp32 [co]."""
    gx = np.random.Generator(np.random.PCG64(np.random.SeedSequence([0, c.wid, TAG_CONV_X])))
    gw = np.random.Generator(np.random.PCG64(np.random.SeedSequence([0, c.wid, TAG_CONV_W])))
    gb = np.random.Generator(np.random.PCG64(np.random.SeedSequence([0, c.wid, TAG_CONV_B])))
    x = f32_to_bf16_bits(gx.standard_normal((c.T, c.H, c.W, c.ci), dtype=np.float32))
    w = gw.standard_normal((c.co, 3, 3, 3, c.ci), dtype=np.float32)
    w = f32_to_bf16_bits((w.astype(np.float64) / np.sqrt(27.0 * c.ci)).astype(np.float32))
    b = (gb.standard_normal(c.co, dtype=np.float32) * np.float32(0.1)).astype(np.float32)
    return x, w, b
