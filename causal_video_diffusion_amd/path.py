"""Device-side drivers of the windowed chunk-attention path.

Thin Python over the C ABI (libust.so): allocation of the caller-owned
buffers with torch (device memory and streams only), and the order of calls
for one layer-chunk and for a whole clip.  Every arithmetic step runs in the
library's kernels.

Layer-chunk (UnStep, abstract): the value projection is the truncated-SVD
product (X A_r) B_r; the chunk's keys are RoPE'd and appended with the values
to the frame-slot ring; the chunk's queries attend over the limited window;
the output projection is again (O A_r) B_r.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Tuple

import numpy as np
import torch

from . import _binding as B


# ------------------------------------------------------------------ tensors

def to_device_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bf16 bit patterns -> bf16 device tensor (same bits)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def from_device_bf16(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> uint16 bit patterns on the host."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def output_major(bits: np.ndarray) -> np.ndarray:
    """[in][out] weight bits -> [out][in] (the layout the projection reads)."""
    return np.ascontiguousarray(bits.T)


# ------------------------------------------------------------------ state

class Ring:
    """Caller-owned KV ring: keys [n_slots][H][T][D], values [n_slots][H][D][TV]."""

    def __init__(self, g: B.Geom, n_slots: int, n_sink: int, device="cuda",
                 fill_bits: Optional[int] = None):
        T = g.grid_h * g.grid_w
        self.T = T
        self.TV = B.ust_v_row_len(T)
        self.k = torch.empty((n_slots, g.n_heads, T, g.head_dim),
                             dtype=torch.bfloat16, device=device)
        self.v = torch.empty((n_slots, g.n_heads, g.head_dim, self.TV),
                             dtype=torch.bfloat16, device=device)
        if fill_bits is not None:
            self.fill(fill_bits)
        self.n_slots, self.n_sink = n_slots, n_sink
        self.abi = B.kv(self.k, self.v, n_slots, n_sink)

    def fill(self, bits: int) -> None:
        val = np.array([bits], dtype=np.uint16).view(np.int16)[0]
        self.k.view(torch.int16).fill_(int(val))
        self.v.view(torch.int16).fill_(int(val))

    def host_k(self) -> np.ndarray:
        return from_device_bf16(self.k)

    def host_v_natural(self) -> np.ndarray:
        """Values as [n_slots][H][T][D] bits (transposed back for comparison)."""
        v = from_device_bf16(self.v)[..., :self.T]
        return np.ascontiguousarray(v.transpose(0, 1, 3, 2))


class RopeTable:
    """Cached fp32 cos/sin [n_frames][grid_h][grid_w][P] built on the GPU for the
    frames first_frame .. first_frame + n_frames - 1.

    The path reads only the rows of the chunk it processes, so a table of
    chunk_frames frames, rebuilt in place for each chunk (`rebuild`), serves a
    stream of any length in constant memory."""

    def __init__(self, g: B.Geom, n_frames: int, theta: float, device="cuda",
                 first_frame: int = 0):
        P = g.head_dim // 2
        self.g, self.theta = g, theta
        self.n_frames = n_frames
        self.cos = torch.empty((n_frames, g.grid_h, g.grid_w, P), dtype=torch.float32,
                               device=device)
        self.sin = torch.empty_like(self.cos)
        self.rebuild(first_frame)

    def rebuild(self, first_frame: int) -> None:
        """Refill the same buffers with the rows of frames first_frame onward."""
        B.ust_rope_table_build(self.g, self.n_frames, self.theta, self.cos, self.sin,
                               first_frame=first_frame)
        self.first_frame = first_frame


@dataclass
class LowRank:
    """Factors of one projection on the device, output-major: a [r][K], b [N][r]
    (b None for a dense weight given as a [N][K])."""
    a: torch.Tensor
    b: Optional[torch.Tensor]

    @property
    def rank(self) -> int:
        return self.a.shape[0]

    @property
    def k_in(self) -> int:
        return self.a.shape[1]

    @property
    def n_out(self) -> int:
        return self.b.shape[0] if self.b is not None else self.a.shape[0]

    @staticmethod
    def from_bits(a_bits: np.ndarray, b_bits: Optional[np.ndarray], device="cuda"):
        """a_bits [K][r] (= A_r), b_bits [r][N] (= B_r) or None."""
        a = to_device_bf16(output_major(a_bits), device)
        b = to_device_bf16(output_major(b_bits), device) if b_bits is not None else None
        return LowRank(a, b)


def lowrank_apply(p: LowRank, x: torch.Tensor, y: Optional[torch.Tensor] = None,
                  t_work: Optional[torch.Tensor] = None) -> torch.Tensor:
    M = x.shape[0]
    if y is None:
        y = torch.empty((M, p.n_out), dtype=torch.bfloat16, device=x.device)
    if p.b is not None and t_work is None:
        t_work = torch.empty((M, p.rank), dtype=torch.bfloat16, device=x.device)
    B.ust_lowrank_proj(x, p.a, p.b, None, t_work, y, M, p.k_in, p.rank, p.n_out)
    return y


def densify(a_bits: np.ndarray, b_bits: np.ndarray, device="cuda") -> torch.Tensor:
    """W_r = A_r B_r re-densified on the GPU (one bf16 rounding of the fp32
    product), returned output-major [N][K] for ust_qkv_append or a dense
    ust_lowrank_proj.  a_bits [K][r], b_bits [r][N]; the rank is zero-padded
    to a multiple of 8, which leaves the product unchanged.  Worth it when r
    is above the break-even K N / (K + N) (768 at 1536 x 1536)."""
    K, r = a_bits.shape
    N = b_bits.shape[1]
    rp = -(-r // 8) * 8
    a_pad = np.zeros((K, rp), np.uint16)
    a_pad[:, :r] = a_bits
    b_pad = np.zeros((rp, N), np.uint16)
    b_pad[:r] = b_bits
    # W_r^T = B_r^T A_r^T: x = B_r^T [N][rp] (B_r output-major), weight rows =
    # rows of A_r [K][rp] (A_r as stored, input-major)
    x = to_device_bf16(output_major(b_pad), device)
    a = to_device_bf16(a_pad, device)
    y = torch.empty((N, K), dtype=torch.bfloat16, device=device)
    B.ust_lowrank_proj(x, a, None, None, None, y, N, rp, K, K)
    return y


def qkv_weights(wq_bits: np.ndarray, wk_bits: np.ndarray, wv, device="cuda") -> torch.Tensor:
    """The fused projection's weight [3 H D][hidden], output-major: W_q, W_k
    ([in][out] bits) and W_v, given as [in][out] bits or as a device tensor
    already output-major (e.g. from densify)."""
    parts = [to_device_bf16(output_major(wq_bits), device),
             to_device_bf16(output_major(wk_bits), device),
             wv if isinstance(wv, torch.Tensor) else to_device_bf16(output_major(wv), device)]
    return torch.cat(parts, dim=0).contiguous()


# ------------------------------------------------------------------ layer-chunk

def attn_units(g: B.Geom) -> int:
    """(head, 256-query tile) units of one chunk's attention."""
    n_q = g.grid_h * g.grid_w * g.chunk_frames
    return -(-n_q // 256) * g.n_heads


def pick_attn_schedule(g: B.Geom, device=None) -> str:
    """'split' when the chunk has more (head, query tile) units than the device
    has compute units, else 'whole'.  With at most one unit per CU every unit
    runs at once; splitting would only fill the idle CUs, which under a
    power-limited clock gains less than the merge costs (measured on the
    windowed Wan layer-chunk: 492 vs 496 µs).  With more units than CUs the
    whole schedule needs a partly empty extra round (720p: 516 units, 256 CUs:
    4138 vs 3040 µs)."""
    n_cu = torch.cuda.get_device_properties(device or torch.cuda.current_device()) \
        .multi_processor_count
    return "split" if attn_units(g) > n_cu else "whole"


@dataclass
class LayerBuffers:
    """Per-call output and scratch buffers, allocated once."""
    v: torch.Tensor        # [NQ][H*D]
    o: torch.Tensor        # [NQ][H*D]
    y: torch.Tensor        # [NQ][H*D]
    t_v: Optional[torch.Tensor]
    t_o: Optional[torch.Tensor]
    lse: Optional[torch.Tensor]
    attn_work: Optional[torch.Tensor] = None   # key-split workspace, or None

    @staticmethod
    def alloc(n_q: int, hidden: int, n_heads: int, rank_v: Optional[int],
              rank_o: Optional[int], with_lse: bool = False, device="cuda",
              g: Optional[B.Geom] = None, schedule: str = "auto"):
        """With g given, the attention schedule: "split" allocates the
        workspace of the key-split attention (one workgroup per compute unit
        of the current device), "whole" does not, "auto" decides by
        pick_attn_schedule."""
        bf = dict(dtype=torch.bfloat16, device=device)
        work = None
        if schedule not in ("auto", "split", "whole"):
            raise ValueError(f"schedule {schedule!r}")
        if g is not None and schedule == "auto":
            schedule = pick_attn_schedule(g)
        if g is not None and schedule == "split":
            nbytes = B.ust_window_attn_work_bytes(g, 0)
            if nbytes <= 0:
                raise RuntimeError("ust_window_attn_work_bytes failed")
            work = torch.empty(nbytes // 4, dtype=torch.float32, device=device)
        return LayerBuffers(
            v=torch.empty((n_q, hidden), **bf), o=torch.empty((n_q, hidden), **bf),
            y=torch.empty((n_q, hidden), **bf),
            t_v=torch.empty((n_q, rank_v), **bf) if rank_v else None,
            t_o=torch.empty((n_q, rank_o), **bf) if rank_o else None,
            lse=torch.empty((n_heads, n_q), dtype=torch.float32, device=device)
            if with_lse else None,
            attn_work=work)


def v_into_ring(wv: LowRank, bufs: LayerBuffers) -> bool:
    """Whether the value projection can store V straight into the ring: a
    truncated-SVD projection (a second factor) whose rank is a multiple of 64,
    with its rank-r scratch in bufs."""
    return wv.b is not None and wv.rank % 64 == 0 and bufs.t_v is not None


def layer_chunk(g: B.Geom, ring: Ring, table: RopeTable, x: torch.Tensor,
                q: torch.Tensor, k_new: torch.Tensor, wv: LowRank, wo: LowRank,
                frame_start: int, n_recent: int, bufs: LayerBuffers,
                scale: float = 0.0) -> torch.Tensor:
    """One layer-chunk of the path; returns the output projection Y [NQ][H*D].

    x: hidden states [NQ][hidden]; q, k_new: [NQ][H*D] un-rotated (from the
    dense query/key projections).  The attention runs on the key-split
    schedule when bufs holds its workspace.  A truncated-SVD value projection
    whose rank is a multiple of 64 stores V straight into the ring, and the
    keys' RoPE and append ride in its first product's launch
    (ust_lowrank_proj_v_append with k_new); other value projections go
    through bufs.v and the full append."""
    if v_into_ring(wv, bufs):
        B.ust_lowrank_proj_v_append(g, ring.abi, x, wv.a, wv.b, bufs.t_v, wv.k_in, wv.rank,
                                    frame_start, k_new=k_new, cos_tab=table.cos,
                                    sin_tab=table.sin, n_tab_frames=table.n_frames,
                                    tab_first_frame=table.first_frame)
    else:
        lowrank_apply(wv, x, bufs.v, bufs.t_v)
        B.ust_kv_append(g, ring.abi, k_new, bufs.v, table.cos, table.sin,
                        table.n_frames, frame_start, tab_first_frame=table.first_frame)
    if bufs.attn_work is not None:
        B.ust_window_attn_split(g, ring.abi, q, table.cos, table.sin, table.n_frames,
                                frame_start, n_recent, scale, bufs.o, bufs.lse,
                                bufs.attn_work, 0, tab_first_frame=table.first_frame)
    else:
        B.ust_window_attn(g, ring.abi, q, table.cos, table.sin, table.n_frames,
                          frame_start, n_recent, scale, bufs.o, bufs.lse,
                          tab_first_frame=table.first_frame)
    lowrank_apply(wo, bufs.o, bufs.y, bufs.t_o)
    return bufs.y


def layer_chunk_fused(g: B.Geom, ring: Ring, table: RopeTable, x: torch.Tensor,
                      w_qkv: torch.Tensor, wo: LowRank, frame_start: int, n_recent: int,
                      bufs: LayerBuffers, q_buf: torch.Tensor,
                      scale: float = 0.0) -> torch.Tensor:
    """One layer-chunk with the fused projection: Q/K/V in one product whose
    epilogue rotates K and appends K and V to the ring, then the attention
    and the output projection.  x: [NQ][hidden]; q_buf: [NQ][H*D]."""
    hidden = x.shape[1]
    B.ust_qkv_append(g, ring.abi, x, w_qkv, hidden, table.cos, table.sin, table.n_frames,
                     frame_start, q_buf, tab_first_frame=table.first_frame)
    if bufs.attn_work is not None:
        B.ust_window_attn_split(g, ring.abi, q_buf, table.cos, table.sin, table.n_frames,
                                frame_start, n_recent, scale, bufs.o, bufs.lse,
                                bufs.attn_work, 0, tab_first_frame=table.first_frame)
    else:
        B.ust_window_attn(g, ring.abi, q_buf, table.cos, table.sin, table.n_frames,
                          frame_start, n_recent, scale, bufs.o, bufs.lse,
                          tab_first_frame=table.first_frame)
    lowrank_apply(wo, bufs.o, bufs.y, bufs.t_o)
    return bufs.y


# ------------------------------------------------------------------ clip

def clip_forwards(n_chunks: int, first_steps: int, later_steps: int,
                  clean_pass: bool) -> List[Tuple[int, int, bool]]:
    """(chunk, forward index, is clean-cache forward) in execution order
    (UnStep, Table 3: the first chunk runs first_steps denoising forwards, the
    later chunks later_steps, and each chunk one clean-cache forward that
    writes the cache last)."""
    seq = []
    for c in range(n_chunks):
        n = first_steps if c == 0 else later_steps
        seq.extend((c, i, False) for i in range(n))
        if clean_pass:
            seq.append((c, n, True))
    return seq


# ------------------------------------------------------------------ sampler

SAMPLER_RAW_STEPS_4 = (1000, 750, 500, 250)   # the few-step model's four (Table 4)
SAMPLER_RAW_STEPS_2 = (1000, 500)             # an UnStep later chunk's two (a reading)


def sample_chunk(dit, x: torch.Tensor, noises, raw_steps, sigma_star: float,
                 shift: float = 5.0):
    """One chunk of the sampler on the device (UnStep, Tables 3 and 4).

    A denoising forward per raw step, each followed by ust_flow_step, which
    renoises to the next level (the last step to sigma_star). Then come the
    label-0 clean-cache forward and its step to level 0. dit(x, t) returns the
    velocity as a bf16 device tensor shaped like x, for latent x at label t.
    x is the chunk's initial noise, fp32 on the device; it is updated in
    place. noises[i] is the fp32 draw for the renoising after step i (unused
    when that level is 0). Returns (x, the levels of the forwards, the labels
    passed)."""
    levels, labels = B.ust_sigma_schedule(list(raw_steps), shift)
    n = x.numel()
    seen, passed = [], []
    for i, (s, t) in enumerate(zip(levels, labels)):
        nxt = levels[i + 1] if i + 1 < len(levels) else float(sigma_star)
        v = dit(x, t)
        seen.append(s)
        passed.append(t)
        B.ust_flow_step(x, v, noises[i] if nxt != 0 else None, s, nxt, None, x, n)
    v = dit(x, 0.0)
    seen.append(float(sigma_star))
    passed.append(0.0)
    B.ust_flow_step(x, v, None, float(sigma_star), 0.0, None, x, n)
    return x, seen, passed
