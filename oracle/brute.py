"""Brute-force scalar versions of the oracle's steps, for tiny inputs only.

TEST INFRASTRUCTURE ONLY.  Pure-Python loops over the definitions, written by
a different route from ust_oracle (complex multiplication for RoPE, a frame
membership test per key for the window, scalar sums for the products), so a
slip in either shows up as a mismatch.  Citations as in ust_oracle.
"""
from __future__ import annotations

import cmath
import math
from typing import List, Sequence


def rope_rotate(vec: Sequence[float], f: int, y: int, x: int,
                pairs: Sequence[int], theta: float) -> List[float]:
    """RoPE of one head vector as complex multiplication: the pair
    (v[2p], v[2p+1]) is the complex number v[2p] + i v[2p+1], multiplied by
    exp(i * pos * theta**(-j/n)) for pair j of its axis (UnStep, abstract:
    3-D RoPE from precomputed coefficients; axis split is a reading)."""
    out = []
    p = 0
    for axis_pairs, pos in zip(pairs, (f, y, x)):
        for j in range(axis_pairs):
            z = complex(vec[2 * p], vec[2 * p + 1])
            w = z * cmath.exp(1j * pos * math.pow(theta, -j / axis_pairs))
            out.extend([w.real, w.imag])
            p += 1
    return out


def in_window(frame: int, frame_start: int, chunk_frames: int, n_sink: int,
              n_recent: int) -> bool:
    """Is latent frame `frame` visible to the chunk starting at frame_start?"""
    if frame_start <= frame < frame_start + chunk_frames:
        return True
    if frame >= frame_start:
        return False
    if frame < n_sink:
        return True
    return n_recent < 0 or frame_start - frame <= n_recent


def ring_simulation(n_frames: int, n_slots: int, n_sink: int) -> List[int]:
    """Slot of each frame 0..n_frames-1 found by simulating the cache: sinks
    take the next free slot for good; every other frame takes a free slot if
    one is left, else the slot of the oldest non-sink frame still held."""
    held = {}                      # slot -> frame
    order = []                     # non-sink slots, oldest first
    out = []
    for f in range(n_frames):
        free = [s for s in range(n_slots) if s not in held]
        if f < n_sink:
            s = free[0]
        elif free:
            s = free[0]
            order.append(s)
        else:
            s = order.pop(0)
            order.append(s)
        held[s] = f
        out.append(s)
    return out


def attention(q_rows, keys, values, scale):
    """Softmax attention for lists of vectors: returns (outputs, lse)."""
    outs, lses = [], []
    for qv in q_rows:
        scores = [scale * sum(a * b for a, b in zip(qv, kv)) for kv in keys]
        m = max(scores)
        ex = [math.exp(s - m) for s in scores]
        tot = sum(ex)
        o = [sum(e * vv[d] for e, vv in zip(ex, values)) / tot
             for d in range(len(values[0]))]
        outs.append(o)
        lses.append(m + math.log(tot))
    return outs, lses


def window_attention(q, k_chunks, v_chunks, frame_start, chunk_frames,
                     grid_h, grid_w, n_sink, n_recent, pairs, theta, head):
    """Attention of a chunk's queries (un-rotated, [n][H][D] nested lists) for
    one head over every key of every frame so far that lies in the window.

    k_chunks / v_chunks: {frame: [T][H][D]} un-rotated keys and values of all
    frames written so far.  Keys are rotated here, at their own position."""
    T = grid_h * grid_w
    D = len(q[0][head])
    keys, values = [], []
    for f in sorted(k_chunks):
        if not in_window(f, frame_start, chunk_frames, n_sink, n_recent):
            continue
        for t in range(T):
            keys.append(rope_rotate(k_chunks[f][t][head], f, t // grid_w,
                                    t % grid_w, pairs, theta))
            values.append(list(v_chunks[f][t][head]))
    q_rows = []
    for n in range(len(q)):
        f = frame_start + n // T
        t = n % T
        q_rows.append(rope_rotate(q[n][head], f, t // grid_w, t % grid_w,
                                  pairs, theta))
    return attention(q_rows, keys, values, 1.0 / math.sqrt(D))


def matmul(a, b):
    """Plain triple loop over nested lists."""
    n, k, m = len(a), len(b), len(b[0])
    return [[sum(a[i][t] * b[t][j] for t in range(k)) for j in range(m)]
            for i in range(n)]


def shifted_sigma(raw: int, shift: float = 5.0, n_train: int = 1000) -> float:
    """Table 4's shift mapping written as 1 / ((1/u - 1) / shift + 1)."""
    u = raw / n_train
    if u == 0:
        return 0.0
    return 1.0 / ((1.0 / u - 1.0) / shift + 1.0)


def sample_chunk(dit, x_init: Sequence[float], noises, raw_steps: Sequence[int],
                 sigma_star: float, shift: float = 5.0):
    """The sampler of one chunk with scalar loops (UnStep, Tables 3 and 4;
    readings as in ust_oracle): renoising written as x0 + s (eps - x0).
    Returns (chunk kept, levels, labels)."""
    levels = [shifted_sigma(r, shift) for r in raw_steps] + [float(sigma_star)]
    x = [float(a) for a in x_init]
    seen, labels = [], []
    for i in range(len(raw_steps)):
        s, s_next = levels[i], levels[i + 1]
        v = dit(x, 1000.0 * s)
        seen.append(s)
        labels.append(1000.0 * s)
        est = [x[k] - s * v[k] for k in range(len(x))]
        if s_next == 0:
            x = est
        else:
            x = [est[k] + s_next * (noises[i][k] - est[k]) for k in range(len(x))]
    v = dit(x, 0.0)
    seen.append(levels[-1])
    labels.append(0.0)
    return [x[k] - levels[-1] * v[k] for k in range(len(x))], seen, labels


def conv3d_causal(x, w, bias=None):
    """Causal 3-D convolution as a scalar quadruple loop over the input
    positions each output reads (UnStep, abstract: the decoder's convolution
    kernels; causality and padding are readings): out[t][y][x][o] sums
    w[o][dt][dy][dx][i] x[t'][y'][x'][i] over t' = t - 2 .. t, y' = y - 1 ..
    y + 1, x' = x - 1 .. x + 1 inside the input, nested lists in and out."""
    T, H, W = len(x), len(x[0]), len(x[0][0])
    Ci, Co = len(x[0][0][0]), len(w)
    out = []
    for t in range(T):
        frame = []
        for y in range(H):
            row = []
            for xx in range(W):
                vals = []
                for o in range(Co):
                    acc = 0.0 if bias is None else float(bias[o])
                    for tp in range(t - 2, t + 1):
                        if tp < 0:
                            continue
                        for yp in range(y - 1, y + 2):
                            if yp < 0 or yp >= H:
                                continue
                            for xp in range(xx - 1, xx + 2):
                                if xp < 0 or xp >= W:
                                    continue
                                wk = w[o][tp - t + 2][yp - y + 1][xp - xx + 1]
                                for i in range(Ci):
                                    acc += wk[i] * x[tp][yp][xp][i]
                    vals.append(acc)
                row.append(vals)
            frame.append(row)
        out.append(frame)
    return out
