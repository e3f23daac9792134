"""GPU parity of the decoder convolution (ust_conv3d_causal) against the
fp64 oracle on the same bf16 inputs: max-abs 2e-2 and relative L2 1e-2, all
outputs; bit-exact where the arithmetic is exact (a delta kernel copies or
shifts the input: one product by 1.0 per output, then one rounding to bf16
of a bf16 value)."""
import numpy as np
import pytest
import torch

from causal_video_diffusion_amd import _binding as B
from causal_video_diffusion_amd import path as P
from causal_video_diffusion_amd import workload as wl
import oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load()


def _conv_gpu(c, x_bits, w_bits, bias):
    x = P.to_device_bf16(x_bits)
    w = P.to_device_bf16(w_bits)
    b = torch.from_numpy(bias).cuda() if bias is not None else None
    y = torch.full((c.T, c.H, c.W, c.co), float("nan"), dtype=torch.bfloat16, device="cuda")
    B.ust_conv3d_causal(x, w, b, y, c.T, c.H, c.W, c.ci, c.co)
    torch.cuda.synchronize()
    return P.from_device_bf16(y)


@pytest.mark.parametrize("name", ["conv_tiny", "conv_mid", "vae_conv_in", "vae_conv"])
def test_conv3d_matches_oracle(name):
    c = wl.CONV_ALL[name]
    print(f"[conv3d {name}: {c.T}x{c.H}x{c.W}, {c.ci} -> {c.co}]", flush=True)
    x, w, b = wl.conv_tensors(c)
    got = wl.bf16_bits_to_f64(_conv_gpu(c, x, w, b))
    ref = O.conv3d_causal(wl.bf16_bits_to_f64(x), wl.bf16_bits_to_f64(w), b.astype(np.float64))
    assert np.isfinite(got).all()
    d = got - ref
    ma = float(np.abs(d).max())
    rl = float(np.linalg.norm(d) / np.linalg.norm(ref))
    print(f"  {name}: max_abs={ma:.3e} rel_l2={rl:.3e}", flush=True)
    assert ma <= 2e-2 and rl <= 1e-2
    # the first frames see no earlier frames: frame 0 must equal the
    # convolution of frame 0 alone
    ref0 = O.conv3d_causal(wl.bf16_bits_to_f64(x)[:1], wl.bf16_bits_to_f64(w), b.astype(np.float64))
    assert np.max(np.abs(got[:1] - ref0)) <= 2e-2


@pytest.mark.parametrize("tap", [(2, 1, 1), (0, 1, 1), (1, 0, 2)])
def test_conv3d_delta_kernel_is_exact(tap):
    """Identity weights at one tap: the output is the input shifted by the
    tap, bit for bit, zero where the shift leaves the input."""
    c = wl.ConvWorkload(wid=44, name="conv_delta", T=5, H=9, W=13, ci=128, co=128)
    x, _, _ = wl.conv_tensors(c)
    w = np.zeros((c.co, 3, 3, 3, c.ci), np.uint16)
    dt, dy, dx = tap
    w[np.arange(c.co), dt, dy, dx, np.arange(c.ci)] = 0x3F80          # 1.0
    got = _conv_gpu(c, x, w, None)
    want = np.zeros_like(x)
    st, sy, sx = dt - 2, dy - 1, dx - 1                               # input offset of the tap
    T, H, W = c.T, c.H, c.W
    want[max(0, -st):T - max(0, st), max(0, -sy):H - max(0, sy), max(0, -sx):W - max(0, sx)] = \
        x[max(0, st):T + min(0, st), max(0, sy):H + min(0, sy), max(0, sx):W + min(0, sx)]
    assert np.array_equal(got, want)


def test_conv3d_deterministic_and_causal():
    """Two runs agree bit for bit; changing frames 2 and later leaves output
    frames 0 and 1 bit-identical."""
    c = wl.CONV_MID
    x, w, b = wl.conv_tensors(c)
    y1 = _conv_gpu(c, x, w, b)
    y2 = _conv_gpu(c, x, w, b)
    assert np.array_equal(y1, y2)
    x2 = x.copy()
    x2[2:] = wl.f32_to_bf16_bits(np.random.default_rng(5).standard_normal(x2[2:].shape).astype(np.float32))
    y3 = _conv_gpu(c, x2, w, b)
    assert np.array_equal(y1[:2], y3[:2])
    assert not np.array_equal(y1[2:], y3[2:])


# input widths 16 and 32 .. 512 (multiples of 32, including the 96 / 192 /
# 384 of some decoders), output widths that are multiples of 32 but not of
# the 128-channel tile, and degenerate and ragged grids: a single position,
# H = 1, W = 1, T = 1, fewer positions than one 512-position tile, a ragged
# last tile
_EDGE = [
    (45, 1, 1, 1, 32, 128),
    (46, 2, 1, 37, 32, 128),
    (47, 3, 7, 1, 128, 256),
    (48, 6, 11, 17, 32, 384),
    (49, 1, 30, 52, 64, 128),
    (50, 9, 6, 10, 16, 128),
    (51, 4, 5, 33, 128, 128),
    (52, 3, 8, 12, 96, 96),
    (53, 2, 9, 14, 192, 224),
    (54, 3, 6, 11, 384, 384),
    (55, 2, 5, 7, 512, 160),
    (56, 4, 6, 9, 256, 32),
]


@pytest.mark.parametrize("wid,T,H,W,ci,co", _EDGE)
def test_conv3d_edge_shapes(wid, T, H, W, ci, co):
    c = wl.ConvWorkload(wid=wid, name=f"conv_edge{wid}", T=T, H=H, W=W, ci=ci, co=co)
    print(f"[conv3d edge {T}x{H}x{W}, {ci} -> {co}]", flush=True)
    x, w, b = wl.conv_tensors(c)
    got = wl.bf16_bits_to_f64(_conv_gpu(c, x, w, b))
    ref = O.conv3d_causal(wl.bf16_bits_to_f64(x), wl.bf16_bits_to_f64(w), b.astype(np.float64))
    assert np.isfinite(got).all()
    d = got - ref
    ma = float(np.abs(d).max())
    rl = float(np.linalg.norm(d) / np.linalg.norm(ref))
    print(f"  max_abs={ma:.3e} rel_l2={rl:.3e}", flush=True)
    assert ma <= 2e-2 and rl <= 1e-2


def _stream_chunks(c, x_dev, w_dev, b_dev, chunk=3):
    """The clip through ust_conv3d_causal_stream, chunk by chunk: each call
    gets the previous chunk's last two input frames (zeros first) and the
    chunk's frames, contiguous."""
    outs = []
    zeros = torch.zeros((2, c.H, c.W, c.ci), dtype=torch.bfloat16, device="cuda")
    for t0 in range(0, c.T, chunk):
        n = min(chunk, c.T - t0)
        hist = zeros if t0 == 0 else (x_dev[t0 - 2:t0] if t0 >= 2 else
                                      torch.cat([zeros[:2 - t0], x_dev[:t0]]))
        x_ext = torch.cat([hist, x_dev[t0:t0 + n]]).contiguous()
        y = torch.full((n, c.H, c.W, c.co), float("nan"), dtype=torch.bfloat16, device="cuda")
        B.ust_conv3d_causal_stream(x_ext, w_dev, b_dev, y, n, c.H, c.W, c.ci, c.co)
        outs.append(y)
    torch.cuda.synchronize()
    return torch.cat(outs)


@pytest.mark.parametrize("name", ["conv_mid", "vae_conv"])
def test_conv3d_stream_chunks_equal_whole_clip(name):
    """Decoding the clip in chunks of three latent frames with the two
    history frames reproduces the whole-clip convolution bit for bit."""
    c = wl.CONV_ALL[name]
    print(f"[conv3d stream {name}: {c.T}x{c.H}x{c.W}, {c.ci} -> {c.co}]", flush=True)
    x, w, b = wl.conv_tensors(c)
    xd, wd, bd = P.to_device_bf16(x), P.to_device_bf16(w), torch.from_numpy(b).cuda()
    whole = torch.empty((c.T, c.H, c.W, c.co), dtype=torch.bfloat16, device="cuda")
    B.ust_conv3d_causal(xd, wd, bd, whole, c.T, c.H, c.W, c.ci, c.co)
    got = _stream_chunks(c, xd, wd, bd)
    assert torch.equal(got.view(torch.int16), whole.view(torch.int16))


@pytest.mark.parametrize("wid,T,H,W,ci,co", [(57, 3, 9, 13, 64, 128), (58, 1, 6, 11, 16, 96),
                                             (59, 2, 5, 7, 192, 160)])
def test_conv3d_stream_random_history_matches_oracle(wid, T, H, W, ci, co):
    """Random history frames (not a previous chunk of the same clip) against
    the oracle's history form."""
    c = wl.ConvWorkload(wid=wid, name=f"conv_hist{wid}", T=T, H=H, W=W, ci=ci, co=co)
    x, w, b = wl.conv_tensors(c)
    hist = wl.f32_to_bf16_bits(
        np.random.default_rng(wid).standard_normal((2, H, W, ci)).astype(np.float32))
    x_ext = np.concatenate([hist, x])
    y = torch.full((T, H, W, co), float("nan"), dtype=torch.bfloat16, device="cuda")
    B.ust_conv3d_causal_stream(P.to_device_bf16(x_ext), P.to_device_bf16(w),
                               torch.from_numpy(b).cuda(), y, T, H, W, ci, co)
    torch.cuda.synchronize()
    got = wl.bf16_bits_to_f64(P.from_device_bf16(y))
    ref = O.conv3d_causal(wl.bf16_bits_to_f64(x), wl.bf16_bits_to_f64(w), b.astype(np.float64),
                          history=wl.bf16_bits_to_f64(hist))
    d = got - ref
    ma = float(np.abs(d).max())
    rl = float(np.linalg.norm(d) / np.linalg.norm(ref))
    print(f"  history {T}x{H}x{W} {ci}->{co}: max_abs={ma:.3e} rel_l2={rl:.3e}", flush=True)
    assert np.isfinite(got).all() and ma <= 2e-2 and rl <= 1e-2
