"""ust_lowrank_proj_static: the low-rank projection with its rank-r
intermediate in the library's fixed device array instead of a caller
buffer, for callers that cannot allocate.  Checked through the C ABI
against ust_lowrank_proj (same kernels: bit for bit) and against the fp64
oracle, on two calls in a row, the second smaller than the first, so a
stale intermediate from the first call would show."""
import numpy as np
import pytest
import torch

import causal_video_diffusion_amd as cvd
from causal_video_diffusion_amd import _binding as B
from causal_video_diffusion_amd import path as P
from causal_video_diffusion_amd import workload as wl
import oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load()


def _operands(w, M, r):
    """X [M][hidden] and the SVD factors of W_v at rank r, bf16 bits."""
    x = wl.activations(w, 5)[:M]
    a, b = wl.svd_factors_bf16(w, wl.TAG_WV, r)
    return x, a, b


def test_static_scratch_matches_caller_buffer():
    cases = [(wl.WAN_WINDOW, 4680, 512), (wl.MID, 200, 64)]   # second call smaller
    for w, M, r in cases:
        print(f"[lowrank static {w.name}: M={M} K={w.hidden} r={r}]", flush=True)
        x, a, b = _operands(w, M, r)
        lr = P.LowRank.from_bits(a, b)
        xd = P.to_device_bf16(x)
        N, K = w.hidden, w.hidden
        y_ref = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        t_work = torch.empty((M, r), dtype=torch.bfloat16, device="cuda")
        B.ust_lowrank_proj(xd, lr.a, lr.b, None, t_work, y_ref, M, K, r, N)
        y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        B.ust_lowrank_proj_static(xd, lr.a, lr.b, None, y, M, K, r, N)
        torch.cuda.synchronize()
        got, ref = P.from_device_bf16(y), P.from_device_bf16(y_ref)
        assert np.array_equal(got, ref), "static scratch differs from the caller buffer"
        rows = np.unique(np.concatenate([np.arange(16), np.arange(M - 16, M),
                                         np.random.default_rng(0).choice(M, 48, replace=False)]))
        f64 = wl.bf16_bits_to_f64
        want = O.lowrank_proj(f64(x)[rows], f64(a), f64(b))
        d = f64(got)[rows] - want
        ma, rl = float(np.abs(d).max()), float(np.linalg.norm(d) / np.linalg.norm(want))
        print(f"  max_abs={ma:.3e} rel_l2={rl:.3e}", flush=True)
        assert ma <= 2e-2 and rl <= 1e-2


def test_static_scratch_limit_and_dense_mode():
    w = wl.MID
    K = N = w.hidden
    lim = B.UST_LOWRANK_STATIC_MAX_ELEMS
    r = 64
    M = lim // r + 8                      # one row block past the limit
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    a = torch.zeros((r, K), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((N, r), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(cvd.UstError, match="UST_E_RANGE"):
        B.ust_lowrank_proj_static(x, a, b, None, y, M, K, r, N)
    # dense mode (b NULL) needs no scratch, at any M
    wd = torch.ones((N, K), dtype=torch.bfloat16, device="cuda") / 64
    B.ust_lowrank_proj_static(x[:100], wd, None, None, y[:100], 100, K, N, N)
    torch.cuda.synchronize()
    assert torch.all(y[:100] == 0)
