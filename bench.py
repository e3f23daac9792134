#!/usr/bin/env python3
"""Benchmark of the windowed chunk-attention hot path on one MI355X.

A step is one layer-chunk of the path at the Wan2.1-1.3B windowed workload,
steady state (chunks 3, 4 and 5 in turn; window = 3 sink + 6 recent + 3
current frames = 18720 keys; 4680 queries; 12 heads x 128; rank-512 V/O):
    V = (X A_v) B_v  ->  RoPE-K + KV append  ->  window plan + RoPE-Q +
    windowed attention  ->  Y = (O A_o) B_o
with every input resident in HBM when the timed region starts (the ring holds
the window's earlier frames, written by the same path before timing).

The attention schedule is the path's own choice by default (`--schedule
auto`: the key-split ust_window_attn_split plus its merge kernel when the
chunk has more (head, query tile) units than the GPU has compute units, else
ust_window_attn with one workgroup per unit); `--schedule split|whole` forces
one.

Prints one JSON line.  `value` is the attention's algorithmic TFLOP per
layer-chunk divided by the whole step's time; `roofline` is the attention's
own rate, timed with HIP events on its stream inside the timed region (for
the split schedule the events span both the attention and the merge
kernels); `cpu_baseline` is the CPU fp64 oracle on a bounded sample of the
same layer-chunk.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 dense bf16 flop/clk/CU
PEAK_HBM_GBS = 8000.0
METRIC = ("windowed chunk-attn TFLOP/s + µs per layer-chunk (Wan-1.3B shape), "
          "% MFMA/HBM peak")

# HBM traffic of one steady-state attention (rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE per dispatch on this workload, scaled by the counter-to-byte
# factors of a 1 GiB device copy in the same run: read = 2 x FETCH_SIZE KiB,
# written = WRITE_SIZE KiB), per (workload, schedule), with the hash of the
# attention kernel's sources the counters were taken on.  The line reports
# the figure only while the sources still hash the same (null otherwise).
ATTN_SOURCES = ("window_attn.hip", "attn_schedule.h", "ust_device.h")
ATTN_TRAFFIC = {
    ("wan_window", "whole"): {"src_sha16": "cf5e64c3889d6500",
                              "bytes": (2 * 108159 + 17698) * 1024},
    # the split schedule: the attention and the merge kernel together
    ("wan_720p", "split"): {"src_sha16": "cf5e64c3889d6500",
                            "bytes": (2 * (588995 + 17004) + 62660 + 204) * 1024},
}
# the decoder convolution, per workload, same scaling and keying
CONV_SOURCES = ("conv3d.hip", "ust_device.h")
CONV_TRAFFIC = {
    "vae_conv": {"src_sha16": "a69f954fab1ff211", "bytes": (2 * 62222 + 32760) * 1024},
    "vae_conv_in": {"src_sha16": "a69f954fab1ff211", "bytes": (2 * 3970 + 32760) * 1024},
}
# the sampler's flow step at the Wan chunk latent, per launch averaged over
# one clip's 23 (16 renoising ones read the noise: FETCH 1478 KiB; 7
# clean-cache ones do not: 892 KiB; every one writes 1170 KiB), same scaling
SAMPLER_TRAFFIC_BYTES = round((2 * (16 * 1478 + 7 * 892) / 23 + 1170) * 1024)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", choices=("wan_window", "wan_720p", "wan_clip", "wan_fused",
                                            "wan_sampler", "vae_conv", "vae_conv_in"),
                    default="wan_window",
                    help="the windowed Wan2.1-1.3B layer-chunk (default); the same layer "
                         "at 720p (45x80 tokens/frame, rank 256); the whole 81-frame "
                         "clip schedule over 30 layers (a step is then one clip); or the "
                         "windowed layer-chunk with the fused Q/K/V projection and the "
                         "pages' rank 1413, re-densified")
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--schedule", choices=("auto", "split", "whole"), default="auto",
                    help="attention schedule: the path's choice (default), key-split "
                         "over one workgroup per CU, or one workgroup per head and "
                         "query tile")
    ap.add_argument("--cpu-reps", type=int, default=2,
                    help="layer-chunks the CPU oracle baseline runs")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="before timing, run one plain device copy of this many MiB "
                         "(a known-size reference for HBM traffic counters)")
    ap.add_argument("--no-calib", action="store_true",
                    help="skip the measured MFMA-rate and copy-rate calibration")
    return ap.parse_args()


def attn_flops(n_q, n_k, d, h):
    return 4.0 * n_q * n_k * d * h      # QK^T and PV, 2 flop per multiply-add


def source_sha16(names):
    """sha256 (first 16 hex digits) of a kernel's sources under csrc/."""
    import hashlib
    hs = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "causal_video_diffusion_amd", "csrc", name), "rb") as f:
            hs.update(f.read())
    return hs.hexdigest()[:16]


def attn_source_sha16():
    """sha256 (first 16 hex digits) of the attention kernel's sources."""
    return source_sha16(ATTN_SOURCES)


def attn_traffic(workload, schedule):
    """Counter-measured bytes of the attention, if taken on these sources."""
    t = ATTN_TRAFFIC.get((workload, schedule))
    return t["bytes"] if t and t["src_sha16"] == attn_source_sha16() else None


def conv_traffic(workload):
    """Counter-measured bytes of the decoder convolution, if taken on these sources."""
    t = CONV_TRAFFIC.get(workload)
    return t["bytes"] if t and t["src_sha16"] == source_sha16(CONV_SOURCES) else None


def reference_copy(mb):
    """One plain device copy of `mb` MiB: the known-size reference the HBM
    traffic counters are scaled by (its FETCH_SIZE and WRITE_SIZE)."""
    import torch
    n = mb << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def pct(xs):
    """median, p10, p90 of a list of times."""
    import numpy as np
    a = np.asarray(xs, np.float64)
    return {"median": round(float(np.median(a)), 3), "p10": round(float(np.percentile(a, 10)), 3),
            "p90": round(float(np.percentile(a, 90)), 3)}


def calibrate(stream):
    """Rates this GPU sustains, measured in this process before the timed
    region: the bf16 MFMA rate of a kernel that only issues MFMAs on
    pseudo-random operands (one workgroup of 8 waves per compute unit,
    ~10 ms; the power-limited clock makes the rate depend on the operands'
    bits, and random ones are what real data looks like), and a plain 1 GiB
    device copy (bytes read + written per second)."""
    import torch
    from causal_video_diffusion_amd import _binding as B
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(cus * 8, dtype=torch.float32, device="cuda")
    iters = 4000
    for _ in range(3):
        B.ust_calib_mfma_bf16(cus, iters, out)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    reps, flops = 10, 0.0
    e0.record(stream)
    for _ in range(reps):
        flops += B.ust_calib_mfma_bf16(cus, iters, out)
    e1.record(stream)
    torch.cuda.synchronize()
    mfma_tflops = flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return {"mfma_bf16_TFLOPs": round(mfma_tflops, 1), "copy_GBs": round(copy_gbs, 1),
            "note": f"MFMA-only kernel (ust_calib_mfma_bf16: {cus} workgroups x 8 waves, 4 "
                    f"independent 32x32x16 bf16 chains per wave on pseudo-random operands, {reps} "
                    f"launches) and a 1 GiB "
                    f"device copy (read + written bytes), both timed with HIP events in this "
                    f"process before the timed region"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (got --gpus {args.gpus}); "
              "the path has no multi-GPU implementation", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import causal_video_diffusion_amd as cvd
    from causal_video_diffusion_amd import _binding as B
    from causal_video_diffusion_amd import path as P
    from causal_video_diffusion_amd import workload as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    B.load()
    torch.cuda.set_device(0)
    if args.workload == "wan_clip":
        return main_clip(args)
    if args.workload == "wan_fused":
        return main_fused(args)
    if args.workload == "wan_sampler":
        return main_sampler(args)
    if args.workload in ("vae_conv", "vae_conv_in"):
        return main_conv(args)
    w = wl.ALL[args.workload]
    C = 5                                   # last chunk prepared
    # Steady-state chunks timed in turn.  The windowed layer's 21-slot ring
    # keeps frames 0-17 at once, so chunks 3, 4 and 5 (12-frame windows
    # each) can run in any order; re-appending a chunk rewrites its slots
    # with the same values.  The 720p ring (15 slots) holds one steady
    # window at a time: chunk 5.
    steady = (3, 4, 5) if w.name == "wan_window" else (5,)
    F0 = 3 * C
    g = cvd.geom(*w.geom_tuple())
    stream = torch.cuda.current_stream()

    # ---- inputs, resident in HBM ----
    av, bv = wl.svd_factors_bf16(w, wl.TAG_WV, w.rank)
    ao, bo = wl.svd_factors_bf16(w, wl.TAG_WO, w.rank)
    wv, wo = P.LowRank.from_bits(av, bv), P.LowRank.from_bits(ao, bo)
    table = P.RopeTable(g, w.n_tab_frames, w.theta)
    ring = P.Ring(g, w.n_slots, w.n_sink, fill_bits=0x7FC1)
    bufs = P.LayerBuffers.alloc(w.n_q, w.hidden, w.n_heads, w.rank, w.rank)
    chunks = []
    for c in range(C + 1):
        chunks.append((P.to_device_bf16(wl.activations(w, c)),
                       P.to_device_bf16(wl.chunk_tokens(w, wl.TAG_Q, c).reshape(w.n_q, -1)),
                       P.to_device_bf16(wl.chunk_tokens(w, wl.TAG_K, c).reshape(w.n_q, -1))))
    for c in range(C):                      # fill the window's earlier frames
        x, q, k = chunks[c]
        P.layer_chunk(g, ring, table, x, q, k, wv, wo, 3 * c, w.n_recent, bufs)
    torch.cuda.synchronize()
    x, q, k = chunks[C]
    n_ks = {len(B.ust_window_plan(g, ring.abi, 3 * c, w.n_recent)[0]) * w.T for c in steady}
    assert len(n_ks) == 1, "the timed chunks have windows of one size"
    n_k = n_ks.pop()
    flops = attn_flops(w.n_q, n_k, w.head_dim, w.n_heads)
    schedule = P.pick_attn_schedule(g) if args.schedule == "auto" else args.schedule
    split = schedule == "split"
    if split:
        nbytes = B.ust_window_attn_work_bytes(g, 0)
        work = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")

    def attention(q, f0):
        if split:
            B.ust_window_attn_split(g, ring.abi, q, table.cos, table.sin, w.n_tab_frames, f0,
                                    w.n_recent, 0.0, bufs.o, None, work, 0)
        else:
            B.ust_window_attn(g, ring.abi, q, table.cos, table.sin, w.n_tab_frames, f0,
                              w.n_recent, 0.0, bufs.o, None)

    # step i runs the layer-chunk of chunk steady[i % len(steady)]
    # ev: None, or 4 events; all=False records only the two around the
    # attention kernel (each event costs ~2-3 µs of step time, so the timed
    # region carries only those; the per-stage split is a separate pass)
    # the value projection stores V straight into the ring and the keys'
    # RoPE + append ride in its first product's launch (rank a multiple of 64)
    v_ring = P.v_into_ring(wv, bufs)

    def v_proj_keys(xc, kc, c, keys=True):
        B.ust_lowrank_proj_v_append(g, ring.abi, xc, wv.a, wv.b, bufs.t_v, w.hidden, w.rank,
                                    3 * c, k_new=kc if keys else None, cos_tab=table.cos,
                                    sin_tab=table.sin, n_tab_frames=w.n_tab_frames)

    def step(i, ev=None, all=False):
        c = steady[i % len(steady)]
        xc, qc, kc = chunks[c]
        if ev is not None and all:
            ev[0].record(stream)
        if v_ring:
            v_proj_keys(xc, kc, c)
        else:
            P.lowrank_apply(wv, xc, bufs.v, bufs.t_v)
            B.ust_kv_append(g, ring.abi, kc, bufs.v, table.cos, table.sin, w.n_tab_frames, 3 * c)
        if ev is not None:
            ev[1].record(stream)
        attention(qc, 3 * c)
        if ev is not None:
            ev[2].record(stream)
        P.lowrank_apply(wo, bufs.o, bufs.y, bufs.t_o)
        if ev is not None and all:
            ev[3].record(stream)

    if args.calib_copy_mb:
        reference_copy(args.calib_copy_mb)

    calib = None if args.no_calib else calibrate(stream)

    for i in range(max(args.warmup, len(steady))):   # every timed chunk appended once
        step(i)
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(i, evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    attn_each = [1000.0 * e[1].elapsed_time(e[2]) for e in evs]
    attn_us = float(np.mean(attn_each))
    # one step spans the end of one attention to the end of the next
    step_each = [evs[i][2].elapsed_time(evs[i + 1][2]) for i in range(args.steps - 1)]

    # per-stage split, outside the timed region, with all four events
    sevs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, sevs[i], all=True)
    torch.cuda.synchronize()
    names = ["v_proj_k_append_us", "window_attn_us", "o_proj_us"]
    stage = {n: 1000.0 * float(np.mean([e[i].elapsed_time(e[i + 1]) for e in sevs]))
             for i, n in enumerate(names)}
    # what the keys add to the value projection's launch: 20 calls with and
    # 20 without them, back to back (no event between calls)
    if v_ring:
        def per_call(keys):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for j in range(20):
                c = steady[j % len(steady)]
                v_proj_keys(chunks[c][0], chunks[c][2], c, keys)
            e1.record(stream)
            torch.cuda.synchronize()
            return 1000.0 * e0.elapsed_time(e1) / 20
        with_k = float(np.median([per_call(True) for _ in range(3)]))
        without_k = float(np.median([per_call(False) for _ in range(3)]))
        stage["v_proj_with_keys_back_to_back_us"] = with_k
        stage["v_proj_alone_back_to_back_us"] = without_k
        stage["k_append_in_v_proj_us"] = with_k - without_k
    # the append alone (keys and values: the a3 entry point), 20 launches
    # back to back between two events (it is idempotent: the same values into
    # the same slots), so the per-launch time carries no event overhead; V is
    # the chunk's value projection, the bits the step stored in the ring
    P.lowrank_apply(wv, x, bufs.v, bufs.t_v)
    # one launch first: the step does not use this entry point, and a
    # kernel's first launch also loads its code
    B.ust_kv_append(g, ring.abi, k, bufs.v, table.cos, table.sin, w.n_tab_frames, F0)
    torch.cuda.synchronize()
    b0 = torch.cuda.Event(enable_timing=True)
    b1 = torch.cuda.Event(enable_timing=True)
    b0.record(stream)
    for _ in range(20):
        B.ust_kv_append(g, ring.abi, k, bufs.v, table.cos, table.sin, w.n_tab_frames, F0)
    b1.record(stream)
    torch.cuda.synchronize()
    stage["rope_k_append_batched_us"] = 1000.0 * b0.elapsed_time(b1) / 20
    # the append from HBM: reading 512 MiB before each append evicts its
    # inputs from L2 and the 256 MB MALL (a read leaves no dirty lines behind
    # whose write-back the append would pay for).  No event sits between a
    # flush and its append: 20 (flush, append) pairs back to back are timed
    # against 20 flushes alone, and the difference is the 20 cold appends.
    # (a float32 sum: torch reads the buffer once and writes one value; an
    # integer sum of bytes would first write a widened copy)
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    fsum = torch.empty((), dtype=torch.float32, device="cuda")

    def flush_read():
        torch.sum(flush, dim=0, out=fsum)

    def timed(op):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(20):
            flush_read()
            if op is not None:
                op()
        e1.record(stream)
        torch.cuda.synchronize()
        return 1000.0 * e0.elapsed_time(e1)

    def cold_us(op):
        timed(op)
        each = []
        for _ in range(5):
            pair_us, flush_us = timed(op), timed(None)
            each.append((pair_us - flush_us) / 20)
        return float(np.median(each))

    stage["rope_k_append_cold_us"] = cold_us(
        lambda: B.ust_kv_append(g, ring.abi, k, bufs.v, table.cos, table.sin, w.n_tab_frames, F0))
    # the same measurement for a plain device copy of the append's K and V
    # (read once, written once): what a cold launch of this size reaches
    csrc = torch.empty(2 * w.n_q * w.hidden, dtype=torch.bfloat16, device="cuda").normal_()
    cdst = torch.empty_like(csrc)
    stage["copy_same_bytes_cold_us"] = cold_us(lambda: cdst.copy_(csrc))
    del flush, csrc, cdst
    attn_tflops = flops / (attn_us * 1e-6) / 1e12
    append_bytes = 4.0 * w.n_q * w.hidden * 2 + w.n_q * (w.head_dim // 2) * 8
    # V and O projections: each (X A_r) B_r, 2 M K r + 2 M r N flop with N = K
    lowrank_flops = 2 * 4.0 * w.n_q * w.hidden * w.rank
    # the two projections' algorithmic bytes (X and Y, both factors) and the
    # roofline that bounds them: min(MFMA peak, intensity x HBM peak)
    lowrank_bytes = 2 * (2.0 * w.n_q * w.hidden * 2 + 2.0 * w.rank * w.hidden * 2)
    lowrank_roof = min(PEAK_BF16_TFLOPS, lowrank_flops / lowrank_bytes * PEAK_HBM_GBS / 1e3)
    # the two projections' stage times, without what the keys add
    lowrank_us = (stage["v_proj_k_append_us"] - stage.get("k_append_in_v_proj_us", 0.0)
                  + stage["o_proj_us"])

    result = {
        "metric": METRIC,
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name} layer-chunk: Wan2.1-1.3B self-attention layer, "
                        f"{w.n_heads} heads x {w.head_dim}, {w.grid_h}x{w.grid_w} = {w.T} "
                        f"tokens/frame, 3-frame chunk = {w.n_q} queries, window {w.n_sink} "
                        f"sink + {w.n_recent} recent + 3 current frames = {n_k} keys, "
                        f"{w.n_slots}-slot ring, rank-{w.rank} V/O, steady-state chunk"
                        + (f"s {', '.join(map(str, steady))} in turn" if len(steady) > 1
                           else f" {steady[0]}"),
            "n_q": w.n_q, "n_k": n_k, "n_heads": w.n_heads, "head_dim": w.head_dim,
            "rank": w.rank, "attn_gflop": round(flops / 1e9, 2),
            "schedule": schedule,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(attn_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": attn_traffic(w.name, schedule),
            "kernel": ("window_attn_kernel<128> + window_attn_combine_kernel (one span)" if split
                       else "window_attn_kernel<128>"),
            "kernel_us": round(attn_us, 2),
            "kernel_us_spread": pct(attn_each),
            "attn_src_sha16": attn_source_sha16(),
        },
        "ms_per_step_spread": pct(step_each),
        "stages_us": {k: round(v, 2) for k, v in stage.items()},
        "stages_note": "separate untimed pass with an event between every stage "
                       "(each event adds ~2-3 us; stage times include launch gaps); "
                       "v_proj_k_append_us: the value projection storing V straight into the "
                       "ring with the keys' RoPE + append in its first product's launch "
                       "(ust_lowrank_proj_v_append with k_new); k_append_in_v_proj_us: what "
                       "the keys add to that call, 20 calls with and 20 without them back to "
                       "back; the low-rank V/O rate leaves that out; "
                       "rope_k_append_batched_us: 20 full appends (keys and values, "
                       "ust_kv_append) back to back, per launch "
                       "(no event overhead; inputs warm); rope_k_append_cold_us: 20 "
                       "(512 MiB read, append) pairs minus 20 reads alone, per append, "
                       "median of 5 (no event between a read and its append); the 60% "
                       "HBM target is compared with this cold figure; copy_same_bytes_cold_us: "
                       "the same measurement for a plain device copy of the append's K and V "
                       "(28.8 MB read, 28.8 MB written), what a cold launch of that size reaches",
        "stages": {
            "rope_k_append_batched_hbm_frac": round(
                append_bytes / (stage["rope_k_append_batched_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "rope_k_append_cold_hbm_frac": round(append_bytes / (stage["rope_k_append_cold_us"]
                                                                 * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "copy_same_bytes_cold_hbm_frac": round(4.0 * w.n_q * w.hidden * 2 / (
                stage["copy_same_bytes_cold_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "lowrank_v_o_TFLOPs": round(lowrank_flops / (lowrank_us * 1e-6) / 1e12, 1),
            "lowrank_v_o_roofline_TFLOPs": round(lowrank_roof, 1),
            "lowrank_v_o_frac_of_roofline": round(
                lowrank_flops / (lowrank_us * 1e-6) / 1e12 / lowrank_roof, 4),
        },
        "targets": {
            "attention_frac_of_bf16_peak": {"target": 0.5, "got": round(attn_tflops / PEAK_BF16_TFLOPS, 4)},
            "rope_k_append_cold_hbm_frac": {"target": 0.6, "got": round(
                append_bytes / (stage["rope_k_append_cold_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
        },
    }
    if calib is not None:
        result["calibration"] = calib
        result["roofline"]["measured_peak"] = calib["mfma_bf16_TFLOPs"]
        result["roofline"]["frac_of_measured_peak"] = round(attn_tflops / calib["mfma_bf16_TFLOPs"], 4)
        result["stages"]["rope_k_append_cold_frac_of_measured_copy"] = round(
            append_bytes / (stage["rope_k_append_cold_us"] * 1e-6) / 1e9 / calib["copy_GBs"], 4)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, C, args.cpu_reps)
    print(json.dumps(result), flush=True)


def main_fused(args):
    """The windowed Wan layer-chunk (chunk 5, steady state) with the fused
    projection: one product X [W_q | W_k | W_v]^T whose epilogue rotates K
    and appends K and V to the ring (ust_qkv_append), the attention, and the
    output projection.  V and O use the pages' SVD rank 1413 (0.92 x 1536),
    above the 768 break-even, so both run dense with W_r = A_r B_r
    re-densified once.  Unlike the default step, this one includes the Q and
    K projections."""
    import numpy as np
    import torch

    import causal_video_diffusion_amd as cvd
    from causal_video_diffusion_amd import _binding as B
    from causal_video_diffusion_amd import path as P
    from causal_video_diffusion_amd import workload as wl

    w = wl.WAN_WINDOW
    C, F0, rank = 5, 15, 1413
    g = cvd.geom(*w.geom_tuple())
    stream = torch.cuda.current_stream()
    av, bv = wl.svd_factors_bf16(w, wl.TAG_WV, rank)
    ao, bo = wl.svd_factors_bf16(w, wl.TAG_WO, rank)
    w_qkv = P.qkv_weights(wl.dense_weight_bf16(w, wl.TAG_WQ), wl.dense_weight_bf16(w, wl.TAG_WK),
                          P.densify(av, bv))
    wo = P.LowRank(P.densify(ao, bo), None)
    table = P.RopeTable(g, w.n_tab_frames, w.theta)
    ring = P.Ring(g, w.n_slots, w.n_sink, fill_bits=0x7FC1)
    bufs = P.LayerBuffers.alloc(w.n_q, w.hidden, w.n_heads, None, None, g=g)
    schedule = "split" if bufs.attn_work is not None else "whole"
    qbuf = torch.empty((w.n_q, w.hidden), dtype=torch.bfloat16, device="cuda")
    xs = [P.to_device_bf16(wl.activations(w, c)) for c in range(C + 1)]
    for c in range(C):
        P.layer_chunk_fused(g, ring, table, xs[c], w_qkv, wo, 3 * c, w.n_recent, bufs, qbuf)
    torch.cuda.synchronize()
    x = xs[C]
    n_k = len(B.ust_window_plan(g, ring.abi, F0, w.n_recent)[0]) * w.T
    flops = attn_flops(w.n_q, n_k, w.head_dim, w.n_heads)
    if args.calib_copy_mb:
        reference_copy(args.calib_copy_mb)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        B.ust_qkv_append(g, ring.abi, x, w_qkv, w.hidden, table.cos, table.sin, w.n_tab_frames,
                         F0, qbuf)
        if ev is not None:
            ev[1].record(stream)
        if bufs.attn_work is not None:
            B.ust_window_attn_split(g, ring.abi, qbuf, table.cos, table.sin, w.n_tab_frames, F0,
                                    w.n_recent, 0.0, bufs.o, None, bufs.attn_work, 0)
        else:
            B.ust_window_attn(g, ring.abi, qbuf, table.cos, table.sin, w.n_tab_frames, F0,
                              w.n_recent, 0.0, bufs.o, None)
        if ev is not None:
            ev[2].record(stream)
        P.lowrank_apply(wo, bufs.o, bufs.y)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    sevs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for e in sevs:
        step(e)
    torch.cuda.synchronize()
    names = ["qkv_proj_rope_k_append_us", "window_attn_us", "o_proj_us"]
    stage = {n: round(1000.0 * float(np.mean([e[i].elapsed_time(e[i + 1]) for e in sevs])), 2)
             for i, n in enumerate(names)}

    # The fused projection against the separate path it replaces (three dense
    # projections, then ust_kv_append rotating K and appending K and V into a
    # ring of its own), each launched 20 times back to back with no event in
    # between, alternating, 5 rounds; per call, median over the rounds.
    HD = w.n_heads * w.head_dim
    ring_sep = P.Ring(g, w.n_slots, w.n_sink, fill_bits=0x7FC1)
    ysep = [torch.empty((w.n_q, HD), dtype=torch.bfloat16, device="cuda") for _ in range(3)]

    def fused_only():
        B.ust_qkv_append(g, ring.abi, x, w_qkv, w.hidden, table.cos, table.sin, w.n_tab_frames,
                         F0, qbuf)

    def separate_only():
        for i in range(3):
            B.ust_lowrank_proj(x, w_qkv[i * HD:(i + 1) * HD], None, None, None, ysep[i], w.n_q,
                               w.hidden, HD, HD)
        B.ust_kv_append(g, ring_sep.abi, ysep[1], ysep[2], table.cos, table.sin, w.n_tab_frames,
                        F0)

    def back_to_back(fn, reps=20):
        for _ in range(3):
            fn()
        b0 = torch.cuda.Event(enable_timing=True)
        b1 = torch.cuda.Event(enable_timing=True)
        b0.record(stream)
        for _ in range(reps):
            fn()
        b1.record(stream)
        torch.cuda.synchronize()
        return 1000.0 * b0.elapsed_time(b1) / reps

    pair = {"fused": [], "separate": []}
    for _ in range(5):
        pair["fused"].append(back_to_back(fused_only))
        pair["separate"].append(back_to_back(separate_only))
    stage["qkv_fused_back_to_back_us"] = round(float(np.median(pair["fused"])), 2)
    stage["qkv_separate_back_to_back_us"] = round(float(np.median(pair["separate"])), 2)
    attn_tflops = flops / (stage["window_attn_us"] * 1e-6) / 1e12
    qkv_flops = 3 * 2.0 * w.n_q * w.hidden * w.n_heads * w.head_dim
    o_flops = 2.0 * w.n_q * w.hidden * w.hidden
    result = {
        "metric": METRIC,
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "wan_fused layer-chunk: the wan_window layer-chunk (4680 queries, "
                        "18720 window keys, 12 heads x 128) with one fused Q/K/V projection "
                        "(RoPE-K and the K/V append in its epilogue) and V/O at SVD rank 1413 "
                        "re-densified; the step includes the Q and K projections",
            "n_q": w.n_q, "n_k": n_k, "rank": rank, "attn_gflop": round(flops / 1e9, 2),
            "schedule": schedule,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(attn_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
            # the same attention kernel at the same shape and schedule as
            # the windowed layer-chunk's line: its counter-measured bytes
            "traffic": attn_traffic(w.name, schedule),
            "kernel": "window_attn_kernel<128> (per-stage pass)",
        },
        "stages_us": stage,
        "stages": {
            "qkv_TFLOPs": round(qkv_flops / (stage["qkv_proj_rope_k_append_us"] * 1e-6) / 1e12, 1),
            "o_proj_TFLOPs": round(o_flops / (stage["o_proj_us"] * 1e-6) / 1e12, 1),
            "qkv_fused_gain_vs_separate": round(
                stage["qkv_separate_back_to_back_us"] / stage["qkv_fused_back_to_back_us"] - 1.0, 4),
        },
        "stages_note": "separate untimed pass with events between the stages (each event "
                       "adds ~2-3 us; stage times include launch gaps); "
                       "qkv_fused_back_to_back_us / qkv_separate_back_to_back_us: the fused "
                       "projection + append, and the three dense projections + ust_kv_append it "
                       "replaces, each 20 times back to back, alternating, median of 5 rounds, "
                       "per call; qkv_fused_gain_vs_separate = separate / fused - 1",
    }
    print(json.dumps(result), flush=True)


def main_sampler(args):
    """The chunk sampler over one UnStep clip (Tables 3 and 4): 7 chunks of
    the Wan latent (3 x 16 x 60 x 104 fp32 each); chunk 0 takes four
    denoising steps, the later chunks two, and each chunk then the
    clean-cache step (sigma* = 0.02), 23 ust_flow_step launches per clip.
    No DiT runs: each forward's velocity is a pre-drawn bf16 stand-in, so the
    step is the sampler's own HBM traffic.  A step is one clip."""
    import numpy as np
    import torch

    from causal_video_diffusion_amd import _binding as B
    from causal_video_diffusion_amd import path as P
    from causal_video_diffusion_amd import workload as wl

    w = wl.WAN_CLIP
    n = int(np.prod(wl.latent_shape(w)))
    n_chunks, s_star = 7, 0.02
    plan = []                   # (chunk, forward, sigma, sigma_next) in clip order
    for c in range(n_chunks):
        steps = P.SAMPLER_RAW_STEPS_4 if c == 0 else P.SAMPLER_RAW_STEPS_2
        levels, _ = B.ust_sigma_schedule(list(steps))
        for i, sg in enumerate(levels):
            plan.append((c, i, sg, levels[i + 1] if i + 1 < len(levels) else s_star))
        plan.append((c, len(levels), s_star, 0.0))
    assert len(plan) == 23
    lat0 = [torch.from_numpy(wl.latent_noise(w, c, 0)).cuda() for c in range(n_chunks)]
    lat = [t.clone() for t in lat0]
    noise = [[torch.from_numpy(wl.latent_noise(w, c, i + 1)).cuda() for i in range(4)]
             for c in range(n_chunks)]
    vel = [[P.to_device_bf16(wl.stand_in_velocity(w, c, f)) for f in range(5)]
           for c in range(n_chunks)]
    # algorithmic bytes: x (4 B) and v (2 B) read, x_next (4 B) written, and
    # the noise (4 B) read when renoising to a level above 0
    nbytes = [n * (14 if sn != 0 else 10) for (_, _, _, sn) in plan]
    stream = torch.cuda.current_stream()

    def clip():
        for (c, f, sg, sn) in plan:
            B.ust_flow_step(lat[c], vel[c][f], noise[c][f] if sn != 0 else None, sg, sn, None,
                            lat[c], n)

    for _ in range(args.warmup):
        clip()
    for t, t0 in zip(lat, lat0):
        t.copy_(t0)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        clip()
    e1.record(stream)
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / args.steps
    # the same clip captured in a HIP graph (no memset nodes) and replayed:
    # the launch cost a DiT pipeline that captures its forwards would see
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        clip()
    stream.wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        clip()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_clip = e0.elapsed_time(e1) / args.steps
    us_per_launch = 1000.0 * ms_per_clip / len(plan)
    gbs = sum(nbytes) / (ms_per_clip * 1e-3) / 1e9
    # the same kernel over all seven chunks' latents at once (29 MB): its rate
    # away from the launch-latency regime of one 1.2 MB chunk
    big = torch.cat(lat0)
    bv = torch.cat([vel[c][0] for c in range(n_chunks)])
    bz = torch.cat([noise[c][0] for c in range(n_chunks)])
    for _ in range(5):
        B.ust_flow_step(big, bv, bz, 0.9375, 0.8333333, None, big, big.numel())
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(50):
        B.ust_flow_step(big, bv, bz, 0.9375, 0.8333333, None, big, big.numel())
    e1.record(stream)
    torch.cuda.synchronize()
    big_us = 1000.0 * e0.elapsed_time(e1) / 50
    big_gbs = big.numel() * 14 / (big_us * 1e-6) / 1e9
    result = {
        "metric": "chunk-sampler step GB/s (ust_flow_step at the Wan chunk latent), % HBM peak",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_clip, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "wan_sampler: one UnStep clip of the chunk sampler, 7 chunks of the Wan "
                        "latent 3x16x60x104 fp32 (299520 elements); 4 denoising steps for chunk "
                        "0, 2 for each later chunk, then each chunk's clean-cache step at "
                        "sigma* 0.02: 23 flow steps; velocities pre-drawn (no DiT); a step is "
                        "one clip, replayed from a HIP graph",
            "latent_elems": n, "launches_per_clip": len(plan),
            "bytes_per_clip": int(sum(nbytes)),
            "eager_ms_per_clip": round(eager_ms, 4),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": SAMPLER_TRAFFIC_BYTES,
            "kernel": "flow_step_kernel (23 graph-replayed launches, per-launch average "
                      "including the gaps between them)",
            "kernel_us": round(us_per_launch, 2),
        },
        "all_chunks_at_once": {
            "elems": int(big.numel()), "us": round(big_us, 2), "GBs": round(big_gbs, 1),
            "hbm_frac": round(big_gbs / PEAK_HBM_GBS, 4),
        },
    }
    if not args.no_cpu_baseline:
        import oracle as O
        cpu_lat = [wl.latent_noise(w, c, 0).astype(np.float64) for c in range(n_chunks)]
        cpu_noise = [[wl.latent_noise(w, c, i + 1) for i in range(4)] for c in range(n_chunks)]
        cpu_vel = [[wl.bf16_bits_to_f64(wl.stand_in_velocity(w, c, f)) for f in range(5)]
                   for c in range(n_chunks)]
        t0 = time.perf_counter()
        reps = 2
        for _ in range(reps):
            for (c, f, sg, sn) in plan:
                _, cpu_lat[c] = O.flow_step(cpu_lat[c], cpu_vel[c][f],
                                            cpu_noise[c][f] if sn != 0 else None, sg, sn)
        cpu_s = (time.perf_counter() - t0) / reps
        result["cpu_baseline"] = {
            "value": round(sum(nbytes) / cpu_s / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "ms_per_step": round(cpu_s * 1e3, 1),
            "sample": f"the whole clip's 23 flow steps in fp64 NumPy, {reps} times; value = the "
                      "same algorithmic bytes / wall time (elementwise NumPy is single-threaded)",
        }
    print(json.dumps(result), flush=True)


def main_conv(args):
    """One causal 3x3x3 convolution of the decoder runtime stack (UnStep,
    abstract: VAE decoding with an optimised memory layout, precision and
    convolution kernels; Table 3: the decoder's input is 21 latent frames of
    16 x 60 x 104): channels last, bf16 with fp32 accumulation, at the latent
    resolution; vae_conv is 128 -> 128 channels, vae_conv_in the decoder's
    first convolution, 16 -> 128 (channel counts are a reading).  A step is
    one convolution."""
    import numpy as np
    import torch

    from causal_video_diffusion_amd import _binding as B
    from causal_video_diffusion_amd import path as P
    from causal_video_diffusion_amd import workload as wl

    c = wl.CONV_ALL[args.workload]
    stream = torch.cuda.current_stream()
    x, w, b = wl.conv_tensors(c)
    xd, wd, bd = P.to_device_bf16(x), P.to_device_bf16(w), torch.from_numpy(b).cuda()
    y = torch.empty((c.T, c.H, c.W, c.co), dtype=torch.bfloat16, device="cuda")
    if args.calib_copy_mb:
        reference_copy(args.calib_copy_mb)
    calib = None if args.no_calib else calibrate(stream)

    def step():
        B.ust_conv3d_causal(xd, wd, bd, y, c.T, c.H, c.W, c.ci, c.co)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # events only between groups of G back-to-back launches: an event pair
    # around every launch would add its own gap to a ~100 us kernel
    G = 5
    groups = max(1, args.steps // G)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(groups + 1)]
    evs[0].record(stream)
    for gi in range(groups):
        for _ in range(G):
            step()
        evs[gi + 1].record(stream)
    torch.cuda.synchronize()
    ms_per_step = evs[0].elapsed_time(evs[-1]) / (groups * G)
    each = [1000.0 * evs[i].elapsed_time(evs[i + 1]) / G for i in range(groups)]
    kern_us = float(np.mean(each))
    tflops = c.flops / (kern_us * 1e-6) / 1e12
    nbytes = 2 * c.positions * (c.ci + c.co) + 2 * c.co * 27 * c.ci + 4 * c.co
    result = {
        "metric": f"decoder causal conv3d TFLOP/s ({c.name}), % MFMA peak",
        "value": round(c.flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": groups * G,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{c.name}: causal 3x3x3 convolution, {c.T} frames x {c.H} x {c.W} "
                        f"(the decoder's latent resolution, Table 3), {c.ci} -> {c.co} channels, "
                        f"channels last, bf16 in and out, fp32 accumulation, bias; a step is "
                        f"one convolution",
            "gflop": round(c.flops / 1e9, 2), "algorithmic_MB": round(nbytes / 1e6, 2),
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": conv_traffic(args.workload),
            "kernel": f"conv3d_causal_kernel<{min(c.ci, 32)}, {c.ci}>",
            "kernel_us": round(kern_us, 2),
            "kernel_us_spread": pct(each),
            "timing": f"HIP events on the launch stream around groups of {G} back-to-back "
                      f"launches; kernel_us = group time / {G} (includes the launch gaps)",
        },
    }
    if calib is not None:
        result["calibration"] = calib
        result["roofline"]["measured_peak"] = calib["mfma_bf16_TFLOPs"]
        result["roofline"]["frac_of_measured_peak"] = round(tflops / calib["mfma_bf16_TFLOPs"], 4)
    if not args.no_cpu_baseline:
        import oracle as O
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            cores = 1
        xf, wf = wl.bf16_bits_to_f64(x), wl.bf16_bits_to_f64(w)
        bf = b.astype(np.float64)
        reps = 2
        tc = time.perf_counter()
        for _ in range(reps):
            O.conv3d_causal(xf, wf, bf)
        cpu_s = (time.perf_counter() - tc) / reps
        result["cpu_baseline"] = {
            "value": round(c.flops / cpu_s / 1e12, 5), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "ms_per_step": round(cpu_s * 1e3, 1),
            "sample": f"the whole convolution in fp64 NumPy (27 matrix products over the "
                      f"zero-padded input), {reps} times; cores = BLAS threads",
        }
    print(json.dumps(result), flush=True)


def main_clip(args):
    """The 81-frame clip (UnStep, Table 3): 7 chunks of 3 latent frames; chunk
    0 runs 4 denoising forwards and each later chunk 2, every chunk one more
    clean-cache forward; 23 forwards x 30 layers = 690 layer-chunks, each
    with its own weights and KV ring, in one stream.  Per layer-chunk: dense
    Q and K projections (harness support, reported apart), then the path.
    After each forward, the sampler steps the chunk's latent (ust_flow_step
    at Table 4's levels, the clean-cache one at sigma* = 0.02); its velocity
    is a pre-drawn stand-in, since the layers' outputs are not one.  A step
    is one whole clip."""
    import numpy as np
    import torch

    import causal_video_diffusion_amd as cvd
    from causal_video_diffusion_amd import _binding as B
    from causal_video_diffusion_amd import path as P
    from causal_video_diffusion_amd import workload as wl

    w = wl.WAN_CLIP
    g = cvd.geom(*w.geom_tuple())
    stream = torch.cuda.current_stream()
    sched = P.clip_forwards(w.n_chunks, w.first_steps, w.later_steps, w.clean_pass)
    table = P.RopeTable(g, w.n_tab_frames, w.theta)
    layers = []
    for layer in range(w.layers):
        if layer % 10 == 0:
            print(f"[bench clip] preparing layer {layer} of {w.layers}", file=sys.stderr, flush=True)
        av, bv = wl.svd_factors_bf16(w, wl.TAG_WV, w.rank, layer)
        ao, bo = wl.svd_factors_bf16(w, wl.TAG_WO, w.rank, layer)
        layers.append(dict(
            wq=P.LowRank(P.to_device_bf16(P.output_major(wl.dense_weight_bf16(w, wl.TAG_WQ, layer))), None),
            wk=P.LowRank(P.to_device_bf16(P.output_major(wl.dense_weight_bf16(w, wl.TAG_WK, layer))), None),
            wv=P.LowRank.from_bits(av, bv), wo=P.LowRank.from_bits(ao, bo),
            ring=P.Ring(g, w.n_slots, w.n_sink, fill_bits=0x7FC1)))
    xs = [P.to_device_bf16(wl.activations(w, c, s)) for (c, s, _) in sched]
    bufs = P.LayerBuffers.alloc(w.n_q, w.hidden, w.n_heads, w.rank, w.rank, g=g)
    schedule = "split" if bufs.attn_work is not None else "whole"
    qbuf = torch.empty((w.n_q, w.hidden), dtype=torch.bfloat16, device="cuda")
    kbuf = torch.empty_like(qbuf)
    # attention flops of every layer-chunk (window sizes from the host plan)
    n_keys = [len(B.ust_window_plan(g, layers[0]["ring"].abi, 3 * c, w.n_recent)[0]) * w.T
              for (c, _, _) in sched]
    flops = sum(w.layers * attn_flops(w.n_q, nk, w.head_dim, w.n_heads) for nk in n_keys)
    n_lc = len(sched) * w.layers
    # the sampler on each chunk's latent: (sigma, sigma_next) per forward
    n_lat = int(np.prod(wl.latent_shape(w)))
    s_star = 0.02
    samp = []
    for (c, i, clean) in sched:
        steps = P.SAMPLER_RAW_STEPS_4 if (c == 0 or w.later_steps == 4) else P.SAMPLER_RAW_STEPS_2
        lv, _ = B.ust_sigma_schedule(list(steps))
        if clean:
            samp.append((s_star, 0.0))
        else:
            samp.append((lv[i], lv[i + 1] if i + 1 < len(lv) else s_star))
    lat = [torch.from_numpy(wl.latent_noise(w, c, 0)).cuda() for c in range(w.n_chunks)]
    lat_noise = [[torch.from_numpy(wl.latent_noise(w, c, i + 1)).cuda() for i in range(4)]
                 for c in range(w.n_chunks)]
    lat_vel = [P.to_device_bf16(wl.stand_in_velocity(w, c, i)) for (c, i, _) in sched]

    def attention(ring, c):
        if bufs.attn_work is not None:
            B.ust_window_attn_split(g, ring.abi, qbuf, table.cos, table.sin, w.n_tab_frames,
                                    3 * c, w.n_recent, 0.0, bufs.o, None, bufs.attn_work, 0)
        else:
            B.ust_window_attn(g, ring.abi, qbuf, table.cos, table.sin, w.n_tab_frames, 3 * c,
                              w.n_recent, 0.0, bufs.o, None)

    # ev: None, or a list that receives 4 events per layer-chunk: before the
    # Q/K projections, before the path, around the attention
    def clip(ev=None):
        for fi, (c, _, _) in enumerate(sched):
            x = xs[fi]
            for L in layers:
                e = [torch.cuda.Event(enable_timing=True) for _ in range(5)] if ev is not None else None
                if e:
                    e[0].record(stream)
                P.lowrank_apply(L["wq"], x, qbuf)
                P.lowrank_apply(L["wk"], x, kbuf)
                if e:
                    e[1].record(stream)
                if P.v_into_ring(L["wv"], bufs):
                    B.ust_lowrank_proj_v_append(g, L["ring"].abi, x, L["wv"].a, L["wv"].b,
                                                bufs.t_v, w.hidden, w.rank, 3 * c, k_new=kbuf,
                                                cos_tab=table.cos, sin_tab=table.sin,
                                                n_tab_frames=w.n_tab_frames)
                else:
                    P.lowrank_apply(L["wv"], x, bufs.v, bufs.t_v)
                    B.ust_kv_append(g, L["ring"].abi, kbuf, bufs.v, table.cos, table.sin,
                                    w.n_tab_frames, 3 * c)
                if e:
                    e[2].record(stream)
                attention(L["ring"], c)
                if e:
                    e[3].record(stream)
                P.lowrank_apply(L["wo"], bufs.o, bufs.y, bufs.t_o)
                if e:
                    e[4].record(stream)
                    ev.append(e)
            sg, sn = samp[fi]
            i = sched[fi][1]
            B.ust_flow_step(lat[c], lat_vel[fi], lat_noise[c][i] if sn != 0 else None, sg, sn,
                            None, lat[c], n_lat)

    print("[bench clip] warm-up", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        clip()
    torch.cuda.synchronize()
    print("[bench clip] timing", file=sys.stderr, flush=True)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        clip()
    t1.record(stream)
    torch.cuda.synchronize()
    clip_ms = t0.elapsed_time(t1) / args.steps
    # split of one clip, outside the timed region (events add ~2-3 us each)
    evs = []
    clip(evs)
    torch.cuda.synchronize()
    qk_ms = sum(e[0].elapsed_time(e[1]) for e in evs)
    path_ms = sum(e[1].elapsed_time(e[4]) for e in evs)
    attn_ms = sum(e[2].elapsed_time(e[3]) for e in evs)
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": round(flops / (clip_ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(clip_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"wan_clip: 81-frame clip = {w.n_chunks} chunks x 3 latent frames, "
                        f"{len(sched)} forwards (4 + 2 per later chunk, + 1 clean-cache "
                        f"forward per chunk) x {w.layers} layers = {n_lc} layer-chunks; each "
                        f"Wan2.1-1.3B self-attention layer-chunk with dense Q/K projections, "
                        f"rank-{w.rank} V/O, window {w.n_sink} sink + {w.n_recent} recent + 3 "
                        f"current frames, {w.n_slots}-slot ring per layer; the chunk sampler "
                        f"steps each chunk's latent after each forward; a step is one clip",
            "layer_chunks": n_lc, "attn_tflop_per_clip": round(flops / 1e12, 2),
            "sampler_steps": len(samp),
            "schedule": schedule,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(attn_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": None,
            "kernel": "window_attn_kernel<128>, all 690 launches of one clip",
            "kernel_ms_per_clip": round(attn_ms, 3),
        },
        "clip_ms": round(clip_ms, 3),
        "layer_chunk_us_mean": round(1000.0 * clip_ms / n_lc, 2),
        "split_ms": {"qk_dense_proj": round(qk_ms, 3), "path": round(path_ms, 3),
                     "attention": round(attn_ms, 3)},
        "split_note": "one clip in a separate pass with events around each layer-chunk's "
                      "Q/K projections, its path (V projection, append, attention, O "
                      "projection) and its attention; events add ~2-3 us each",
    }
    if not args.no_cpu_baseline:
        cb = cpu_baseline(wl.WAN_WINDOW, 5, args.cpu_reps)
        rate = cb["value"] * 1e12               # oracle attention flop/s, steady layer-chunk
        cb["extrapolated_clip_s"] = round(flops / rate, 1)
        cb["sample"] = ("one steady-state layer-chunk of the clip's shape (the wan_window "
                        "layer-chunk), whole, timed; the clip's time is extrapolated from it "
                        "by attention flops over the 690 layer-chunks. " + cb["sample"])
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


def cpu_baseline(w, C, reps):
    """The CPU fp64 oracle, untuned, on the same layer-chunk: V projection,
    KV append, windowed attention of every query row, O projection; run
    `reps` times (setup of the earlier chunks' cache is not timed)."""
    import numpy as np
    import oracle as O
    from causal_video_diffusion_amd import workload as wl
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = 1
    f64 = wl.bf16_bits_to_f64
    cos, sin = O.rope_table(w.n_tab_frames, w.grid_h, w.grid_w, w.pairs, w.theta)
    cache = O.KVCache(w.n_slots, w.n_heads, w.T, w.head_dim)
    av, bv = wl.svd_factors_bf16(w, wl.TAG_WV, w.rank)
    ao, bo = wl.svd_factors_bf16(w, wl.TAG_WO, w.rank)
    for c in range(C):
        O.kv_append(cache, f64(wl.chunk_tokens(w, wl.TAG_K, c)),
                    f64(wl.chunk_tokens(w, wl.TAG_V, c)), cos, sin, 3 * c, 3,
                    w.grid_h, w.grid_w, w.n_slots, w.n_sink)
    xb = f64(wl.activations(w, C))
    kb = f64(wl.chunk_tokens(w, wl.TAG_K, C))
    qb = f64(wl.chunk_tokens(w, wl.TAG_Q, C))
    A_v, B_v, A_o, B_o = f64(av), f64(bv), f64(ao), f64(bo)
    t0 = time.perf_counter()
    for _ in range(reps):
        v = O.lowrank_proj(xb, A_v, B_v).reshape(w.n_q, w.n_heads, -1)
        O.kv_append(cache, kb, v, cos, sin, 3 * C, 3, w.grid_h, w.grid_w, w.n_slots, w.n_sink)
        o, _ = O.window_attn(cache, qb, cos, sin, 3 * C, 3, w.grid_h, w.grid_w, w.n_slots,
                             w.n_sink, w.n_recent)
        O.lowrank_proj(o.reshape(w.n_q, -1), A_o, B_o)
    dt = (time.perf_counter() - t0) / reps
    frames = O.window_frames(3 * C, 3, w.n_sink, w.n_recent)
    flops = attn_flops(w.n_q, len(frames) * w.T, w.head_dim, w.n_heads)
    return {
        "value": round(flops / dt / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "ms_per_step": round(dt * 1e3, 1),
        "sample": f"the same {w.name} steady-state layer-chunk, whole, {reps} times: fp64 "
                  f"V projection, KV append, attention of all {w.n_q} queries over "
                  f"{len(frames) * w.T} keys (materialised softmax in 1024-row blocks) and O "
                  f"projection; value = attention flops / mean layer-chunk wall time; "
                  f"cores = BLAS threads (NumPy elementwise work is single-threaded)",
    }


if __name__ == "__main__":
    main()
