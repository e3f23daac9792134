"""ctypes binding of libust.so: same names as the C ABI, argument marshalling only.

Tensors are torch tensors on the GPU; the binding passes their data pointers
and torch's current HIP stream.  The C argument that names a RoPE table's
first frame (first_frame of ust_rope_table_build, tab_first_frame of its
consumers) is a keyword argument here, last, defaulting to 0: a table from
frame 0.  Every step of the path runs in the library's
kernels.  If libust.so has not been built, loading raises: there is no CPU
fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libust.so")

UST_MAX_WINDOW_FRAMES = 128
STATUS = {0: "UST_OK", 1: "UST_E_NULL", 2: "UST_E_SHAPE", 3: "UST_E_RANGE",
          4: "UST_E_ALIGN", 5: "UST_E_UNSUPPORTED", 6: "UST_E_HIP"}

# every entry point the header declares
EXPORTS = ("ust_v_row_len", "ust_rope_table_build", "ust_kv_append",
           "ust_window_attn", "ust_window_attn_work_bytes", "ust_window_attn_split",
           "ust_qkv_append", "ust_lowrank_proj", "ust_flow_step", "ust_slot_of_frame",
           "ust_window_plan", "ust_sigma_schedule", "ust_status_str", "ust_last_error",
           "ust_calib_mfma_bf16", "ust_lowrank_proj_static", "ust_conv3d_causal",
           "ust_conv3d_causal_stream", "ust_lowrank_proj_v_append")


class UstError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{self.name}: {detail}")


class Geom(ctypes.Structure):
    _fields_ = [("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("pairs_t", ctypes.c_int32), ("pairs_h", ctypes.c_int32),
                ("pairs_w", ctypes.c_int32), ("chunk_frames", ctypes.c_int32)]


class Kv(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("n_slots", ctypes.c_int32), ("n_sink", ctypes.c_int32)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libust.so once (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m causal_video_diffusion_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, F32, F64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_double
    SZ = ctypes.c_size_t
    GP, KP = ctypes.POINTER(Geom), ctypes.POINTER(Kv)
    IP = ctypes.POINTER(ctypes.c_int32)
    sig = {
        "ust_v_row_len": (I32, [I32]),
        "ust_rope_table_build": (I32, [GP, I32, I32, F64, P, P, P]),
        "ust_kv_append": (I32, [GP, KP, P, P, P, P, I32, I32, I32, P]),
        "ust_window_attn": (I32, [GP, KP, P, P, P, I32, I32, I32, I32, F32, P, P, P]),
        "ust_window_attn_work_bytes": (SZ, [GP, I32]),
        "ust_window_attn_split": (I32, [GP, KP, P, P, P, I32, I32, I32, I32, F32, P, P, P, SZ,
                                        I32, P]),
        "ust_qkv_append": (I32, [GP, KP, P, P, I32, P, P, I32, I32, I32, P, P]),
        "ust_lowrank_proj": (I32, [P, P, P, P, P, P, I32, I32, I32, I32, P]),
        "ust_lowrank_proj_v_append": (I32, [GP, KP, P, P, P, P, I32, I32, P, P, P, I32, I32, I32,
                                            P]),
        "ust_lowrank_proj_static": (I32, [P, P, P, P, P, I32, I32, I32, I32, P]),
        "ust_conv3d_causal": (I32, [P, P, P, P, I32, I32, I32, I32, I32, P]),
        "ust_conv3d_causal_stream": (I32, [P, P, P, P, I32, I32, I32, I32, I32, P]),
        "ust_flow_step": (I32, [P, P, P, F32, F32, P, P, ctypes.c_int64, P]),
        "ust_sigma_schedule": (I32, [IP, I32, F64, I32, ctypes.POINTER(F64),
                                     ctypes.POINTER(F64)]),
        "ust_slot_of_frame": (I32, [KP, I32]),
        "ust_window_plan": (I32, [GP, KP, I32, I32, IP, IP, I32, IP]),
        "ust_calib_mfma_bf16": (I32, [I32, I32, P, ctypes.POINTER(F64), P]),
        "ust_status_str": (ctypes.c_char_p, [I32]),
        "ust_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        raise UstError(status, load().ust_last_error().decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def geom(grid_h, grid_w, n_heads, head_dim, pairs_t, pairs_h, pairs_w,
         chunk_frames) -> Geom:
    return Geom(grid_h, grid_w, n_heads, head_dim, pairs_t, pairs_h, pairs_w,
                chunk_frames)


def kv(k, v, n_slots: int, n_sink: int) -> Kv:
    """k, v: device tensors (or raw addresses) of the ring."""
    kp = k if isinstance(k, int) or k is None else _ptr(k)
    vp = v if isinstance(v, int) or v is None else _ptr(v)
    return Kv(kp, vp, n_slots, n_sink)


# ------------------------------------------------------------------ entry points

def ust_v_row_len(T: int) -> int:
    return load().ust_v_row_len(T)


def ust_rope_table_build(g: Geom, n_frames: int, theta: float, cos_out, sin_out,
                         stream=None, first_frame: int = 0) -> None:
    _check(load().ust_rope_table_build(ctypes.byref(g), first_frame, n_frames, theta,
                                       _ptr(cos_out), _ptr(sin_out), _stream(stream)))


def ust_kv_append(g: Geom, ring: Kv, k_new, v_new, cos_tab, sin_tab,
                  n_tab_frames: int, frame_start: int, stream=None,
                  tab_first_frame: int = 0) -> None:
    _check(load().ust_kv_append(ctypes.byref(g), ctypes.byref(ring), _ptr(k_new),
                                _ptr(v_new), _ptr(cos_tab), _ptr(sin_tab), tab_first_frame,
                                n_tab_frames, frame_start, _stream(stream)))


def ust_window_attn(g: Geom, ring: Kv, q, cos_tab, sin_tab, n_tab_frames: int,
                    frame_start: int, n_recent: int, scale: float, out,
                    lse=None, stream=None, tab_first_frame: int = 0) -> None:
    _check(load().ust_window_attn(ctypes.byref(g), ctypes.byref(ring), _ptr(q),
                                  _ptr(cos_tab), _ptr(sin_tab), tab_first_frame, n_tab_frames,
                                  frame_start, n_recent, scale, _ptr(out),
                                  _ptr(lse), _stream(stream)))


def ust_window_attn_work_bytes(g: Geom, n_workgroups: int = 0) -> int:
    return load().ust_window_attn_work_bytes(ctypes.byref(g), n_workgroups)


def ust_window_attn_split(g: Geom, ring: Kv, q, cos_tab, sin_tab, n_tab_frames: int,
                          frame_start: int, n_recent: int, scale: float, out,
                          lse=None, work=None, n_workgroups: int = 0,
                          stream=None, tab_first_frame: int = 0) -> None:
    """work: a device tensor of at least ust_window_attn_work_bytes bytes."""
    nbytes = 0 if work is None else work.numel() * work.element_size()
    _check(load().ust_window_attn_split(ctypes.byref(g), ctypes.byref(ring), _ptr(q),
                                        _ptr(cos_tab), _ptr(sin_tab), tab_first_frame,
                                        n_tab_frames,
                                        frame_start, n_recent, scale, _ptr(out),
                                        _ptr(lse), _ptr(work), nbytes, n_workgroups,
                                        _stream(stream)))


def ust_qkv_append(g: Geom, ring: Kv, x, w_qkv, hidden: int, cos_tab, sin_tab,
                   n_tab_frames: int, frame_start: int, q_out, stream=None,
                   tab_first_frame: int = 0) -> None:
    _check(load().ust_qkv_append(ctypes.byref(g), ctypes.byref(ring), _ptr(x), _ptr(w_qkv),
                                 hidden, _ptr(cos_tab), _ptr(sin_tab), tab_first_frame,
                                 n_tab_frames, frame_start, _ptr(q_out), _stream(stream)))


def ust_lowrank_proj_v_append(g: Geom, ring: Kv, x, a, b, t_work, hidden: int, rank: int,
                              frame_start: int, stream=None, k_new=None, cos_tab=None,
                              sin_tab=None, n_tab_frames: int = 0,
                              tab_first_frame: int = 0) -> None:
    """k_new and the table (keyword arguments here) also append the keys."""
    _check(load().ust_lowrank_proj_v_append(ctypes.byref(g), ctypes.byref(ring), _ptr(x), _ptr(a),
                                            _ptr(b), _ptr(t_work), hidden, rank, _ptr(k_new),
                                            _ptr(cos_tab), _ptr(sin_tab), tab_first_frame,
                                            n_tab_frames, frame_start, _stream(stream)))


def ust_lowrank_proj(x, a, b, bias, t_work, y, M: int, K: int, r: int, N: int,
                     stream=None) -> None:
    _check(load().ust_lowrank_proj(_ptr(x), _ptr(a), _ptr(b), _ptr(bias),
                                   _ptr(t_work), _ptr(y), M, K, r, N,
                                   _stream(stream)))


def ust_lowrank_proj_static(x, a, b, bias, y, M: int, K: int, r: int, N: int,
                            stream=None) -> None:
    _check(load().ust_lowrank_proj_static(_ptr(x), _ptr(a), _ptr(b), _ptr(bias), _ptr(y),
                                          M, K, r, N, _stream(stream)))


UST_LOWRANK_STATIC_MAX_ELEMS = 4 * 1024 * 1024


def ust_conv3d_causal(x, w, bias, y, T: int, H: int, W: int, Ci: int, Co: int,
                      stream=None) -> None:
    _check(load().ust_conv3d_causal(_ptr(x), _ptr(w), _ptr(bias), _ptr(y), T, H, W, Ci, Co,
                                    _stream(stream)))


def ust_conv3d_causal_stream(x, w, bias, y, T: int, H: int, W: int, Ci: int, Co: int,
                             stream=None) -> None:
    _check(load().ust_conv3d_causal_stream(_ptr(x), _ptr(w), _ptr(bias), _ptr(y), T, H, W, Ci,
                                           Co, _stream(stream)))


def ust_flow_step(x, v, noise, sigma: float, sigma_next: float, x0_out, x_next, n: int,
                  stream=None) -> None:
    _check(load().ust_flow_step(_ptr(x), _ptr(v), _ptr(noise), sigma, sigma_next,
                                _ptr(x0_out), _ptr(x_next), n, _stream(stream)))


def ust_sigma_schedule(raw_steps, shift: float = 5.0, n_train: int = 1000):
    """(levels, labels) of the raw timesteps, as Python lists."""
    n = len(raw_steps)
    raw = (ctypes.c_int32 * max(n, 1))(*raw_steps)
    sig = (ctypes.c_double * max(n, 1))()
    lab = (ctypes.c_double * max(n, 1))()
    _check(load().ust_sigma_schedule(raw, n, shift, n_train, sig, lab))
    return list(sig[:n]), list(lab[:n])


def ust_slot_of_frame(ring: Kv, frame: int) -> int:
    return load().ust_slot_of_frame(ctypes.byref(ring), frame)


def ust_window_plan(g: Geom, ring: Kv, frame_start: int, n_recent: int,
                    cap: int = UST_MAX_WINDOW_FRAMES) -> Tuple[list, list]:
    frames = (ctypes.c_int32 * max(cap, 1))()
    slots = (ctypes.c_int32 * max(cap, 1))()
    n = ctypes.c_int32(0)
    _check(load().ust_window_plan(ctypes.byref(g), ctypes.byref(ring), frame_start,
                                  n_recent, frames, slots, cap, ctypes.byref(n)))
    return list(frames[:n.value]), list(slots[:n.value])


def ust_calib_mfma_bf16(n_workgroups: int, iters: int, out, stream=None) -> float:
    """Launch the MFMA-only measurement kernel; returns its flop count."""
    flops = ctypes.c_double(0.0)
    _check(load().ust_calib_mfma_bf16(n_workgroups, iters, _ptr(out), ctypes.byref(flops),
                                      _stream(stream)))
    return flops.value
