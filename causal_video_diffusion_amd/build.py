"""Build libust.so (the C-ABI library and its gfx950 kernels) in-tree.

    python -m causal_video_diffusion_amd.build [-v]

Every source is compiled by hipcc for gfx950 (device code) and x86-64 (host
code), then linked into causal_video_diffusion_amd/libust.so.  Packed fp32
vector ops are disabled on the device side.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libust.so")
OBJ = os.path.join(PKG, "_build")
ARCH = "gfx950"

SOURCES = ["ust_host.cpp", "rope_table.hip", "kv_append.hip", "window_attn.hip", "sampler.hip",
           "gemm.hip"]

COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
          "-I", os.path.join(ROOT, "include")]
DEVICE = ["-x", "hip", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fgpu-flush-denormals-to-zero", "-munsafe-fp-atomics"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, verbose: bool) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + COMMON
    if src.endswith(".hip"):
        cmd += DEVICE
    cmd += ["-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{err}")
    if verbose and err.strip():
        print(err, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    """Compile and link libust.so; returns its path."""
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libust.so failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    _build_c_check(verbose)
    return OUT


C_CHECK = os.path.join(OBJ, "c_abi_check")


def _build_c_check(verbose: bool) -> None:
    """tests/c_abi_check.c: a C11 program that uses libust.so through its C
    ABI alone (run on the GPU by the parity tests).  Built here, on the build
    host, so that no test compiles anything."""
    src = os.path.join(ROOT, "tests", "c_abi_check.c")
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cmd = [shutil.which("gcc") or "gcc", "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), src, "-o", C_CHECK, "-L", PKG, "-lust",
           "-Wl,-rpath,$ORIGIN/..", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath," + os.path.join(rocm, "lib"), "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling c_abi_check failed:\n{r.stderr}")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
