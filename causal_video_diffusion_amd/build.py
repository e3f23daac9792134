"""Build libust.so (the C-ABI library and its gfx950 kernels) in-tree.

    python -m causal_video_diffusion_amd.build [-v]

Every source is compiled by hipcc for gfx950 (device code) and x86-64 (host
code), then linked into causal_video_diffusion_amd/libust.so.  Packed fp32
vector ops are disabled on the device side.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
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
           "gemm.hip", "calib.hip", "conv3d.hip"]
# sources whose inline-asm global->LDS loads take a scalar base address
DMA_SOURCES = ["window_attn.hip", "gemm.hip", "conv3d.hip"]

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


def _sgpr_set(tok: str) -> set:
    m = re.fullmatch(r"s(\d+)", tok)
    if m:
        return {int(m.group(1))}
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    return set()


def check_dma_base_hazards(asm: str) -> list:
    """Scan gfx950 assembly for inline-asm `global_load_lds_dwordx4 vN, s[a:b]`
    whose scalar base was written by a vector instruction fewer than 5 wait
    states earlier.  The hardware does not interlock a VALU write of an SGPR
    with a vector-memory read of it (the CDNA3/CDNA4 ISA guides list 5 wait
    states), and the compiler inserts none before inline asm, so such a load
    can use a stale address.  The look-back follows every path into a block
    (branches to its label and the fall-through) and every instruction
    counts one wait state (s_nop N counts N + 1).  Returns one message per
    offending load and path."""
    lines = [l.strip() for l in asm.split("\n")]
    label_at = {}
    preds = {}
    for i, t in enumerate(lines):
        m = re.match(r"(\.LBB\d+_\d+):", t)
        if m:
            label_at[m.group(1)] = i
        m = re.match(r"s_c?branch\w* (\.LBB\d+_\d+)", t)
        if m:
            preds.setdefault(m.group(1), []).append(i)

    def is_insn(t: str) -> bool:
        return bool(t) and not t.startswith(";") and not t.startswith(".") and not t.endswith(":")

    found = []

    def walk(j: int, ws: int, base: set, load_line: int, seen: set) -> None:
        while j >= 0 and ws < 5:
            t = lines[j]
            m = re.match(r"(\.LBB\d+_\d+):", t)
            if m:
                # every path into the block: branches to it and the fall-through
                for src in preds.get(m.group(1), []):
                    if (src, ws) not in seen:
                        seen.add((src, ws))
                        walk(src, ws, base, load_line, seen)
                k = j - 1
                while k >= 0 and not is_insn(lines[k]) and not re.match(r"\.LBB\d+_\d+:", lines[k]) \
                        and not re.match(r"[A-Za-z_][\w.$]*:", lines[k]):
                    k -= 1
                if k >= 0 and is_insn(lines[k]) and lines[k].split()[0] in ("s_branch", "s_endpgm", "s_setpc_b64"):
                    return
                j -= 1
                continue
            if re.match(r"[A-Za-z_][\w.$]*:", t):
                return   # function entry: nothing precedes
            j -= 1
            if not is_insn(t):
                continue
            op = t.split()[0]
            if op == "s_nop":
                ws += int(t.split()[1], 0) + 1
                continue
            if op.startswith("v_") and len(t.split()) > 1 and _sgpr_set(t.split()[1].rstrip(",")) & base:
                found.append(f"line {load_line + 1}: base written by '{t}' (line {j + 2}) "
                             f"{ws} wait states before")
                return
            ws += 1

    for i, t in enumerate(lines):
        m = re.match(r"global_load_lds_dwordx4 v\d+, (s\[\d+:\d+\])", t)
        if m:
            walk(i - 1, 0, _sgpr_set(m.group(1)), i, set())
    return found


def _check_dma_source(src: str, verbose: bool) -> None:
    path = os.path.join(CSRC, src)
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".s")
    cmd = [hipcc()] + COMMON + DEVICE + ["--cuda-device-only", "-S", path, "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"assembling {src} failed:\n{r.stderr}")
    bad = check_dma_base_hazards(open(out).read())
    if bad:
        raise RuntimeError(f"{src}: scalar base of a global->LDS load written by a vector "
                           f"instruction without the 5 wait states:\n" + "\n".join(bad[:20]))


def build(verbose: bool = False) -> str:
    """Compile and link libust.so; returns its path.  The device assembly of
    the sources with global->LDS loads is checked for a vector-written
    scalar base (check_dma_base_hazards)."""
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + len(DMA_SOURCES))) as ex:
        checks = [ex.submit(_check_dma_source, s, verbose) for s in DMA_SOURCES]
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
        for c in checks:
            c.result()
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
