"""Build libconvrot_amd.so (HIP, gfx950 only) in-tree with hipcc."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libconvrot_amd.so")
SOURCES = ["rotq.hip", "route.hip", "gemm.hip", "combine.hip", "g16.hip", "peaks.hip", "convrot_api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # every fp32 expression is evaluated as written: no fused multiply-add, no packed fp32 math
    "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wextra", "-Werror", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"),
    "-I" + BUILD,
]
CC = os.environ.get("CC", "gcc")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def silu_table(kind: str = "inc") -> str:
    """Build and run the host generator of the SwiGLU gate activation table (every bf16 input); returns the
    path of its output (`inc`: C initializer included by gemm.hip, `bin`: 65536 little-endian floats)."""
    os.makedirs(BUILD, exist_ok=True)
    exe = os.path.join(BUILD, "silu_table_gen")
    src = os.path.join(CSRC, "silu_table_gen.c")
    r = subprocess.run([CC, "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", src, "-o", exe, "-lm"],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"silu table generator failed to build:\n{r.stdout}\n{r.stderr}")
    out = os.path.join(BUILD, "silu_table." + kind)
    with open(out + ".tmp", "wb") as fh:
        r = subprocess.run([exe, kind], stdout=fh, stderr=subprocess.PIPE)
    if r.returncode != 0:
        raise RuntimeError(f"silu table generator failed:\n{r.stderr.decode()}")
    os.replace(out + ".tmp", out)
    return out


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    silu_table("inc")
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
