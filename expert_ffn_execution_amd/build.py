"""Build libftmoe.so (HIP, gfx950) in-tree with hipcc.

    python -m expert_ffn_execution_amd.build          # compile + link

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled (the compiler keeps to scalar fp32 VALU forms).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libftmoe.so")
# stand-alone matrix-core issue-rate probe (not part of the library)
PROBE_SRC = "mfma_rate.hip"
PROBE = os.path.join(PKG, "mfma_rate")
SOURCES = ["api.cpp", "slot_cache.cpp", "route.hip", "align.hip", "gemm_mfma.hip", "router_mfma.hip",
           "ffn_stream.hip", "combine.hip", "step.cpp", "host_ffn.cpp", "noalloc.hip", "fused_decode.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Wno-unused-result", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          f"-I{os.path.join(ROOT, 'include')}"]


# host-only C++ (no device code): the host compiler
HOST_SOURCES = {"host_ffn.cpp"}
HOST_CFLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-pthread", f"-I{os.path.join(ROOT, 'include')}"]


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    if src in HOST_SOURCES:
        cmd = ["g++", *HOST_CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"g++ failed for {src}:\n{r.stderr}")
        return obj
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *CFLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    if r.stderr.strip():
        warn = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
        if warn:
            sys.stderr.write("\n".join(warn) + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "-pthread", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    build_probe()
    if verbose:
        print(f"built {LIB} and {PROBE}")
    return LIB


def build_probe() -> str:
    cmd = [HIPCC, *[f for f in CFLAGS if f != "-fPIC"], "-x", "hip", os.path.join(CSRC, PROBE_SRC),
           "-o", PROBE + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {PROBE_SRC}:\n{r.stderr}")
    os.replace(PROBE + ".tmp", PROBE)
    return PROBE


if __name__ == "__main__":
    build()
