"""Builds libdsa.so (HIP kernels for gfx950 + the C ABI) and libdsa_peak.so (the
rate probes the benchmark measures peaks with) in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdsa.so")
PEAK_LIB = os.path.join(PKG, "libdsa_peak.so")

SOURCES = ["dsa_api.cpp", "indexer_prefill.hip", "topk_select.hip", "sparse_attn.hip", "quant.hip", "paged.hip", "overlap.hip"]

# -packed-fp32-ops: never emit v_pk_{add,mul,fma}_f32 (only the device pass
# knows the feature; the host pass warns and ignores it).
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libdsa)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    # --no-undefined: a kernel whose host stub was not emitted fails here, not at load
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,--no-undefined", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compiles every source, links libdsa.so and libdsa_peak.so; returns the
    path of libdsa.so."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES) + 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES + ["peak.hip"]))
    _link(objs[:-1], LIB)
    _link(objs[-1:], PEAK_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
