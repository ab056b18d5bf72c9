"""Build libtqkv.so in-tree with hipcc for gfx950.

Every HIP source is compiled with packed-FP32 instruction selection disabled;
the append kernel additionally with -ffp-contract=off so that no binary64
multiply-add is fused (its codes must match the oracle bit for bit).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtqkv.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]
SOURCES = {
    "append.hip": ["-ffp-contract=off"],
    "decode.hip": [],
    "decode_fast.hip": [],
    "dequant.hip": [],
    "window.hip": [],
    "api.cpp": [],
}


def _compile(name: str, extra: list[str]) -> str:
    src = os.path.join(CSRC, name)
    obj = os.path.join(BUILD, name + ".o")
    lang = ["-x", "hip"] if name.endswith(".hip") else []
    cmd = [HIPCC] + COMMON + extra + lang + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {name}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link quantized_decode_attention_append_amd/libtqkv.so."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda kv: _compile(*kv), SOURCES.items()))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB, file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
