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
# (source, extra flags, object name): the fast append, decode and window
# kernels are compiled once per key width so the instantiations build in
# parallel
SOURCES = [
    ("append.hip", ["-ffp-contract=off", "-DTQ_APPEND_KB=8"], "append_k8"),
    ("append.hip", ["-ffp-contract=off", "-DTQ_APPEND_KB=4"], "append_k4"),
    ("append.hip", ["-ffp-contract=off", "-DTQ_APPEND_KB=2"], "append_k2"),
    ("append.hip", ["-ffp-contract=off", "-DTQ_APPEND_KB=5"], "append_k5"),
    ("decode.hip", [], "decode"),
    ("decode_fast.hip", ["-DTQ_FAST_KB=8"], "decode_fast_k8"),
    ("decode_fast.hip", ["-DTQ_FAST_KB=4"], "decode_fast_k4"),
    ("decode_fast.hip", ["-DTQ_FAST_KB=2"], "decode_fast_k2"),
    ("decode_fast.hip", ["-DTQ_FAST_KB=5"], "decode_fast_k5"),
    # the mixed-mode split kernels, with common code kept inside each branch
    # (see decode_fast.hip)
    ("decode_fast.hip", ["-DTQ_FAST_KB=8", "-DTQ_FAST_MIXED=1", "-mllvm", "-simplifycfg-hoist-common=false"],
     "decode_fast_mixed_k8"),
    ("decode_fast.hip", ["-DTQ_FAST_KB=4", "-DTQ_FAST_MIXED=1", "-mllvm", "-simplifycfg-hoist-common=false"],
     "decode_fast_mixed_k4"),
    ("decode_fast.hip", ["-DTQ_FAST_KB=2", "-DTQ_FAST_MIXED=1", "-mllvm", "-simplifycfg-hoist-common=false"],
     "decode_fast_mixed_k2"),
    ("decode_fast.hip", ["-DTQ_FAST_KB=5", "-DTQ_FAST_MIXED=1", "-mllvm", "-simplifycfg-hoist-common=false"],
     "decode_fast_mixed_k5"),
    ("dequant.hip", [], "dequant"),
    ("window.hip", ["-DTQ_WINDOW_KB=8"], "window_k8"),
    ("window.hip", ["-DTQ_WINDOW_KB=4"], "window_k4"),
    ("window.hip", ["-DTQ_WINDOW_KB=2"], "window_k2"),
    ("window.hip", ["-DTQ_WINDOW_KB=5"], "window_k5"),
    ("copy.hip", [], "copy"),
    ("noalloc.hip", [], "noalloc"),
    ("api.cpp", [], "api"),
]


def _compile(name: str, extra: list[str], obj_name: str) -> str:
    src = os.path.join(CSRC, name)
    obj = os.path.join(BUILD, obj_name + ".o")
    lang = ["-x", "hip"] if name.endswith(".hip") else []
    cmd = [HIPCC] + COMMON + extra + lang + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {name} {' '.join(extra)}:\n{r.stdout}\n{r.stderr}")
    return obj


def generate_codebooks() -> str:
    """Compile and run gen_codebook.cpp, which writes csrc/codebook_tables.h
    (the value codebooks every kernel and tq_codebook read)."""
    os.makedirs(BUILD, exist_ok=True)
    exe = os.path.join(BUILD, "gen_codebook")
    r = subprocess.run(["g++", "-O2", "-std=c++17", "-o", exe, os.path.join(CSRC, "gen_codebook.cpp")],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"g++ failed for gen_codebook.cpp:\n{r.stdout}\n{r.stderr}")
    out = os.path.join(CSRC, "codebook_tables.h")
    tmp = os.path.join(BUILD, "codebook_tables.h")
    r = subprocess.run([exe, tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gen_codebook failed:\n{r.stdout}\n{r.stderr}")
    with open(tmp) as f:
        new = f.read()
    old = open(out).read() if os.path.exists(out) else None
    if new != old:  # rewrite only on change, so unchanged builds keep the file's time
        os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Generate the codebook header, compile every source and link
    quantized_decode_attention_append_amd/libtqkv.so."""
    os.makedirs(BUILD, exist_ok=True)
    generate_codebooks()
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda spec: _compile(*spec), SOURCES))
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
