"""Build libqattn.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m bit_quantized_attention_amd.build

Each source is compiled with hipcc to an object under ``_build/`` (in
parallel), then linked into ``bit_quantized_attention_amd/libqattn.so``. The
benchmark's peak-rate micro-benchmarks (``csrc/peaks.hip``) go into a library
of their own, ``libqattn_peaks.so``, which the attention path never loads.
"""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqattn.so")
PEAKS_LIB = os.path.join(PKG, "libqattn_peaks.so")
SOURCES = ["smooth_quant.hip", "block_mask.hip", "attn_fwd.hip", "head_error.hip", "lowbit_mask.hip",
           "stripes.hip", "patterns.hip",
           "api.cpp"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


# per-source flags: the 4-bit score kernel keeps its matrix results in ordinary
# VGPRs (the compiler's default puts them in AGPRs, and every estimate then
# costs a v_accvgpr_read before its max)
FILE_FLAGS = {"lowbit_mask.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, extra=()) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *FILE_FLAGS.get(src, []), *extra, "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True, extra=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES + ["peaks.hip"]))
    _link(objs[:-1], LIB)
    _link(objs[-1:], PEAKS_LIB)
    if verbose:
        print(f"built {LIB} and {PEAKS_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
