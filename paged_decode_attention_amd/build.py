"""Build libkvq.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc.

    python -m paged_decode_attention_amd.build        # or __graft_entry__.build()

Every translation unit is compiled to an object file in parallel under ``_build/`` and the
objects are linked into ``paged_decode_attention_amd/libkvq.so``. Flags:
  --offload-arch=gfx950                       MI355X only
  -fhip-fp32-correctly-rounded-divide-sqrt    IEEE float division (the quantizer's codes must
                                              match a correctly rounded reference bit for bit)
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                              no packed-FP32 VALU instructions
  -mllvm -amdgpu-mfma-vgpr-form               MFMA accumulators in VGPRs, so the VALU work on
                                              them (Horner shifts, rescaling) needs no copies
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvq.so")
# the streaming probes that measure the HBM ceiling (measurement support, include/kvq_stream.h)
STREAM_LIB = os.path.join(PKG, "libkvq_stream.so")
STREAM_SOURCES = ["kvq_stream.hip"]
SOURCES = ["kvq_api.hip", "kvq_append.hip", "kvq_decode.hip", "kvq_decode_mfma.hip", "kvq_chunk_attn.hip", "kvq_dequant.hip",
           "kvq_baseline_bf16.hip", "kvq_pc.hip", "kvq_pc_write.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CFLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


# Per-source extras. The write path never sees a NaN it must order (its min / max run on finite
# rotated values), and neither does the large-chunk attention (its maxima run on scores that are
# finite or -inf: rows past a sequence and tokens on invalid pages get zero scale and zero), so
# NaN-honouring min / max lowering - a canonicalising move that keeps the DPP row reductions from
# fusing into single instructions - is switched off there.
EXTRA_CFLAGS = {"kvq_append.hip": ["-fno-honor-nans"], "kvq_pc_write.hip": ["-fno-honor-nans"],
                "kvq_chunk_attn.hip": ["-fno-honor-nans"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *EXTRA_CFLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}", file=sys.stderr)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + STREAM_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB, verbose)
    _link(objs[len(SOURCES):], STREAM_LIB, verbose)
    return LIB


if __name__ == "__main__":
    build()
