"""Builds the HIP library libblasst.so in-tree for gfx950 (hipcc cross-compiles without a GPU), and
beside it libblasst_ceiling.so, the benchmark's read-only streaming ceilings (measurement only)."""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libblasst.so")
CEILING_SRC = os.path.join(HERE, "ceiling", "stream_read.hip")
CEILING_OUT = os.path.join(HERE, "libblasst_ceiling.so")
BUILD_DIR = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


# Per-file code-generation options.  decode_mla.hip keeps its score MFMAs in VGPRs (their results
# feed VALU code) while its output accumulators live in AGPRs through explicit operands;
# prefill_bwd.hip uses the VGPR form throughout (measured 5-10 % faster than the compiler's
# default choice for its dK/dV kernel, whose accumulators otherwise shuttle between register files).
EXTRA = {"decode_mla.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"],
         "prefill_bwd.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON, *EXTRA.get(os.path.basename(src), []), *lang, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    tmp = CEILING_OUT + ".tmp"
    cmd = [HIPCC, *COMMON, "-shared", "-x", "hip", CEILING_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {CEILING_SRC}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, CEILING_OUT)
    if verbose:
        print(f"built {CEILING_OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
