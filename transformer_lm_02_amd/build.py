"""Build libgpt_hip.so in-tree with hipcc for gfx950.

    python -m transformer_lm_02_amd.build        # or build() from Python

Every source under csrc/ is compiled to objects in _build/ (in parallel), then
linked into transformer_lm_02_amd/libgpt_hip.so.  Always recompiles.  The
kernels and the host orchestration are compiled twice, once per 16-bit
activation format (bfloat16, and IEEE binary16 with GPT_HALF_FP16 defined);
api.cpp, the C ABI that picks between the two, once.
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
LIB = os.path.join(PKG, "libgpt_hip.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    # packed fp32 instructions off for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


ONCE = ("api.cpp",)


def _compile(job) -> str:
    src, fp16 = job
    obj = os.path.join(BUILD, os.path.basename(src) + (".f16.o" if fp16 else ".o"))
    cmd = [HIPCC, *FLAGS]
    if fp16:
        cmd += ["-DGPT_HALF_FP16"]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-6000:]}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))
    jobs = [(f, False) for f in srcs] + [(f, True) for f in srcs
                                          if os.path.basename(f) not in ONCE]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(_compile, jobs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-6000:]}")
    shutil.move(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources", flush=True)
    return LIB


if __name__ == "__main__":
    try:
        build()
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
