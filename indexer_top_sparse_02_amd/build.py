"""Builds libsia.so, the gfx950 HIP library behind include/sia.h, in-tree.

    python -m indexer_top_sparse_02_amd.build

Every .hip file under csrc/ is compiled to an object with hipcc for gfx950,
then linked into indexer_top_sparse_02_amd/libsia.so. The streaming-read
calibration kernel under csrc/probe/ becomes libsia_probe.so, which only the
benchmark loads.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsia.so")
PROBE_SRC = os.path.join(CSRC, "probe", "read_probe.hip")
PROBE_LIB = os.path.join(PKG, "libsia_probe.so")
ARCH = os.environ.get("SIA_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-file code generation options: MFMA results in vector registers. The
# compiler's default for a kernel that needs more than 256 registers, or that
# uses accumulation registers itself (the whole-tile attention kernel holds its
# query operand there), is to put MFMA results in accumulation registers and
# copy them back and forth around the vector arithmetic on them (the causal
# prefill indexer's head sums, the attention softmax).
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
# The score passes place each MFMA group and the vector work meant to run in
# its shadow between scheduling fences. Machine sinking moves MFMAs (which touch
# no memory) past those fences toward the first use of their result, i.e. into
# the next step and across its barrier; the vector work on that result then
# waits for the group it was meant to hide behind.
_NO_SINK = ["-mllvm", "-disable-machine-sink"]
FILE_FLAGS: dict = {"attention.hip": _VGPR_FORM, "indexer.hip": _VGPR_FORM + _NO_SINK}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    extra = FILE_FLAGS.get(os.path.basename(src), [])
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and _NO_SINK[1] in extra and _NO_SINK[1] in r.stderr:
        # a compiler without that option: build with its default code placement
        print(f"{os.path.basename(src)}: compiler rejects {_NO_SINK[1]}; building without it", file=sys.stderr)
        kept = [f for i, f in enumerate(extra) if f != _NO_SINK[1] and not (f == "-mllvm" and i + 1 < len(extra)
                                                                            and extra[i + 1] == _NO_SINK[1])]
        cmd = [HIPCC, *FLAGS, *kept, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    for line in r.stderr.splitlines():
        if line.strip() and noise not in line:
            print(line, file=sys.stderr)
    return obj


def build(jobs: int = 4) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    r = subprocess.run([HIPCC, *FLAGS, "-shared", "-o", PROBE_LIB + ".tmp", PROBE_SRC], capture_output=True,
                       text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {PROBE_SRC}:\n{r.stderr}")
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
