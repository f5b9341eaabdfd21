"""Build libqmm.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqmm.so")
SOURCES = ["qmm_api.hip", "qmm_quantize.hip", "qmm_fused.hip", "qmm_mmvq.hip", "qmm_mmq.hip", "qmm_mmq2.hip",
           "qmm_mmq_q8k.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def build(out: str = LIB, extra=()) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, *srcs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
