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
           "qmm_mmq_q8k.hip", "qmm_mmq_q8k2.hip", "qmm_skinny.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# Per-file code generation options.  The small-batch kernel keeps its MFMA
# operands and results in ordinary VGPRs (its epilogue reads every result; the
# accumulator-register form would add one copy per value).
FILE_FLAGS = {"qmm_skinny.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def build(out: str = LIB, extra=()) -> str:
    """Compile every source to an object of its own (in parallel), then link."""
    import concurrent.futures
    import tempfile

    with tempfile.TemporaryDirectory(prefix="qmm_build_") as tmpdir:
        def compile_one(src):
            obj = os.path.join(tmpdir, os.path.splitext(src)[0] + ".o")
            cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), *extra, "-I", INCLUDE, "-I", CSRC, "-c",
                   os.path.join(CSRC, src), "-o", obj]
            subprocess.run(cmd, check=True)
            return obj

        with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        tmp = out + ".tmp"
        subprocess.run([HIPCC, *FLAGS, *extra, *objs, "-o", tmp], check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
