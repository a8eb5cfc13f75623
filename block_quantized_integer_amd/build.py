"""Build libbqi.so (all HIP kernels + the C ABI) for gfx950, in-tree.

    python -m block_quantized_integer_amd.build

Compiles with hipcc for --offload-arch=gfx950 only.  Flags that matter for
exactness: no fast-math, fp32 denormals kept (HIP's default), correctly rounded
fp32 division (HIP's default), no FP contraction (every fma is written out),
and packed-fp32 VALU instructions disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libbqi.so")
SOURCES = ["api.hip", "quantize.hip", "gemv_thin.hip", "gemm_mfma.hip", "grouped_w4a8.hip",
           "moe_combine.hip", "gguf_import.hip", "host_w4a8.cpp"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + ["-I", os.path.join(PKG, "..", "include")] + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature and says so; drop that line
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if out.strip() and verbose:
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
