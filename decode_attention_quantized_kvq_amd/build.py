"""Build libkvq.so (the C-ABI library with the gfx950 HIP kernels) in-tree.

    python -m decode_attention_quantized_kvq_amd.build

hipcc cross-compiles for gfx950 without a GPU.  The build runs in two passes
so that the device-only switches reach the device compiler alone:

1. device pass (``--cuda-device-only``): the gfx950 code object, with
   packed-FP32 instructions turned off (``-target-feature -packed-fp32-ops``);
2. host pass (``--cuda-host-only``): the host code, embedding that code
   object (``-fcuda-include-gpubinary``) and registering its kernels;

then the host object is linked into the shared library.  fp32 division stays
correctly rounded (the HIP default), which the quantizer's codes depend on.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
SRC = PKG / "csrc" / "kvq.hip"
LIB = PKG / "libkvq.so"
ARCH = os.environ.get("KVQ_OFFLOAD_ARCH", "gfx950")

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wno-unused-command-line-argument",
    f"-I{ROOT / 'include'}",
]
DEVICE_FLAGS = ["--cuda-device-only", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> Path:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB.with_name(LIB.name + ".tmp")
    with tempfile.TemporaryDirectory(prefix="kvq_build_") as d:
        fatbin = Path(d) / "kvq.hipfb"
        obj = Path(d) / "kvq.o"
        steps = [
            [hipcc, *COMMON_FLAGS, *DEVICE_FLAGS, "-c", str(SRC), "-o", str(fatbin)],
            [hipcc, *COMMON_FLAGS, "--cuda-host-only", "-Xclang", "-fcuda-include-gpubinary", "-Xclang", str(fatbin),
             "-c", str(SRC), "-o", str(obj)],
            [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", str(obj), "-o", str(tmp)],
        ]
        for cmd in steps:
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
