"""Build libkvq.so (the C-ABI library with the gfx950 HIP kernels) in-tree.

    python -m decode_attention_quantized_kvq_amd.build

hipcc cross-compiles for gfx950 without a GPU.  Packed-FP32 instructions are
turned off (`-packed-fp32-ops`); fp32 division stays correctly rounded (the
HIP default), which the quantizer's codes depend on.
"""
from __future__ import annotations

import os
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
SRC = PKG / "csrc" / "kvq.hip"
LIB = PKG / "libkvq.so"
ARCH = os.environ.get("KVQ_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{ROOT / 'include'}",
]


def build(verbose: bool = False) -> Path:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB.with_name(LIB.name + ".tmp")
    cmd = [hipcc, *HIPCC_FLAGS, str(SRC), "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
