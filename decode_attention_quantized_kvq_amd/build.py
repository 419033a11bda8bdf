"""Build libkvq.so (the C-ABI library with the gfx950 HIP kernels) in-tree.

    python -m decode_attention_quantized_kvq_amd.build

hipcc cross-compiles for gfx950 without a GPU.  The library is kvq.hip (the C
ABI, dispatch and the smaller kernels) plus kvq_inst.hip compiled once per
family of the split kernel's instances (key width, value width, paged
storage, zero point); the units compile in parallel.  Each unit builds in
two passes so that the device-only switches reach the device compiler alone:

1. device pass (``--cuda-device-only``): the gfx950 code object, with
   packed-FP32 instructions turned off (``-target-feature -packed-fp32-ops``);
2. host pass (``--cuda-host-only``): the host code, embedding that code
   object (``-fcuda-include-gpubinary``) and registering its kernels;

then the host objects are linked into the shared library.  fp32 division
stays correctly rounded (the HIP default), which the quantizer's codes
depend on.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
MAIN = CSRC / "kvq.hip"
INST = CSRC / "kvq_inst.hip"
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

# (key bits, value bits, paged, zero point): the families kvq.hip declares
FAMILIES = [(kb, vb, pg, zp) for pg, zp in (("false", "false"), ("true", "false"), ("false", "true"), ("true", "true"))
            for kb, vb in ((8, 8), (8, 4), (4, 4), (4, 8))]


def _units():
    yield "kvq", MAIN, []
    for kb, vb, pg, zp in FAMILIES:
        name = f"kvq_inst_k{kb}v{vb}{'_paged' if pg == 'true' else ''}{'_zp' if zp == 'true' else ''}"
        yield name, INST, [f"-DKVQ_KB={kb}", f"-DKVQ_VB={vb}", f"-DKVQ_PG={pg}", f"-DKVQ_ZP={zp}"]


def build(verbose: bool = False) -> Path:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    jobs = max(1, min(int(os.environ.get("MAX_JOBS", os.cpu_count() or 1)), os.cpu_count() or 1, 16))
    tmp = LIB.with_name(LIB.name + ".tmp")
    with tempfile.TemporaryDirectory(prefix="kvq_build_") as d:
        def unit(args):
            name, src, defs = args
            fatbin = Path(d) / f"{name}.hipfb"
            obj = Path(d) / f"{name}.o"
            steps = [
                [hipcc, *COMMON_FLAGS, *defs, *DEVICE_FLAGS, "-c", str(src), "-o", str(fatbin)],
                [hipcc, *COMMON_FLAGS, *defs, "--cuda-host-only", "-Xclang", "-fcuda-include-gpubinary", "-Xclang",
                 str(fatbin), "-c", str(src), "-o", str(obj)],
            ]
            for cmd in steps:
                if verbose:
                    print(" ".join(cmd), flush=True)
                subprocess.run(cmd, check=True)
            return obj

        with ThreadPoolExecutor(jobs) as pool:
            objs = list(pool.map(unit, list(_units())))
        cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
