"""Build liblla.so (the C-ABI LLA library) for gfx950 with hipcc.

Run as ``python -m local_linear_attention_flashlla_amd.build`` or call
``build()``. The library is written next to this file, in-tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB_NAME = "liblla.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = os.environ.get("LLA_OFFLOAD_ARCH", "gfx950")

SOURCES = ["lla_api.hip", "lla_valu.hip", "lla_mfma.hip", "lla_decode.hip", "lla_bwd.hip"]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    f"--offload-arch={ARCH}",
    # keep the compiler from emitting packed fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in the architectural VGPR file: the CG state
    # that the vector ALU reads between key sweeps then never has to be copied
    # between the accumulation and architectural register files in the loop
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build liblla.so)")


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    fd, tmp = tempfile.mkstemp(prefix="liblla.", suffix=".so.tmp", dir=HERE)
    os.close(fd)
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    try:
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB_PATH)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
