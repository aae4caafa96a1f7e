"""Build liblla.so (the C-ABI LLA library) for gfx950 with hipcc.

Run as ``python -m local_linear_attention_flashlla_amd.build`` or call
``build()``. The library is written next to this file, in-tree.
"""
from __future__ import annotations

import hashlib
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

SOURCES = ["lla_api.hip", "lla_valu.hip", "lla_mfma.hip", "lla_decode.hip", "lla_bwd.hip",
           "lla_naive.hip"]
# headers the sources include (part of the source hash)
HEADERS = [os.path.join(CSRC, "lla_internal.h"), os.path.join(CSRC, "lla_mfma_common.h"),
           os.path.join(ROOT, "include", "lla.h")]

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


def source_hash() -> str:
    """SHA-256 over the library's sources, headers and compiler flags: the
    value the built library reports through lla_source_hash()."""
    h = hashlib.sha256()
    for path in [os.path.join(CSRC, s) for s in SOURCES] + HEADERS:
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + b"\0" + f.read() + b"\0")
    h.update(" ".join(HIPCC_FLAGS).encode())
    return h.hexdigest()


def build(verbose: bool = False) -> str:
    """Compile every source to an object in parallel, then link liblla.so."""
    from concurrent.futures import ThreadPoolExecutor
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    define = f"-DLLA_SOURCE_SHA256=\"{source_hash()}\""
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    with tempfile.TemporaryDirectory(prefix="lla_build.", dir=HERE) as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(s) + ".o") for s in srcs]
        cmds = [[hipcc(), *compile_flags, define, "-I", os.path.join(ROOT, "include"), "-c", s, "-o", o]
                for s, o in zip(srcs, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        with ThreadPoolExecutor(max_workers=min(len(cmds), max(1, os.cpu_count() or 1))) as ex:
            for r in ex.map(lambda c: subprocess.run(c, capture_output=True, text=True), cmds):
                if r.returncode != 0:
                    sys.stderr.write(r.stderr)
                    raise subprocess.CalledProcessError(r.returncode, r.args)
        tmp = os.path.join(tmpdir, LIB_NAME)
        link = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.run(link, check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
