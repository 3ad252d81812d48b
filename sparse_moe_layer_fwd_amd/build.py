"""Build libmoe.so (all HIP sources, gfx950) in-tree with hipcc.

    python -m sparse_moe_layer_fwd_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libmoe.so")
SOURCES = ["moe_api.hip", "route.hip", "gemm_f32.hip", "gemm_bf16.hip", "gemm_skinny.hip", "quant.hip"]
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")

# Packed fp32 ALU ops stay off: the compiler must not form v_pk_* fp32 math.
HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe.so)")


def build(verbose: bool = False) -> str:
    """Compile every HIP source into sparse_moe_layer_fwd_amd/lib/libmoe.so."""
    os.makedirs(LIB_DIR, exist_ok=True)
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    fd, tmp = tempfile.mkstemp(prefix="libmoe.", suffix=".so.tmp", dir=LIB_DIR)
    os.close(fd)
    cmd = [hipcc()] + HIPCC_FLAGS + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        os.unlink(tmp)
        raise RuntimeError("hipcc failed (%d):\n%s\n%s" % (res.returncode, res.stdout, res.stderr))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
