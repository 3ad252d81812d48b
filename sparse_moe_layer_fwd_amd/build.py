"""Build libmoe.so (all HIP sources, gfx950) in-tree with hipcc.

    python -m sparse_moe_layer_fwd_amd.build [-v] [--asan-host]

Each source is compiled to an object in its own hipcc process (in parallel),
then the objects are linked into the shared library.  Warnings are errors.

--asan-host builds a second library, lib/libmoe_asan.so, whose host code is
instrumented with AddressSanitizer (device code is compiled as usual): the
CPU-only ABI checks load it to run the host-side argument validation,
workspace planning and status paths under the sanitizer.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libmoe.so")
ASAN_LIB_PATH = os.path.join(LIB_DIR, "libmoe_asan.so")
SOURCES = ["moe_api.hip", "route.hip", "gemm_f32.hip", "gemm_bf16.hip", "gemm_skinny.hip", "quant.hip"]
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")

# Packed fp32 ALU ops stay off: the compiler must not form v_pk_* fp32 math.
HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Werror", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"),
]
# host code only (the flag after each -Xarch_host applies to the host pass)
ASAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
                   "-Xarch_host", "-g"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d): %s\n%s\n%s" % (res.returncode, " ".join(cmd), res.stdout,
                                                              res.stderr))
    # the host pass does not know the device-only target feature: harmless
    return res


def _build(out_path: str, extra: list, verbose: bool) -> str:
    os.makedirs(LIB_DIR, exist_ok=True)
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="libmoe.", dir=LIB_DIR) as tmpdir:
        objs = [os.path.join(tmpdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [[cc] + HIPCC_FLAGS + extra + ["-c", os.path.join(CSRC, s), "-o", o]
                for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(max_workers=min(len(cmds), max(1, os.cpu_count() or 1))) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        tmp = os.path.join(tmpdir, "lib.so")
        _run([cc, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + extra + objs + ["-o", tmp], verbose)
        os.replace(tmp, out_path)
    return out_path


def build(verbose: bool = False) -> str:
    """Compile every HIP source into sparse_moe_layer_fwd_amd/lib/libmoe.so."""
    return _build(LIB_PATH, [], verbose)


def build_asan_host(verbose: bool = False) -> str:
    """The same library with AddressSanitizer on the host code only."""
    return _build(ASAN_LIB_PATH, ASAN_HOST_FLAGS, verbose)


if __name__ == "__main__":
    v = "-v" in sys.argv
    print(build_asan_host(v) if "--asan-host" in sys.argv else build(v))
