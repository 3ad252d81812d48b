"""Build libmoe.so (all HIP sources, gfx950) in-tree with hipcc.

    python -m sparse_moe_layer_fwd_amd.build [-v] [--asan-host]

Each source is compiled to an object under lib/obj/ in its own hipcc process
(in parallel), then the objects are linked into the shared library.  Warnings
are errors.

--asan-host builds a second library, lib/libmoe_asan.so: the host dispatcher
(moe_api.hip: argument validation, workspace planning, status and stage-timer
code) compiled with AddressSanitizer on its host code only (device code as
usual), linked with the other objects.  It is a CPU-side checking build: the
ABI tests load it into a process started with the sanitizer runtime preloaded.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_DIR = os.path.join(PKG, "lib")
OBJ_DIR = os.path.join(LIB_DIR, "obj")
LIB_PATH = os.path.join(LIB_DIR, "libmoe.so")
ASAN_LIB_PATH = os.path.join(LIB_DIR, "libmoe_asan.so")
SOURCES = ["moe_api.hip", "route.hip", "gemm_f32.hip", "gemm_bf16.hip", "gemm_skinny.hip", "quant.hip"]
ASAN_SOURCES = ["moe_api.hip"]
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


def asan_runtime() -> str:
    """The AddressSanitizer runtime of the ROCm clang (to preload into a process)."""
    for cand in sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")):
        return cand
    raise RuntimeError("AddressSanitizer runtime not found under /opt/rocm/llvm")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d): %s\n%s\n%s" % (res.returncode, " ".join(cmd), res.stdout,
                                                              res.stderr))
    return res


def _compile(sources, suffix, extra, verbose):
    """Compile `sources` to OBJ_DIR/<name><suffix>.o in parallel; returns the paths."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    cc = hipcc()
    objs = [os.path.join(OBJ_DIR, os.path.splitext(s)[0] + suffix + ".o") for s in sources]
    cmds = [[cc] + HIPCC_FLAGS + extra + ["-c", os.path.join(CSRC, s), "-o", o + ".tmp"]
            for s, o in zip(sources, objs)]
    with ThreadPoolExecutor(max_workers=min(len(cmds), max(1, os.cpu_count() or 1))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    for o in objs:
        os.replace(o + ".tmp", o)
    return objs


def _link(objs, out_path, verbose):
    tmp = out_path + ".tmp"
    _run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
    os.replace(tmp, out_path)
    return out_path


def build(verbose: bool = False) -> str:
    """Compile every HIP source into sparse_moe_layer_fwd_amd/lib/libmoe.so."""
    return _link(_compile(SOURCES, "", [], verbose), LIB_PATH, verbose)


def build_asan_host(verbose: bool = False) -> str:
    """libmoe_asan.so: the host dispatcher with AddressSanitizer (host code only),
    the other sources as in libmoe.so (compiled first if their objects are missing
    or older than their sources)."""
    others = []
    for s in SOURCES:
        if s in ASAN_SOURCES:
            continue
        o = os.path.join(OBJ_DIR, os.path.splitext(s)[0] + ".o")
        deps = [os.path.join(CSRC, s), os.path.join(CSRC, "common.h")]
        if not os.path.exists(o) or any(os.path.getmtime(o) < os.path.getmtime(d) for d in deps):
            o = _compile([s], "", [], verbose)[0]
        others.append(o)
    san = _compile(ASAN_SOURCES, ".asan", ASAN_HOST_FLAGS, verbose)
    return _link(san + others, ASAN_LIB_PATH, verbose)


if __name__ == "__main__":
    v = "-v" in sys.argv
    print(build_asan_host(v) if "--asan-host" in sys.argv else build(v))
