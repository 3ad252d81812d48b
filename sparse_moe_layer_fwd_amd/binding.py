"""ctypes binding of libmoe.so: the entry points of include/moe.h, same names.

Argument marshalling only; every step of the layer runs in the HIP library.
Importing this module does not load the library; ``lib()`` does, and raises
if it has not been built (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_NO_DEVICE, \
    MOE_ERR_HIP = range(6)
MOE_F32, MOE_BF16, MOE_NVFP4, MOE_FP8 = 0, 1, 2, 3
DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "nvfp4": MOE_NVFP4, "fp8": MOE_FP8}

EXPORTED = ("moe_init", "moe_workspace_size", "moe_route", "moe_forward", "moe_forward_noalloc",
            "moe_quantize_fp8", "moe_nvfp4_tile",
            "moe_destroy", "moe_status_string", "moe_profile_enable", "moe_profile_read",
            "moe_stage_name")
MOE_NUM_STAGES = 13


class MoEConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "d", "latent", "n_experts", "top_k", "ffn", "n_shared", "shared_ffn", "max_tokens",
        "has_latent_proj", "act_dtype", "expert_dtype", "router_on_x", "shared_fp8")]


class MoEWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w_down", "w_router", "b_router", "w1", "w2", "w1_scale", "w2_scale", "w1_gscale",
        "w2_gscale", "w_up", "ws1", "ws2", "act_scale", "ws1_scale", "ws2_scale",
        "shared_act_scale")]


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s" % (where, status_string(status)))


_LIB = None


def lib(path: str = None) -> ctypes.CDLL:
    """Load libmoe.so (once).  Raises FileNotFoundError if it was not built.

    The path defaults to the in-tree build; the environment variable
    MOE_LIBRARY may name another build of the same library (the CPU-side
    sanitizer build used by the ABI tests)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = path or os.environ.get("MOE_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise FileNotFoundError("libmoe.so not built at %s (run python -m sparse_moe_layer_fwd_amd.build)"
                                % path)
    L = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    L.moe_init.argtypes = [ctypes.POINTER(MoEConfig), ctypes.POINTER(MoEWeights), ctypes.POINTER(vp)]
    L.moe_init.restype = ctypes.c_int
    L.moe_workspace_size.argtypes = [vp, i32, ctypes.POINTER(sz)]
    L.moe_workspace_size.restype = ctypes.c_int
    L.moe_route.argtypes = [vp, vp, i32, vp, vp, vp, vp, sz, vp]
    L.moe_route.restype = ctypes.c_int
    L.moe_forward.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, sz, vp]
    L.moe_forward.restype = ctypes.c_int
    L.moe_forward_noalloc.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp]
    L.moe_forward_noalloc.restype = ctypes.c_int
    L.moe_quantize_fp8.argtypes = [vp, ctypes.c_int64, vp, vp, vp]
    L.moe_quantize_fp8.restype = ctypes.c_int
    L.moe_nvfp4_tile.argtypes = [vp, vp, vp, vp, ctypes.c_int64, i32, i32, vp]
    L.moe_nvfp4_tile.restype = ctypes.c_int
    L.moe_destroy.argtypes = [vp]
    L.moe_destroy.restype = ctypes.c_int
    L.moe_status_string.argtypes = [ctypes.c_int]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_profile_enable.argtypes = [ctypes.c_int]
    L.moe_profile_enable.restype = ctypes.c_int
    L.moe_profile_read.argtypes = [ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_double)]
    L.moe_profile_read.restype = ctypes.c_int
    L.moe_stage_name.argtypes = [ctypes.c_int]
    L.moe_stage_name.restype = ctypes.c_char_p
    _LIB = L
    return L


def status_string(st: int) -> str:
    return lib().moe_status_string(int(st)).decode()


def _check(st: int, where: str) -> None:
    if st != MOE_OK:
        raise MoEError(st, where)


def moe_init(cfg: MoEConfig, w: MoEWeights, check: bool = True):
    """Returns (status, handle)."""
    h = ctypes.c_void_p()
    st = lib().moe_init(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(h))
    if check:
        _check(st, "moe_init")
    return st, h


def moe_workspace_size(h, T: int, check: bool = True):
    n = ctypes.c_size_t()
    st = lib().moe_workspace_size(h, int(T), ctypes.byref(n))
    if check:
        _check(st, "moe_workspace_size")
    return st, n.value


def moe_route(h, x, T, idx, gate, counts, ws, ws_bytes, stream, check: bool = True) -> int:
    st = lib().moe_route(h, x, int(T), idx, gate, counts, ws, int(ws_bytes), stream)
    if check:
        _check(st, "moe_route")
    return st


def moe_forward(h, x, T, y, idx, gate, counts, ws, ws_bytes, stream, check: bool = True) -> int:
    st = lib().moe_forward(h, x, int(T), y, idx, gate, counts, ws, int(ws_bytes), stream)
    if check:
        _check(st, "moe_forward")
    return st


def moe_forward_noalloc(h, x, T, y, idx, gate, counts, stream, check: bool = True) -> int:
    st = lib().moe_forward_noalloc(h, x, int(T), y, idx, gate, counts, stream)
    if check:
        _check(st, "moe_forward_noalloc")
    return st


MOE_SCRATCH_BYTES = 64 << 20     # include/moe.h


def moe_quantize_fp8(x, n, scale, out, stream, check: bool = True) -> int:
    st = lib().moe_quantize_fp8(x, int(n), scale, out, stream)
    if check:
        _check(st, "moe_quantize_fp8")
    return st


def moe_nvfp4_tile(codes, scales, codes_tiled, scales_tiled, n_mats, rows, k, stream,
                   check: bool = True) -> int:
    st = lib().moe_nvfp4_tile(codes, scales, codes_tiled, scales_tiled, int(n_mats), int(rows), int(k),
                              stream)
    if check:
        _check(st, "moe_nvfp4_tile")
    return st


def moe_destroy(h) -> int:
    return lib().moe_destroy(h)


def moe_profile_enable(enable) -> int:
    """False / True, or 2: the phase-split timing mode (include/moe.h)."""
    st = lib().moe_profile_enable(int(enable))
    _check(st, "moe_profile_enable")
    return st


def moe_profile_read():
    """-> {stage name: (launches, total ms)}; clears the record."""
    n = (ctypes.c_int32 * MOE_NUM_STAGES)()
    ms = (ctypes.c_double * MOE_NUM_STAGES)()
    _check(lib().moe_profile_read(n, ms), "moe_profile_read")
    return {lib().moe_stage_name(i).decode(): (int(n[i]), float(ms[i])) for i in range(MOE_NUM_STAGES)}
