"""The C-ABI library: it loads, exports every entry point include/moe.h
declares, and its host-side argument checks return the documented codes.
CPU only: no compute call is made (moe_init checks arguments before it looks
for a device, so invalid configurations are rejected without a GPU)."""
import ctypes
import os
import re

import pytest
import torch

from sparse_moe_layer_fwd_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from sparse_moe_layer_fwd_amd.build import build
        build()
    return B.lib()


def test_exports_every_declared_symbol(lib):
    decl = _declared()
    assert set(decl) == set(B.EXPORTED)
    for name in decl:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for st in range(6):
        assert B.status_string(st).startswith("MOE_")
    assert "unknown" in B.status_string(99)


FAKE = 1 << 20          # aligned, never dereferenced by moe_init


def _good_cfg(**kw):
    c = dict(d=256, latent=64, n_experts=16, top_k=4, ffn=128, n_shared=0, shared_ffn=0,
             max_tokens=64, has_latent_proj=1, act_dtype=B.MOE_BF16, expert_dtype=B.MOE_BF16)
    c.update(kw)
    return B.MoEConfig(**c)


def _good_w(**kw):
    w = dict(w_down=FAKE, w_router=FAKE, b_router=None, w1=FAKE, w2=FAKE, w1_scale=None,
             w2_scale=None, w1_gscale=None, w2_gscale=None, w_up=FAKE, ws1=None, ws2=None)
    w.update(kw)
    return B.MoEWeights(**w)


@pytest.mark.parametrize("cfg_kw,w_kw,expect", [
    (dict(top_k=17), {}, B.MOE_ERR_INVALID_ARG),                  # K > N
    (dict(top_k=0), {}, B.MOE_ERR_INVALID_ARG),
    (dict(d=0), {}, B.MOE_ERR_INVALID_ARG),
    (dict(max_tokens=0), {}, B.MOE_ERR_INVALID_ARG),
    (dict(has_latent_proj=0), {}, B.MOE_ERR_INVALID_ARG),         # latent != d without projection
    (dict(act_dtype=7), {}, B.MOE_ERR_INVALID_ARG),
    (dict(n_shared=1, shared_ffn=0), {}, B.MOE_ERR_INVALID_ARG),
    (dict(router_on_x=2), {}, B.MOE_ERR_INVALID_ARG),             # a flag: 0 or 1
    ({}, dict(w1=None), B.MOE_ERR_INVALID_ARG),
    ({}, dict(w_router=FAKE + 4), B.MOE_ERR_INVALID_ARG),        # misaligned
    ({}, dict(w_down=None), B.MOE_ERR_INVALID_ARG),
    (dict(expert_dtype=B.MOE_NVFP4), {}, B.MOE_ERR_INVALID_ARG),  # scales missing
    (dict(n_shared=2, shared_ffn=128), {}, B.MOE_ERR_INVALID_ARG),  # ws1/ws2 missing
    (dict(n_experts=2048, top_k=4), {}, B.MOE_ERR_UNSUPPORTED),
    (dict(n_experts=128, top_k=65), {}, B.MOE_ERR_UNSUPPORTED),
    (dict(latent=96), {}, B.MOE_ERR_UNSUPPORTED),                  # not a multiple of 64
    (dict(act_dtype=B.MOE_F32, expert_dtype=B.MOE_BF16), {}, B.MOE_ERR_UNSUPPORTED),
    (dict(act_dtype=B.MOE_BF16, expert_dtype=B.MOE_F32), {}, B.MOE_ERR_UNSUPPORTED),
    (dict(expert_dtype=4), {}, B.MOE_ERR_INVALID_ARG),
    # FP8 experts: per-matrix weight scales and the two activation scales
    (dict(latent=256, ffn=256, expert_dtype=B.MOE_FP8), {}, B.MOE_ERR_INVALID_ARG),
    (dict(latent=256, ffn=256, expert_dtype=B.MOE_FP8),
     dict(w1_gscale=FAKE, w2_gscale=FAKE, act_scale=FAKE + 2), B.MOE_ERR_INVALID_ARG),  # misaligned
    (dict(latent=64, expert_dtype=B.MOE_FP8),
     dict(w1_gscale=FAKE, w2_gscale=FAKE, act_scale=FAKE), B.MOE_ERR_UNSUPPORTED),      # l < 256
    (dict(latent=256, ffn=192, expert_dtype=B.MOE_FP8),
     dict(w1_gscale=FAKE, w2_gscale=FAKE, act_scale=FAKE), B.MOE_ERR_UNSUPPORTED),      # m % 128
    (dict(act_dtype=B.MOE_F32, expert_dtype=B.MOE_FP8), {}, B.MOE_ERR_UNSUPPORTED),
    # FP8 shared experts
    (dict(shared_fp8=1), {}, B.MOE_ERR_INVALID_ARG),                                 # no shared experts
    (dict(shared_fp8=2, n_shared=1, shared_ffn=256), dict(ws1=FAKE, ws2=FAKE), B.MOE_ERR_INVALID_ARG),
    (dict(shared_fp8=1, n_shared=1, shared_ffn=256), dict(ws1=FAKE, ws2=FAKE), B.MOE_ERR_INVALID_ARG),
    (dict(shared_fp8=1, n_shared=1, shared_ffn=192),
     dict(ws1=FAKE, ws2=FAKE, ws1_scale=FAKE, ws2_scale=FAKE, shared_act_scale=FAKE),
     B.MOE_ERR_UNSUPPORTED),                                                          # sf % 128
    # 32-bit byte offsets: T*K hidden rows of 2048 bf16 reach 4 GiB at T*K = 2^20
    (dict(d=8192, latent=2048, ffn=2048, n_experts=512, top_k=22, max_tokens=48000), {},
     B.MOE_ERR_UNSUPPORTED),
    (dict(d=65536, latent=32768, ffn=128), {}, B.MOE_ERR_UNSUPPORTED),               # W_d = 4 GiB
])
def test_init_rejects_bad_arguments(lib, cfg_kw, w_kw, expect):
    st, h = B.moe_init(_good_cfg(**cfg_kw), _good_w(**w_kw), check=False)
    assert st == expect, B.status_string(st)
    assert not h.value


def test_init_accepts_the_largest_offsets_below_4gib(lib):
    # 47662 tokens * 22 * 2048 * 2 bytes < 2^32: passes the shape rules (then
    # MOE_ERR_NO_DEVICE without a GPU, a handle with one)
    st, h = B.moe_init(_good_cfg(d=8192, latent=2048, ffn=2048, n_experts=512, top_k=22,
                                 max_tokens=47662), _good_w(), check=False)
    assert st in (B.MOE_OK, B.MOE_ERR_NO_DEVICE), B.status_string(st)
    if h.value:
        B.moe_destroy(h)


def test_init_null_pointers(lib):
    h = ctypes.c_void_p()
    assert lib.moe_init(None, ctypes.byref(_good_w()), ctypes.byref(h)) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_init(ctypes.byref(_good_cfg()), None, ctypes.byref(h)) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_init(ctypes.byref(_good_cfg()), ctypes.byref(_good_w()), None) == B.MOE_ERR_INVALID_ARG


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a HIP device is visible")
def test_init_without_device_reports_no_device(lib):
    st, h = B.moe_init(_good_cfg(), _good_w(), check=False)
    assert st == B.MOE_ERR_NO_DEVICE
    assert not h.value


def test_quantize_fp8_argument_checks(lib):
    assert lib.moe_quantize_fp8(FAKE, 0, FAKE, FAKE, None) == B.MOE_OK       # nothing to do
    assert lib.moe_quantize_fp8(FAKE, 15, FAKE, FAKE, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_fp8(FAKE, -16, FAKE, FAKE, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_fp8(None, 16, FAKE, FAKE, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_fp8(FAKE, 16, None, FAKE, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_fp8(FAKE + 8, 16, FAKE, FAKE, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_fp8(FAKE, 16, FAKE + 1, FAKE, None) == B.MOE_ERR_INVALID_ARG


def test_nvfp4_tile_argument_checks(lib):
    A, Bp, C, D = FAKE, FAKE + (1 << 20), FAKE + (2 << 20), FAKE + (3 << 20)
    assert lib.moe_nvfp4_tile(A, Bp, C, D, 0, 8, 64, None) == B.MOE_OK          # nothing to do
    assert lib.moe_nvfp4_tile(A, Bp, C, D, 1, 8, 96, None) == B.MOE_ERR_INVALID_ARG   # k % 64
    assert lib.moe_nvfp4_tile(A, Bp, C, D, 1, 8, 0, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_nvfp4_tile(A, Bp, C, D, 1, 0, 64, None) == B.MOE_ERR_INVALID_ARG   # rows
    assert lib.moe_nvfp4_tile(A, Bp, C, D, -1, 8, 64, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_nvfp4_tile(None, Bp, C, D, 1, 8, 64, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_nvfp4_tile(A, Bp, C + 4, D, 1, 8, 64, None) == B.MOE_ERR_INVALID_ARG  # alignment
    assert lib.moe_nvfp4_tile(A, Bp, A, D, 1, 8, 64, None) == B.MOE_ERR_INVALID_ARG       # in place
    assert lib.moe_nvfp4_tile(A, Bp, A + 128, D, 1, 8, 64, None) == B.MOE_ERR_INVALID_ARG  # overlap
    assert lib.moe_nvfp4_tile(A, Bp, C, C + 16, 1, 8, 64, None) == B.MOE_ERR_INVALID_ARG  # outputs overlap


def test_calls_on_null_handle(lib):
    n = ctypes.c_size_t()
    assert lib.moe_workspace_size(None, 4, ctypes.byref(n)) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_route(None, FAKE, 4, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_forward(None, FAKE, 4, FAKE, None, None, None, FAKE, 1 << 20, None) == \
        B.MOE_ERR_INVALID_ARG
    assert lib.moe_destroy(None) == B.MOE_OK
