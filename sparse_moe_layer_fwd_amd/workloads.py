"""Seeded synthetic workloads for the LatentMoE layer forward.

This module draws the inputs that both the HIP path and the CPU oracle consume.
It holds none of the layer's arithmetic: it only draws random numbers, rounds
them to their storage type (fp32 -> bf16, round-to-nearest-even) and packs
random NVFP4 codes.  Every tensor (and every expert's matrix) has its own
counter-style seed stream ``SeedSequence(seed, spawn_key=(tensor_id, index))``,
so any tensor can be regenerated alone, in any order, on any host.

Shapes follow the pages:
  * latent projection d -> l with d/l ~ 4, N' = N*d/l and K' = K*d/l experts
    ("NVIDIA Nemotron 3: Efficient and Open Intelligence" Korean summary,
    section 2.2 LatentMoE; the d=4096 / l=1024, 512-of-22 ablation shape is
    given there too);
  * Nano's 128 routed experts with 6 active plus 2 always-on shared experts
    (Nemotron 3 Nano blog, granular MoE section);
  * Ultra's d = 8192 with 512 experts and 22 active (Nemotron 3 Ultra release
    news, architecture paragraph);
  * NVFP4: E2M1 elements, 16-element micro-blocks with E4M3 scales and one
    FP32 global scale (Korean summary, section 2.4 NVFP4 Training).

Storage conventions (all row-major, weights stored [out][in] so the reduction
dimension is contiguous):
  x         [T][d]        bf16 (uint16 bits) or fp32
  w_down    [l][d]        act dtype            (absent for a standard MoE)
  w_router  [N][l]        fp32, b_router [N] fp32
  w1        [N][m][l]     bf16 / fp32 / NVFP4
  w2        [N][l][m]     bf16 / fp32 / NVFP4
  w_up      [d][l]        act dtype
  ws1       [S][ms][d], ws2 [S][d][ms]  act dtype (shared experts)
NVFP4 matrix [rows][cols]: codes uint8 [rows][cols/2] (element 2j in the low
nibble, 2j+1 in the high nibble), scales uint8 [rows][cols/16] (one E4M3 byte
per 16 consecutive elements of a row), gscale float32 (one per expert matrix).
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

__all__ = ["MoEConfig", "CONFIGS", "Workload", "f32_to_bf16_bits", "bf16_bits_to_f32",
           "config_by_name"]


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    """Shape and type of one LatentMoE (or standard MoE) layer."""
    name: str
    T: int                 # tokens in the batch
    d: int                 # hidden size
    latent: int            # latent size l (== d for a standard MoE)
    n_experts: int         # N routed experts
    top_k: int             # K active experts per token
    ffn: int               # m, expert FFN width
    n_shared: int = 0      # S always-on shared experts (at d)
    shared_ffn: int = 0    # shared expert FFN width
    has_latent_proj: bool = True
    act: str = "bf16"      # "f32" | "bf16": x, projections, activations
    expert: str = "bf16"   # "f32" | "bf16" | "nvfp4" | "fp8": routed expert weights
    zipf_s: float = 0.0    # > 0: Zipf(s) expert-popularity bias in the router
    router_on_x: bool = False  # router reads x at d instead of the latent z
    shared_fp8: bool = False   # shared expert weights (and their inputs) in FP8 E4M3
    margin: float = 1e-4   # top-K gap required by the margin filter (tests)
    description: str = ""

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)

    # ---- algorithmic work (counts only what the method must compute/move) ----
    def flops(self) -> float:
        T, d, l, N, K, m = self.T, self.d, self.latent, self.n_experts, self.top_k, self.ffn
        f = 2.0 * T * (d if self.router_on_x else l) * N   # router
        f += 4.0 * T * K * l * m                  # expert up + down
        if self.has_latent_proj:
            f += 4.0 * T * d * l                  # down + up projection
        f += 4.0 * T * d * self.shared_ffn * self.n_shared
        return f

    def expert_flops(self) -> float:
        return 4.0 * self.T * self.top_k * self.latent * self.ffn

    def expert_matrix_bytes(self) -> float:
        """Bytes of one expert's W1 + W2 as stored."""
        el = self.latent * self.ffn
        if self.expert == "nvfp4":
            return 2 * (el / 2 + el / 16 + 4)
        if self.expert == "fp8":
            return 2 * (el + 4)
        return 2 * el * (4 if self.expert == "f32" else 2)


def _cfg_list():
    return [
        MoEConfig("tiny_f32", T=64, d=256, latent=64, n_experts=16, top_k=4, ffn=128,
                  act="f32", expert="f32", margin=1e-3,
                  description="Tiny LatentMoE, fp32 everywhere"),
        MoEConfig("std_moe_nano", T=4096, d=2048, latent=2048, n_experts=128, top_k=6,
                  ffn=1024, n_shared=2, shared_ffn=1024, has_latent_proj=False,
                  description="Standard (l = d) MoE, Nano-like, 2 shared experts"),
        MoEConfig("latent_8b_prefill", T=8192, d=4096, latent=1024, n_experts=512,
                  top_k=22, ffn=1024, zipf_s=1.1,
                  description="LatentMoE ablation-like 8B-active prefill, Zipf routing"),
        MoEConfig("latent_ultra_decode", T=64, d=8192, latent=2048, n_experts=512,
                  top_k=22, ffn=2048,
                  description="LatentMoE Ultra-like batch decode, bf16 experts"),
        MoEConfig("latent_ultra_prefill_nvfp4", T=16384, d=8192, latent=2048,
                  n_experts=512, top_k=22, ffn=2048, expert="nvfp4", zipf_s=1.1,
                  description="LatentMoE Ultra-like prefill, NVFP4 experts, Zipf routing"),
        # the ablation pair at equal d and m: standard MoE (128 experts, top-6 at
        # d) against the latent layer of configuration 3 (512 experts, top-22 at
        # l = d / 4), in prefill and in batch decode
        MoEConfig("std_8b_prefill", T=8192, d=4096, latent=4096, n_experts=128, top_k=6,
                  ffn=1024, has_latent_proj=False, zipf_s=1.1,
                  description="Standard MoE at the ablation shape (paired with 3), Zipf routing"),
        MoEConfig("std_8b_decode", T=64, d=4096, latent=4096, n_experts=128, top_k=6,
                  ffn=1024, has_latent_proj=False,
                  description="Standard MoE at the ablation shape, batch decode"),
        MoEConfig("latent_8b_decode", T=64, d=4096, latent=1024, n_experts=512, top_k=22,
                  ffn=1024,
                  description="LatentMoE at the ablation shape (configuration 3), batch decode"),
        # configurations 3 and 8 with the router at d (on x) and two always-on
        # shared experts at d beside the latent routed experts
        MoEConfig("latent_8b_prefill_router_x", T=8192, d=4096, latent=1024, n_experts=512,
                  top_k=22, ffn=1024, n_shared=2, shared_ffn=1024, router_on_x=True,
                  zipf_s=1.1,
                  description="LatentMoE, router and 2 shared experts at d, prefill, Zipf routing"),
        MoEConfig("latent_8b_decode_router_x", T=64, d=4096, latent=1024, n_experts=512,
                  top_k=22, ffn=1024, n_shared=2, shared_ffn=1024, router_on_x=True,
                  description="LatentMoE, router and 2 shared experts at d, batch decode"),
        # FP8 (E4M3) weights and activations: configuration 3's prefill and
        # configuration 4's decode with FP8 experts, and configuration 5 with an
        # FP8 shared expert beside its NVFP4 routed experts
        MoEConfig("latent_8b_prefill_fp8", T=8192, d=4096, latent=1024, n_experts=512,
                  top_k=22, ffn=1024, expert="fp8", zipf_s=1.1,
                  description="LatentMoE ablation-like prefill, FP8 experts, Zipf routing"),
        MoEConfig("latent_ultra_decode_fp8", T=64, d=8192, latent=2048, n_experts=512,
                  top_k=22, ffn=2048, expert="fp8",
                  description="LatentMoE Ultra-like batch decode, FP8 experts"),
        MoEConfig("latent_ultra_prefill_nvfp4_shared_fp8", T=16384, d=8192, latent=2048,
                  n_experts=512, top_k=22, ffn=2048, expert="nvfp4", n_shared=1,
                  shared_ffn=2048, shared_fp8=True, zipf_s=1.1,
                  description="LatentMoE Ultra-like prefill, NVFP4 experts, FP8 shared expert"),
    ]


CONFIGS = {i + 1: c for i, c in enumerate(_cfg_list())}


def config_by_name(name: str) -> MoEConfig:
    for c in CONFIGS.values():
        if c.name == name:
            return c
    raise KeyError(name)


# ---------------------------------------------------------------- storage types
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (b >> 16) & np.uint32(1)
    out = ((b + np.uint32(0x7FFF) + r) >> 16).astype(np.uint16)
    return out


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# Tensor ids for the seed streams.  Never renumber: stored fixtures depend on them.
_TID = {"x": 1, "x_redraw": 2, "w_down": 3, "w_router": 4, "b_router": 5, "w1": 6,
        "w2": 7, "w_up": 8, "ws1": 9, "ws2": 10, "nvfp4_w1": 11, "nvfp4_w2": 12,
        "fp8_w1": 13, "fp8_w2": 14, "fp8_ws1": 15, "fp8_ws2": 16}

# NVFP4 test weights are drawn directly as codes (no quantiser is needed: the
# oracle and the kernels both consume the same packed bits).  One random byte
# per element: its low 7 bits pick the E2M1 magnitude code 0..7 through a
# 128-entry table (bell-like frequencies 15,26,23,19,16,15,9,5 out of 128), its
# top bit is the sign.
_E2M1_MAG_LUT = np.repeat(np.arange(8, dtype=np.uint8),
                          np.array([15, 26, 23, 19, 16, 15, 9, 5]))
assert _E2M1_MAG_LUT.size == 128
# E4M3 block-scale bytes: exponent field 5..8 and any mantissa (positive, finite,
# values 0.25 .. 3.75).  One random byte per block: bits 0-1 -> exponent field
# - 5, bits 2-4 -> mantissa.
# Global scale = _NVFP4_C / sqrt(fan_in) keeps the decoded weights near
# N(0, 1/fan_in) in spread (element rms of code*scale is about 3.5).
_NVFP4_C = 0.3

# FP8 (E4M3) test weights are drawn directly as codes too: per element one
# 16-bit random word; bits 0-6 pick the exponent field through a 128-entry
# table shaped like a quantised N(0, 100^2) (exponent fields 15..6 with
# frequencies 1,25,41,29,16,8,4,2,1,1 out of 128), bits 7-9 the mantissa (7
# becomes 6 under exponent field 15, which would be NaN), bit 10 the sign.
# The per-matrix weight scale _FP8_C / sqrt(fan_in) gives decoded weights of
# rms about 1/sqrt(fan_in) (the codes' rms is 106.5).
_FP8_EXP_LUT = np.repeat(np.array([15, 14, 13, 12, 11, 10, 9, 8, 7, 6], dtype=np.uint8),
                         np.array([1, 25, 41, 29, 16, 8, 4, 2, 1, 1]))
assert _FP8_EXP_LUT.size == 128
_FP8_C = 1.0 / 106.5
# Static per-tensor activation scales of FP8 layers (a calibration constant
# each: amax / 448 for an expected amax of 6 for the unit-variance inputs z and
# x, and 36 for the squared-ReLU hidden activations).
FP8_ACT_AMAX = (6.0, 36.0)


class Workload:
    """Lazily generated, seeded inputs of one layer configuration.

    Every accessor returns the *stored* representation (uint16 bf16 bits,
    float32, or NVFP4 (codes, scales, gscale)).  Accessors may be called in
    any order; each tensor depends only on (seed, tensor id, index).
    """

    def __init__(self, cfg: MoEConfig, seed: int = 0, nvfp4_2d_blocks: bool = False):
        self.cfg = cfg
        self.seed = int(seed)
        self.nvfp4_2d_blocks = nvfp4_2d_blocks
        self._x_override: Optional[np.ndarray] = None

    # ------------------------------------------------------------ rng plumbing
    def _rng(self, name: str, *index: int) -> np.random.Generator:
        ss = np.random.SeedSequence(self.seed, spawn_key=(_TID[name],) + tuple(int(i) for i in index))
        return np.random.Generator(np.random.PCG64(ss))

    def _normal(self, name, shape, std, *index) -> np.ndarray:
        g = self._rng(name, *index)
        a = g.standard_normal(size=shape, dtype=np.float32)
        a *= np.float32(std)
        return a

    def _store(self, a: np.ndarray, dtype: str) -> np.ndarray:
        if dtype == "f32":
            return a.astype(np.float32, copy=False)
        if dtype == "bf16":
            return f32_to_bf16_bits(a)
        raise ValueError(dtype)

    # ------------------------------------------------------------ activations
    def x(self) -> np.ndarray:
        """x [T][d] ~ N(0, 1), stored in the activation dtype."""
        if self._x_override is not None:
            return self._x_override
        c = self.cfg
        return self._store(self._normal("x", (c.T, c.d), 1.0, 0), c.act)

    def x_redraw(self, t: int, attempt: int) -> np.ndarray:
        """A fresh draw of token t's row (used by the test-side margin filter)."""
        c = self.cfg
        return self._store(self._normal("x_redraw", (c.d,), 1.0, t, attempt), c.act)

    def set_x(self, x: np.ndarray) -> None:
        """Replace x (e.g. after the margin filter redrew some rows)."""
        self._x_override = np.ascontiguousarray(x)

    # ------------------------------------------------------------ dense weights
    def w_down(self) -> Optional[np.ndarray]:
        c = self.cfg
        if not c.has_latent_proj:
            return None
        return self._store(self._normal("w_down", (c.latent, c.d), 1.0 / math.sqrt(c.d), 0), c.act)

    def w_up(self) -> Optional[np.ndarray]:
        c = self.cfg
        if not c.has_latent_proj:
            return None
        return self._store(self._normal("w_up", (c.d, c.latent), 1.0 / math.sqrt(c.latent), 0), c.act)

    def w_router(self) -> np.ndarray:
        c = self.cfg
        fan_in = c.d if c.router_on_x else c.latent
        return self._normal("w_router", (c.n_experts, fan_in), 1.0 / math.sqrt(fan_in), 0)

    def b_router(self) -> Optional[np.ndarray]:
        """Zipf(s) popularity bias: b_e = -s * ln(rank_e), rank a seeded permutation of 1..N."""
        c = self.cfg
        if c.zipf_s <= 0:
            return None
        rank = self._rng("b_router", 0).permutation(c.n_experts) + 1
        return (-c.zipf_s * np.log(rank.astype(np.float64))).astype(np.float32)

    def ws1(self):
        """Shared W1 [S][sf][d] in the act dtype, or (E4M3 codes, scale) with shared_fp8."""
        c = self.cfg
        if c.n_shared == 0:
            return None
        if c.shared_fp8:
            return self._fp8("fp8_ws1", (c.n_shared, c.shared_ffn, c.d), c.d, 0)
        return self._store(self._normal("ws1", (c.n_shared, c.shared_ffn, c.d), 1.0 / math.sqrt(c.d), 0), c.act)

    def ws2(self):
        """Shared W2 [S][d][sf], as ws1."""
        c = self.cfg
        if c.n_shared == 0:
            return None
        if c.shared_fp8:
            return self._fp8("fp8_ws2", (c.n_shared, c.d, c.shared_ffn), c.shared_ffn, 0)
        return self._store(self._normal("ws2", (c.n_shared, c.d, c.shared_ffn),
                                        1.0 / math.sqrt(c.shared_ffn), 0), c.act)

    # ------------------------------------------------------------ expert weights
    def _nvfp4(self, name: str, e: int, rows: int, cols: int):
        g = self._rng(name, e)
        r = g.integers(0, 256, size=(rows, cols), dtype=np.uint8)
        code = _E2M1_MAG_LUT[r & 127] | ((r >> 7) << 3)
        packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
        nb = cols // 16
        srows = (rows + 15) // 16 if self.nvfp4_2d_blocks else rows
        sb = g.integers(0, 256, size=(srows, nb), dtype=np.uint8)
        scales = ((((sb & 3) + 5) << 3) | ((sb >> 2) & 7)).astype(np.uint8)
        if self.nvfp4_2d_blocks:        # one scale per 16x16 block
            scales = np.repeat(scales, 16, axis=0)[:rows]
        gscale = np.float32(_NVFP4_C / math.sqrt(cols))
        return packed, np.ascontiguousarray(scales), gscale

    def _fp8(self, name: str, shape, fan_in: int, *index):
        g = self._rng(name, *index)
        r = g.integers(0, 1 << 16, size=shape, dtype=np.uint16)
        e = _FP8_EXP_LUT[r & 127]
        m = ((r >> 7) & 7).astype(np.uint8)
        m = np.where((e == 15) & (m == 7), np.uint8(6), m)
        code = (((r >> 10) & 1).astype(np.uint8) << 7) | (e << 3) | m
        return np.ascontiguousarray(code.astype(np.uint8)), np.float32(_FP8_C / math.sqrt(fan_in))

    def w1(self, e: int):
        """Expert e's W1 [m][l]: an array, (codes, scales, gscale) for NVFP4, or
        (E4M3 codes, scale) for FP8."""
        c = self.cfg
        if c.expert == "nvfp4":
            return self._nvfp4("nvfp4_w1", e, c.ffn, c.latent)
        if c.expert == "fp8":
            return self._fp8("fp8_w1", (c.ffn, c.latent), c.latent, e)
        return self._store(self._normal("w1", (c.ffn, c.latent), 1.0 / math.sqrt(c.latent), e), c.expert)

    def w2(self, e: int):
        """Expert e's W2 [l][m]: as w1."""
        c = self.cfg
        if c.expert == "nvfp4":
            return self._nvfp4("nvfp4_w2", e, c.latent, c.ffn)
        if c.expert == "fp8":
            return self._fp8("fp8_w2", (c.latent, c.ffn), c.ffn, e)
        return self._store(self._normal("w2", (c.latent, c.ffn), 1.0 / math.sqrt(c.ffn), e), c.expert)

    def act_scales(self) -> Optional[np.ndarray]:
        """FP8 experts: the per-tensor scales of the expert inputs z and h."""
        if self.cfg.expert != "fp8":
            return None
        return np.array([a / 448.0 for a in FP8_ACT_AMAX], dtype=np.float32)

    def shared_act_scales(self) -> Optional[np.ndarray]:
        """FP8 shared experts: the per-tensor scales of x and of their hidden rows."""
        if not (self.cfg.shared_fp8 and self.cfg.n_shared):
            return None
        return np.array([a / 448.0 for a in FP8_ACT_AMAX], dtype=np.float32)

    def experts_stacked(self, which: str, threads: int = 8):
        """All experts' W1 or W2 stacked on axis 0 (drawn in parallel threads).

        For NVFP4 returns (codes [N][r][c/2], scales [N][r][c/16], gscale [N]).
        """
        fn = self.w1 if which == "w1" else self.w2
        N = self.cfg.n_experts
        with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
            parts = list(ex.map(fn, range(N)))
        if self.cfg.expert == "nvfp4":
            return (np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]),
                    np.array([p[2] for p in parts], dtype=np.float32))
        if self.cfg.expert == "fp8":
            return np.stack([p[0] for p in parts]), np.array([p[1] for p in parts], dtype=np.float32)
        return np.stack(parts)
