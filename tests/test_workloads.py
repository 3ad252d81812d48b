"""The seeded input generator: reproducibility, storage types, shapes and the
structure the configs ask for (Zipf skew, NVFP4 code validity)."""
import numpy as np
import torch

import oracle
from sparse_moe_layer_fwd_amd.workloads import (CONFIGS, MoEConfig, Workload, bf16_bits_to_f32,
                                                f32_to_bf16_bits)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(a), ref)
    assert np.array_equal(bf16_bits_to_f32(ref), torch.from_numpy(ref.view(np.int16)).view(
        torch.bfloat16).float().numpy())


def test_reproducible_and_order_independent():
    cfg = CONFIGS[3].replace(T=16, n_experts=8, d=64, latent=32, ffn=32)
    a, b = Workload(cfg, 5), Workload(cfg, 5)
    w1_first = a.w1(3)
    _ = b.x(), b.w1(0), b.w2(7)
    assert np.array_equal(w1_first, b.w1(3))
    assert np.array_equal(a.x(), b.x())
    assert not np.array_equal(a.w1(3), a.w1(4))
    assert not np.array_equal(Workload(cfg, 6).x(), a.x())


def test_shapes_and_dtypes_config1():
    cfg = CONFIGS[1]
    wl = Workload(cfg, 0)
    assert wl.x().shape == (64, 256) and wl.x().dtype == np.float32
    assert wl.w_down().shape == (64, 256)
    assert wl.w_up().shape == (256, 64)
    assert wl.w_router().shape == (16, 64) and wl.w_router().dtype == np.float32
    assert wl.w1(0).shape == (128, 64) and wl.w2(0).shape == (64, 128)
    assert wl.b_router() is None


def test_init_scales():
    cfg = MoEConfig("s", T=256, d=512, latent=128, n_experts=4, top_k=2, ffn=256)
    wl = Workload(cfg, 0)
    x = bf16_bits_to_f32(wl.x())
    assert abs(x.std() - 1) < 0.02
    w1 = bf16_bits_to_f32(wl.w1(0))
    assert abs(w1.std() * np.sqrt(128) - 1) < 0.02


def test_zipf_bias_is_log_zipf_of_a_permutation():
    cfg = CONFIGS[3]
    b = Workload(cfg, 0).b_router().astype(np.float64)
    rank = np.rint(np.exp(-b / cfg.zipf_s)).astype(int)
    assert sorted(rank.tolist()) == list(range(1, cfg.n_experts + 1))


def test_nvfp4_codes_are_finite_and_spread_like_the_dense_init():
    cfg = MoEConfig("f", T=8, d=256, latent=256, n_experts=2, top_k=1, ffn=512, expert="nvfp4")
    wl = Workload(cfg, 0)
    codes, scales, g = wl.w1(0)
    assert codes.shape == (512, 128) and scales.shape == (512, 16)
    assert np.all(np.isfinite(oracle.E4M3_TABLE[scales]))
    w = oracle.decode_nvfp4(codes, scales, g)
    assert 0.5 < w.std() * np.sqrt(256) < 2.0
    # every one of the 16 codes occurs
    nib = np.concatenate([codes & 15, codes >> 4]).ravel()
    assert set(np.unique(nib).tolist()) == set(range(16))


def test_nvfp4_2d_blocks_repeat_scales_over_16_rows():
    cfg = MoEConfig("f", T=8, d=64, latent=64, n_experts=1, top_k=1, ffn=48, expert="nvfp4")
    codes, scales, g = Workload(cfg, 0, nvfp4_2d_blocks=True).w1(0)
    assert scales.shape == (48, 4)
    for r in range(48):
        assert np.array_equal(scales[r], scales[(r // 16) * 16])
