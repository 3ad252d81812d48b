"""FP8 (OCP E4M3) weights and activations through the C ABI against the oracle.

The quantiser is compared bit for bit (moe_quantize_fp8 against the oracle's
E4M3 rule on the same bf16 inputs); whole layers to the y bar of 2e-2 with
routing exact, as the bf16 layers.  Shapes span the prefill tiles (128- and
256-row, several tiles per block), the decode kernels, the layer without
latent projection (x quantised by its own kernel), FP8 shared experts (dense
tiled and split-K), NVFP4 routed experts with FP8 shared ones, and the router
on x (latent rows written only as E4M3 codes).
"""
import numpy as np
import pytest
import torch

import oracle
from test_gpu_parity import log, prepare, run_and_check
from sparse_moe_layer_fwd_amd import binding as B
from sparse_moe_layer_fwd_amd.workloads import MoEConfig, f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _bf16_inputs():
    rng = np.random.default_rng(7)
    v = rng.standard_normal(1 << 16) * np.exp(rng.uniform(-12, 7, 1 << 16))
    special = [0.0, -0.0, 1.0, 1.0625, 1.1875, 17.0, 19.0, -3.0, 2.0 ** -10, 3 * 2.0 ** -10,
               15 * 2.0 ** -10, 448.0, 460.0, 1e6, -1e6, 2.0 ** -20, -(2.0 ** -20)]
    v[:len(special)] = special
    return f32_to_bf16_bits(v.astype(np.float32))


@pytest.mark.parametrize("scale", [1.0, 6.0 / 448.0, 3.0, 36.0 / 448.0])
def test_quantize_fp8_bitwise_equals_oracle(scale):
    xb = _bf16_inputs()
    dev = torch.device("cuda:0")
    x = torch.from_numpy(xb.view(np.int16)).to(dev)
    out = torch.empty(xb.size, dtype=torch.uint8, device=dev)
    sc = torch.tensor([scale], dtype=torch.float32, device=dev)
    log("quantize_fp8 n=%d scale=%g" % (xb.size, scale))
    B.moe_quantize_fp8(x.data_ptr(), xb.size, sc.data_ptr(), out.data_ptr(),
                       torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref = oracle.e4m3_quantize(oracle.bf16_to_f64(xb), np.float32(scale))
    got = out.cpu().numpy()
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(oracle.bf16_to_f64(xb[i:i + 1])[0]), hex(got[i]), hex(ref[i]))
                           for i in bad[:5]]


FP8_SMALL = {
    "fp8_prefill": MoEConfig("fp8_prefill", T=300, d=256, latent=256, n_experts=16, top_k=4,
                             ffn=256, expert="fp8"),
    "fp8_hot_cold_shared": MoEConfig("fp8_hot_cold_shared", T=700, d=512, latent=256,
                                     n_experts=8, top_k=4, ffn=512, expert="fp8", zipf_s=1.1,
                                     n_shared=1, shared_ffn=256, shared_fp8=True),
    "fp8_decode": MoEConfig("fp8_decode", T=40, d=512, latent=256, n_experts=32, top_k=4,
                            ffn=512, expert="fp8"),
    "fp8_decode_shared": MoEConfig("fp8_decode_shared", T=24, d=512, latent=256, n_experts=16,
                                   top_k=3, ffn=256, expert="fp8", n_shared=1, shared_ffn=256,
                                   shared_fp8=True),
    "fp8_no_latent_two_shared": MoEConfig("fp8_no_latent_two_shared", T=200, d=256, latent=256,
                                          n_experts=8, top_k=2, ffn=256, expert="fp8",
                                          has_latent_proj=False, n_shared=2, shared_ffn=128,
                                          shared_fp8=True),
    "nvfp4_experts_fp8_shared": MoEConfig("nvfp4_experts_fp8_shared", T=300, d=512, latent=256,
                                          n_experts=16, top_k=4, ffn=256, expert="nvfp4",
                                          n_shared=1, shared_ffn=256, shared_fp8=True),
    "bf16_experts_fp8_shared_decode": MoEConfig("bf16_experts_fp8_shared_decode", T=33, d=512,
                                                latent=256, n_experts=16, top_k=2, ffn=256,
                                                n_shared=1, shared_ffn=512, shared_fp8=True),
    "fp8_router_on_x": MoEConfig("fp8_router_on_x", T=150, d=256, latent=256, n_experts=16,
                                 top_k=3, ffn=256, expert="fp8", router_on_x=True),
    "fp8_decode_router_on_x": MoEConfig("fp8_decode_router_on_x", T=40, d=512, latent=256,
                                        n_experts=16, top_k=4, ffn=256, expert="fp8",
                                        router_on_x=True),
    # reductions of 512 and 1024 codes: 32 codes per lane and step in decode
    "fp8_decode_wide_shared": MoEConfig("fp8_decode_wide_shared", T=24, d=1024, latent=512,
                                        n_experts=16, top_k=3, ffn=1024, expert="fp8",
                                        n_shared=1, shared_ffn=512, shared_fp8=True),
    "fp8_decode_max_experts_max_k": MoEConfig("fp8_decode_max_experts_max_k", T=20, d=256,
                                              latent=256, n_experts=1024, top_k=64, ffn=256,
                                              expert="fp8"),
    # 100 tokens: projections and FP8 shared experts on the split-K skinny
    # kernel over two 64-row chunks
    "fp8_shared_split_k_two_chunks": MoEConfig("fp8_shared_split_k_two_chunks", T=100, d=512,
                                               latent=256, n_experts=16, top_k=4, ffn=256,
                                               n_shared=1, shared_ffn=512, shared_fp8=True),
    # skinny expert kernel above 64 tokens: several 64-row chunks per hot expert
    "fp8_skinny_multi_chunk": MoEConfig("fp8_skinny_multi_chunk", T=120, d=512, latent=512,
                                        n_experts=8, top_k=4, ffn=512, expert="fp8", zipf_s=1.1),
    "fp8_multi_item": MoEConfig("fp8_multi_item", T=8192, d=256, latent=256, n_experts=8,
                                top_k=4, ffn=1024, expert="fp8", zipf_s=1.1),
}


@pytest.mark.parametrize("name", sorted(FP8_SMALL))
def test_fp8_small_shapes(name):
    run_and_check(FP8_SMALL[name])


def test_fp8_deterministic():
    cfg = FP8_SMALL["fp8_hot_cold_shared"]
    wl, dl, x = prepare(cfg, 2)
    y1 = dl.forward(x)
    y2 = dl.forward(x)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
