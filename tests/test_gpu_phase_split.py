"""The phase-split timing mode of the stage timer (moe_profile_enable(2) in
include/moe.h): each tiled grouped expert GEMM runs as two launches of the same
kernel, the full row tiles and then the remainder tiles.  It is a measurement
mode: y, the routing and every expert-sorted row must be bitwise those of the
single launch, and both phases must be recorded for a prefill layer whose
experts leave remainders."""
import pytest
import torch

from test_gpu_parity import log, prepare
from sparse_moe_layer_fwd_amd import binding as B
from sparse_moe_layer_fwd_amd.workloads import MoEConfig

pytestmark = pytest.mark.gpu

CASES = {
    # 64+ rows per expert on average: 256-row tiles plus remainder tiles
    "bf16_256": MoEConfig("split_bf16_256", T=1500, d=512, latent=256, n_experts=16, top_k=4,
                          ffn=512, zipf_s=1.1),
    # fewer rows per expert: 128-row tiles plus 64-row remainder tiles
    "bf16_128": MoEConfig("split_bf16_128", T=300, d=256, latent=128, n_experts=16, top_k=3,
                          ffn=256, n_shared=1, shared_ffn=192),
    "nvfp4_256": MoEConfig("split_nvfp4_256", T=1200, d=512, latent=256, n_experts=8, top_k=4,
                           ffn=512, expert="nvfp4", zipf_s=1.1),
    "fp8_256": MoEConfig("split_fp8_256", T=1500, d=512, latent=256, n_experts=16, top_k=4,
                         ffn=512, expert="fp8"),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_phase_split_is_bitwise_the_single_launch(name):
    cfg = CASES[name]
    log("phase split case %s T=%d" % (name, cfg.T))
    wl, dl, x = prepare(cfg, 0, margin=False)
    ws = dl.new_workspace(cfg.T)
    y1, idx1, gate1, counts1 = dl.forward(x, ws=ws, routing=True)
    torch.cuda.synchronize()
    y1 = y1.clone()
    B.moe_profile_read()
    try:
        B.moe_profile_enable(2)
        y2, idx2, gate2, counts2 = dl.forward(x, ws=ws, routing=True)
        torch.cuda.synchronize()
    finally:
        B.moe_profile_enable(False)
    stages = B.moe_profile_read()
    assert torch.equal(idx1, idx2) and torch.equal(counts1, counts2)
    assert torch.equal(gate1.view(torch.int32), gate2.view(torch.int32))
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), "split launches changed y"
    for k in ("expert_up", "expert_up_rem", "expert_down", "expert_down_rem"):
        assert stages[k][0] == 1, (k, stages[k])
    log("  full %.3f + rem %.3f ms (up), full %.3f + rem %.3f ms (down)" % (
        stages["expert_up"][1], stages["expert_up_rem"][1], stages["expert_down"][1],
        stages["expert_down_rem"][1]))


def test_profile_enable_rejects_other_modes():
    assert B.lib().moe_profile_enable(3) == B.MOE_ERR_INVALID_ARG
    assert B.lib().moe_profile_enable(-1) == B.MOE_ERR_INVALID_ARG
