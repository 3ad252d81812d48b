"""moe_forward captured in a HIP graph (through torch.cuda.graph): every replay
gives bitwise the eager result for the input then in x, with eager work and
synchronisations between the replays.  The library enqueues only kernels (no
allocation, no memset node) on the caller's stream, so a serving loop can
capture a whole step."""
import numpy as np
import pytest
import torch

from test_gpu_parity import log, prepare
from sparse_moe_layer_fwd_amd.workloads import MoEConfig

pytestmark = pytest.mark.gpu

GRAPH_CASES = {
    "prefill_latent_shared": MoEConfig("prefill_latent_shared", T=300, d=256, latent=128,
                                       n_experts=16, top_k=3, ffn=128, n_shared=1, shared_ffn=192),
    "decode_fp8_shared": MoEConfig("decode_fp8_shared", T=40, d=512, latent=256, n_experts=16,
                                   top_k=4, ffn=512, expert="fp8", n_shared=1, shared_ffn=256,
                                   shared_fp8=True),
    "prefill_nvfp4_zipf": MoEConfig("prefill_nvfp4_zipf", T=700, d=512, latent=256, n_experts=8,
                                    top_k=4, ffn=512, expert="nvfp4", zipf_s=1.1),
}


@pytest.mark.parametrize("name", sorted(GRAPH_CASES))
def test_graph_replays_match_eager(name):
    cfg = GRAPH_CASES[name]
    log("graph case %s T=%d" % (name, cfg.T))
    wl, dl, x = prepare(cfg, 0, margin=False)
    ws = dl.new_workspace(cfg.T)
    y_eager = torch.empty((cfg.T, cfg.d), dtype=dl.act_torch_dtype(), device=x.device)
    y_graph = torch.empty_like(y_eager)
    xs = [x.clone()] + [torch.roll(x, shifts=17 * (i + 1), dims=0).contiguous() for i in range(3)]
    x_in = xs[0].clone()
    dl.forward(x_in, ws=ws, y=y_eager)          # eager first: kernel attributes set outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):                   # the library enqueues on the capturing stream
        dl.forward(x_in, ws=ws, y=y_graph)
    torch.cuda.synchronize()
    for i, xi in enumerate(xs):
        x_in.copy_(xi)
        g.replay()
        torch.cuda.synchronize()
        got = y_graph.clone()
        # eager work between replays, on the same workspace
        dl.forward(x_in, ws=ws, y=y_eager)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), y_eager.view(torch.int16)), "replay %d differs" % i
