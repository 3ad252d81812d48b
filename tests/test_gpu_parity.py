"""Parity of the HIP library (through the C ABI) with the fp64 oracle.

Bar: expert index sets and per-expert counts bit-exact; gates within 1e-5
(fp32 router and softmax against fp64); y within max|err|/max|ref| of 2e-2
(bf16), 5e-2 (NVFP4 weights, oracle on the same decoded weights), 2e-2 (FP8
weights and activations, oracle quantising the same way) and 1e-4 for the
all-fp32 layer.  Routing inputs are margin-filtered (no near-ties at the
K/K+1 boundary), as the layer configurations ask.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from helpers import margin_filter
from sparse_moe_layer_fwd_amd.layer import DeviceLayer, x_to_device
from sparse_moe_layer_fwd_amd.workloads import CONFIGS, MoEConfig, Workload

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "nvfp4": 5e-2, "fp8": 2e-2}
GATE_TOL = 1e-5


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def prepare(cfg, seed=0, margin=True, b_router=None):
    wl = Workload(cfg, seed)
    if b_router is not None:
        wl.b_router = lambda: b_router
    if margin:
        margin_filter(wl, cfg)
    dl = DeviceLayer.from_workload(wl)
    x = x_to_device(wl)
    return wl, dl, x


def check_routing(cfg, ref, idx, gate, counts, tokens=None):
    idx = idx.cpu().numpy()
    gate = gate.cpu().numpy()
    counts = counts.cpu().numpy()
    ridx = ref.idx if tokens is None else ref.idx[tokens]
    rgate = ref.gate if tokens is None else ref.gate[tokens]
    if tokens is not None:
        idx, gate = idx[tokens], gate[tokens]
    assert np.array_equal(np.sort(idx, axis=1), np.sort(ridx, axis=1)), "expert index sets differ"
    assert np.array_equal(counts, ref.counts), "per-expert counts differ"
    o = np.argsort(idx, axis=1)
    ro = np.argsort(ridx, axis=1)
    g = np.take_along_axis(gate, o, 1)
    rg = np.take_along_axis(rgate, ro, 1)
    assert np.max(np.abs(g - rg)) <= GATE_TOL, np.max(np.abs(g - rg))
    assert np.all(np.diff(gate, axis=1) <= 0), "gates not in descending-logit order"
    assert np.max(np.abs(gate.sum(axis=1) - 1.0)) <= 1e-6


def rel_err(y, ref_y):
    return float(np.max(np.abs(y - ref_y)) / np.max(np.abs(ref_y)))


def run_and_check(cfg, seed=0, tokens=None, margin=True, b_router=None):
    log("case %s seed=%d T=%d" % (cfg.name, seed, cfg.T))
    wl, dl, x = prepare(cfg, seed, margin, b_router)
    y, idx, gate, counts = dl.forward(x, routing=True)
    torch.cuda.synchronize()
    ref = oracle.forward(wl, cfg, tokens=tokens)
    check_routing(cfg, ref, idx, gate, counts)
    yg = y.float().cpu().numpy().astype(np.float64)
    if tokens is not None:
        yg = yg[tokens]
    err = rel_err(yg, ref.y)
    log("  y rel err %.3e (tol %.0e)" % (err, TOL[cfg.expert]))
    assert err <= TOL[cfg.expert], err
    # moe_route gives exactly the routing moe_forward used
    i2, g2, c2 = dl.route(x)
    torch.cuda.synchronize()
    assert torch.equal(i2, idx) and torch.equal(g2, gate) and torch.equal(c2, counts)
    return wl, dl, x, y


SMALL = {
    "latent_bf16_prefill": MoEConfig("latent_bf16_prefill", T=300, d=256, latent=128, n_experts=16,
                                     top_k=4, ffn=192),
    "latent_nvfp4_prefill_zipf": MoEConfig("latent_nvfp4_prefill_zipf", T=333, d=256, latent=128,
                                           n_experts=24, top_k=5, ffn=256, expert="nvfp4",
                                           zipf_s=1.1),
    "std_shared": MoEConfig("std_shared", T=200, d=256, latent=256, n_experts=8, top_k=2, ffn=128,
                            n_shared=2, shared_ffn=128, has_latent_proj=False),
    "decode_bf16": MoEConfig("decode_bf16", T=48, d=512, latent=256, n_experts=32, top_k=4, ffn=512),
    "decode_nvfp4": MoEConfig("decode_nvfp4", T=64, d=512, latent=256, n_experts=32, top_k=4,
                              ffn=512, expert="nvfp4"),
    "decode_latent_shared": MoEConfig("decode_latent_shared", T=40, d=512, latent=256,
                                      n_experts=16, top_k=3, ffn=256, n_shared=1, shared_ffn=128),
    "prefill_latent_shared": MoEConfig("prefill_latent_shared", T=150, d=256, latent=128,
                                       n_experts=16, top_k=3, ffn=128, n_shared=1, shared_ffn=192),
    "single_token": MoEConfig("single_token", T=1, d=512, latent=256, n_experts=16, top_k=4, ffn=256),
    "f32_grouped": MoEConfig("f32_grouped", T=200, d=128, latent=64, n_experts=8, top_k=3, ffn=128,
                             act="f32", expert="f32", margin=1e-3),
    "k_equals_1": MoEConfig("k_equals_1", T=100, d=256, latent=128, n_experts=8, top_k=1, ffn=128),
    "k_equals_n": MoEConfig("k_equals_n", T=90, d=256, latent=128, n_experts=6, top_k=6, ffn=128),
    "many_experts_small_batch": MoEConfig("many_experts_small_batch", T=70, d=256, latent=128,
                                          n_experts=1000, top_k=12, ffn=128),
    # T*K >= 256*N: 256-row tiles, each expert's remaining rows on 128-row tiles
    "hot_cold_bf16": MoEConfig("hot_cold_bf16", T=600, d=512, latent=256, n_experts=8, top_k=4,
                               ffn=256, zipf_s=1.1),
    "hot_cold_nvfp4": MoEConfig("hot_cold_nvfp4", T=700, d=512, latent=256, n_experts=8, top_k=4,
                                ffn=512, expert="nvfp4", zipf_s=1.1),
    # same regime with l not a multiple of 256
    "big_tiles_no_cold": MoEConfig("big_tiles_no_cold", T=600, d=256, latent=192, n_experts=8,
                                   top_k=4, ffn=128, zipf_s=1.1),
    # K = 64 reductions (latent and ffn): the shortest k-pipelines
    "short_k_bf16": MoEConfig("short_k_bf16", T=300, d=256, latent=64, n_experts=8, top_k=2,
                              ffn=64),
    "short_k_nvfp4_big_tiles": MoEConfig("short_k_nvfp4_big_tiles", T=600, d=256, latent=64,
                                         n_experts=4, top_k=4, ffn=64, expert="nvfp4"),
    # more output tiles than the persistent grid has blocks: each block runs
    # several tiles back to back through one continuous load pipeline
    "multi_item_256": MoEConfig("multi_item_256", T=8192, d=256, latent=256, n_experts=8, top_k=4,
                                ffn=1024, zipf_s=1.1),
    "multi_item_128": MoEConfig("multi_item_128", T=2048, d=256, latent=256, n_experts=64, top_k=4,
                                ffn=1024),
    "multi_item_nvfp4": MoEConfig("multi_item_nvfp4", T=8192, d=256, latent=256, n_experts=8,
                                  top_k=4, ffn=1024, expert="nvfp4", zipf_s=1.1),
    # bf16 experts of 128-255 rows on average: remainders of up to 192 rows on
    # 192-row tiles, longer ones on a partial 256-row tile (uniform routing:
    # both kinds; Zipf routing: also hot experts with full tiles before them)
    "mid_tiles_std_shared": MoEConfig("mid_tiles_std_shared", T=1000, d=256, latent=256,
                                      n_experts=32, top_k=6, ffn=256, n_shared=1, shared_ffn=128,
                                      has_latent_proj=False),
    "mid_tiles_zipf": MoEConfig("mid_tiles_zipf", T=800, d=256, latent=128, n_experts=16, top_k=4,
                                ffn=192, zipf_s=1.1),
    # small batches above 64 tokens on the skinny expert kernel: experts with
    # more than 64 rows run it in several 64-row chunks
    "skinny_multi_chunk_bf16": MoEConfig("skinny_multi_chunk_bf16", T=128, d=512, latent=256,
                                         n_experts=8, top_k=4, ffn=512, zipf_s=1.1),
    "skinny_multi_chunk_nvfp4": MoEConfig("skinny_multi_chunk_nvfp4", T=100, d=512, latent=256,
                                          n_experts=8, top_k=4, ffn=512, expert="nvfp4",
                                          zipf_s=1.1),
    # more than 32 routing chunks of 32 tokens: the per-expert chunk prefix runs
    # on ceil(N / 64) blocks of 16 wavefronts; 36 chunks (the last one 3 tokens)
    # leave wavefronts 12-15 without chunks, and N = 100 / 1000 leave a partial block
    "many_chunks_ragged": MoEConfig("many_chunks_ragged", T=1123, d=256, latent=128,
                                    n_experts=100, top_k=5, ffn=128, zipf_s=1.1),
    "many_chunks_max_experts": MoEConfig("many_chunks_max_experts", T=1100, d=256, latent=128,
                                         n_experts=1000, top_k=8, ffn=128),
    # the largest N and K the ABI accepts (top-K over 1024 logits, 64 per token)
    "max_experts_max_k": MoEConfig("max_experts_max_k", T=130, d=256, latent=128, n_experts=1024,
                                   top_k=64, ffn=128),
    # routing on x at d (shared experts at d beside latent routed experts)
    "router_on_x_shared": MoEConfig("router_on_x_shared", T=300, d=256, latent=128, n_experts=16,
                                    top_k=4, ffn=128, n_shared=1, shared_ffn=128,
                                    router_on_x=True),
    "router_on_x_decode_nvfp4": MoEConfig("router_on_x_decode_nvfp4", T=40, d=512, latent=256,
                                          n_experts=32, top_k=4, ffn=256, n_shared=1,
                                          shared_ffn=256, expert="nvfp4", router_on_x=True),
    "router_on_x_f32": MoEConfig("router_on_x_f32", T=120, d=128, latent=64, n_experts=8, top_k=2,
                                 ffn=128, act="f32", expert="f32", margin=1e-3, router_on_x=True),
}


def test_config1_tiny_f32_all_tokens():
    run_and_check(CONFIGS[1])


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_shapes(name):
    run_and_check(SMALL[name])


def test_all_tokens_to_one_expert():
    cfg = MoEConfig("one_hot_expert", T=260, d=256, latent=128, n_experts=16, top_k=2, ffn=128)
    b = np.zeros(16, dtype=np.float32)
    b[5] = 50.0
    run_and_check(cfg, b_router=b)


def test_deterministic_and_token_shuffle_equivariant():
    cfg = SMALL["latent_bf16_prefill"]
    wl, dl, x = prepare(cfg, 3)
    y1 = dl.forward(x)
    y2 = dl.forward(x)
    perm = torch.from_numpy(np.random.default_rng(0).permutation(cfg.T)).to(x.device)
    y3 = dl.forward(x[perm].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(y1[perm].view(torch.int16), y3.view(torch.int16))


def test_degree_two_homogeneity_bitwise():
    """K = 1 and no router bias: y(2x) = 4 y(x) bit for bit (powers of two are exact
    through bf16 rounding, the fp32 router and the squared ReLU)."""
    cfg = MoEConfig("homog", T=128, d=256, latent=128, n_experts=8, top_k=1, ffn=128)
    wl, dl, x = prepare(cfg, 1)
    y1 = dl.forward(x).float()
    y2 = dl.forward((x.float() * 2).to(x.dtype)).float()
    torch.cuda.synchronize()
    assert torch.equal(y2, 4 * y1)


class _IntegerRouter(Workload):
    """Exact logit ties: integer x in [-2, 2] and a router on x whose rows repeat
    eight integer patterns, so every logit is an integer, exact in fp32 and in
    fp64, and each value is shared by about N/8 experts.  The tie rule (equal
    logits: lower expert id first) then decides the order on both sides."""

    def x(self):
        from sparse_moe_layer_fwd_amd.workloads import f32_to_bf16_bits
        c = self.cfg
        v = np.random.default_rng([self.seed, 101]).integers(-2, 3, size=(c.T, c.d)).astype(np.float32)
        return f32_to_bf16_bits(v)

    def w_router(self):
        c = self.cfg
        pat = np.random.default_rng([self.seed, 102]).integers(-1, 2, size=(8, c.d)).astype(np.float32)
        return np.ascontiguousarray(pat[np.arange(c.n_experts) % 8])

    def b_router(self):
        return None


@pytest.mark.parametrize("n,k", [(40, 6), (300, 22), (1000, 64)])
def test_exact_logit_ties_take_lower_expert_ids(n, k):
    cfg = MoEConfig("ties_%d_%d" % (n, k), T=130, d=128, latent=64, n_experts=n, top_k=k,
                    ffn=128, router_on_x=True)
    log("case %s" % cfg.name)
    wl = _IntegerRouter(cfg, 0)
    dl = DeviceLayer.from_workload(wl)
    y, idx, gate, counts = dl.forward(x_to_device(wl), routing=True)
    torch.cuda.synchronize()
    ref = oracle.forward(wl, cfg)
    assert np.array_equal(idx.cpu().numpy(), ref.idx), "top-K order differs under exact ties"
    assert np.array_equal(counts.cpu().numpy(), ref.counts)
    assert np.max(np.abs(gate.cpu().numpy() - ref.gate)) <= GATE_TOL
    err = rel_err(y.float().cpu().numpy().astype(np.float64), ref.y)
    log("  y rel err %.3e" % err)
    assert err <= TOL["bf16"], err


class _UnitScaleFp4(Workload):
    """NVFP4 weights with global scale 1: their decoded values are exact bf16."""

    def w1(self, e):
        c, s, _ = super().w1(e)
        return c, s, np.float32(1.0)

    def w2(self, e):
        c, s, _ = super().w2(e)
        return c, s, np.float32(1.0)


class _DecodedBf16(Workload):
    """The same weights decoded (exactly) to bf16."""

    def __init__(self, fp4: Workload, cfg):
        super().__init__(cfg, fp4.seed)
        self._fp4 = fp4

    def w1(self, e):
        from sparse_moe_layer_fwd_amd.workloads import f32_to_bf16_bits
        return f32_to_bf16_bits(oracle.decode_expert(self._fp4.w1(e), "nvfp4").astype(np.float32))

    def w2(self, e):
        from sparse_moe_layer_fwd_amd.workloads import f32_to_bf16_bits
        return f32_to_bf16_bits(oracle.decode_expert(self._fp4.w2(e), "nvfp4").astype(np.float32))


@pytest.mark.parametrize("name", ["latent_nvfp4_prefill_zipf", "decode_nvfp4", "hot_cold_nvfp4"])
def test_nvfp4_path_bitwise_equals_bf16_path_on_decoded_weights(name):
    """In-register NVFP4 decode is exact: with a unit global scale the NVFP4 path
    and the bf16 path on the decoded weights give bitwise the same y."""
    cfg = SMALL[name]
    fp4 = _UnitScaleFp4(cfg, 0)
    dense = _DecodedBf16(fp4, cfg.replace(expert="bf16"))
    x = x_to_device(fp4)
    y4 = DeviceLayer.from_workload(fp4).forward(x)
    y16 = DeviceLayer.from_workload(dense).forward(x)
    torch.cuda.synchronize()
    assert torch.equal(y4.view(torch.int16), y16.view(torch.int16))


def test_error_paths_with_a_real_handle():
    from sparse_moe_layer_fwd_amd import binding as B
    cfg = SMALL["decode_bf16"]
    wl, dl, x = prepare(cfg, 0, margin=False)
    h = dl.handle
    ws = dl.new_workspace(cfg.T)
    y = torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device=x.device)
    s = torch.cuda.current_stream().cuda_stream
    fwd = lambda *a: B.moe_forward(*a, check=False)
    assert fwd(h, x.data_ptr(), cfg.T + 1, y.data_ptr(), None, None, None, ws.data_ptr(),
               ws.numel(), s) == B.MOE_ERR_INVALID_ARG
    assert fwd(h, x.data_ptr(), cfg.T, y.data_ptr(), None, None, None, ws.data_ptr(),
               ws.numel() - 1, s) == B.MOE_ERR_WORKSPACE
    assert fwd(h, x.data_ptr(), cfg.T, y.data_ptr(), None, None, None, None, 0, s) == \
        B.MOE_ERR_WORKSPACE
    assert fwd(h, x.data_ptr() + 2, cfg.T, y.data_ptr(), None, None, None, ws.data_ptr(),
               ws.numel(), s) == B.MOE_ERR_INVALID_ARG
    assert fwd(h, x.data_ptr(), cfg.T, None, None, None, None, ws.data_ptr(), ws.numel(), s) == \
        B.MOE_ERR_INVALID_ARG
    assert fwd(h, x.data_ptr(), -1, y.data_ptr(), None, None, None, ws.data_ptr(), ws.numel(), s) \
        == B.MOE_ERR_INVALID_ARG
    # T = 0 is a no-op
    assert fwd(h, x.data_ptr(), 0, y.data_ptr(), None, None, None, None, 0, s) == B.MOE_OK
    assert B.moe_workspace_size(h, 0)[1] == 0
    torch.cuda.synchronize()
