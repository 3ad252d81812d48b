"""NVFP4 decode on the GPU over every E4M3 block scale and every E2M1 code.

NVFP4 weights are E2M1 elements with one E4M3 scale per 16-element block and an
FP32 global scale ("NVIDIA Nemotron 3: Efficient and Open Intelligence" Korean
summary, section 2.4 NVFP4 Training).  The kernels decode them in registers,
the tiled GEMM and the skinny kernel alike, through the hardware's scaled FP4
conversion (which applies the scale's power of two) and one fp32 multiply by
the remaining significand, to half the element's value.  They claim exactness
for every finite scale.  Here every one of the 254 finite E4M3 bytes (both signs,
0x00 and 0x80, the subnormals 0x01-0x07, up to 0x7E = 448) is used: expert e's
W1 and W2 carry scale byte FINITE[e] in every block, each block holds all 16
E2M1 codes once (a seeded permutation), and the global scale is 1.  Routing
is top-1 and forced: token t goes to the expert its spike names, so each
token's output depends on one scale byte only.

Checks, for the skinny kernel (127 tokens) and the tiled kernels (1016 tokens:
64-row tiles of the 4-wavefront kernel; 76200 tokens: 256-row tiles and
128-row remainder tiles of the 8-wavefront kernel):
  * routing exact against the oracle;
  * every token's y within 5e-2 of the oracle relative to that token's own
    largest |y| (outputs span many binades across scales), and exactly 0 for
    the two zero scales;
  * y bitwise equal to the bf16 path run on the same weights decoded by the
    oracle (exact in bf16), so any decode difference on any (code, scale) pair
    that reaches an output shows.
"""
import numpy as np
import pytest
import torch

import oracle
from test_gpu_parity import TOL, log
from sparse_moe_layer_fwd_amd.layer import DeviceLayer, x_to_device
from sparse_moe_layer_fwd_amd.workloads import MoEConfig, Workload, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

FINITE = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=np.uint8)
assert FINITE.size == 254
N = int(FINITE.size)


class _AllScales(Workload):
    """A latent layer with N = 254 NVFP4 experts, one scale byte per expert."""

    def __init__(self, cfg, seed, targets):
        super().__init__(cfg, seed)
        self.targets = np.asarray(targets, dtype=np.int64)

    def x(self):
        c = self.cfg
        v = self._normal("x", (c.T, c.d), 0.25, 0)
        v[np.arange(c.T), self.targets] = 4.0
        return f32_to_bf16_bits(v)

    def w_router(self):
        c = self.cfg
        w = np.zeros((c.n_experts, c.d), dtype=np.float32)
        w[np.arange(c.n_experts), np.arange(c.n_experts)] = 1.0
        return w

    def b_router(self):
        return None

    def _one_scale(self, name, e, rows, cols):
        g = self._rng(name, e)
        nb = cols // 16
        codes = np.argsort(g.random((rows, nb, 16)), axis=2).astype(np.uint8).reshape(rows, cols)
        packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
        scales = np.full((rows, nb), FINITE[e], dtype=np.uint8)
        return packed, scales, np.float32(1.0)

    def w1(self, e):
        return self._one_scale("nvfp4_w1", e, self.cfg.ffn, self.cfg.latent)

    def w2(self, e):
        return self._one_scale("nvfp4_w2", e, self.cfg.latent, self.cfg.ffn)


class _Decoded(_AllScales):
    """The same layer with the expert weights decoded (exactly) to bf16."""

    def w1(self, e):
        return f32_to_bf16_bits(oracle.decode_expert(super().w1(e), "nvfp4").astype(np.float32))

    def w2(self, e):
        return f32_to_bf16_bits(oracle.decode_expert(super().w2(e), "nvfp4").astype(np.float32))


def _cfg(T):
    return MoEConfig("nvfp4_all_scales_T%d" % T, T=T, d=256, latent=256, n_experts=N, top_k=1,
                     ffn=256, expert="nvfp4", router_on_x=True)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("T,offset", [(127, 0), (127, 127), (1016, 0), (76200, 0)])
def test_every_scale_byte_and_code(T, offset):
    cfg = _cfg(T)
    targets = (np.arange(T) + offset) % N
    log("case %s offset %d" % (cfg.name, offset))
    wl = _AllScales(cfg, 0, targets)
    x = x_to_device(wl)
    y4, idx, gate, counts = DeviceLayer.from_workload(wl).forward(x, routing=True)
    y16 = DeviceLayer.from_workload(_Decoded(cfg.replace(expert="bf16"), 0, targets)).forward(x)
    torch.cuda.synchronize()
    ref = oracle.forward(wl, cfg)
    assert np.array_equal(ref.idx[:, 0], targets)
    assert np.array_equal(idx.cpu().numpy(), ref.idx)
    assert np.array_equal(counts.cpu().numpy(), ref.counts)
    yg = y4.float().cpu().numpy().astype(np.float64)
    peak = np.max(np.abs(ref.y), axis=1)
    zero = peak == 0.0
    assert np.array_equal(np.flatnonzero(zero), np.flatnonzero(np.isin(targets, [0, 127])))
    assert np.all(yg[zero] == 0.0), "zero block scale did not decode to zero"
    err = np.max(np.abs(yg[~zero] - ref.y[~zero]), axis=1) / peak[~zero]
    worst = int(np.argmax(err))
    log("  worst per-token rel err %.3e (scale byte 0x%02x); %d zero-scale tokens" % (
        err[worst], FINITE[targets[~zero][worst]], int(zero.sum())))
    assert np.all(np.isfinite(yg))
    assert err.max() <= TOL["nvfp4"]
    same = torch.equal(y4.view(torch.int16), y16.view(torch.int16))
    if not same:
        bad = np.unique(targets[np.any(y4.view(torch.int16).cpu().numpy() != y16.view(torch.int16).cpu().numpy(),
                                       axis=1)])
        raise AssertionError("NVFP4 path differs from bf16 path for scale bytes %s" %
                             ", ".join("0x%02x" % FINITE[e] for e in bad[:16]))
