"""Invariances of the layer, checked on the GPU through the C ABI.

Experts are interchangeable up to their index ("NVIDIA Nemotron 3: Efficient
and Open Intelligence" Korean summary, section 2.2 LatentMoE: the router picks
K of N identical-shape expert FFNs).  Relabelling them (permuting the router
rows, the router bias and the expert weight stacks together) must route every
token to the relabelled experts with the same gates in the same order and give
bitwise the same y: every logit is the same dot product in the same order, the
expert-sorted rows of an expert are the same rows in the same order, and the
combine sums a token's K outputs in logit-rank order, not expert-id order.

A permutation of the latent basis (W_d rows, W_r columns, W1 columns, W2 rows,
W_u columns; whole 16-element blocks so that NVFP4 blocks stay intact) leaves
the layer's value unchanged.  It reorders the fp32 reductions over the latent
dimension (router, W1, W_u), so y is not bitwise equal; routing is checked
exactly against the unpermuted run and y within the bf16 bar.
"""
import numpy as np
import pytest
import torch

from test_gpu_parity import GATE_TOL, SMALL, TOL, log, rel_err
from helpers import margin_filter
from sparse_moe_layer_fwd_amd.layer import DeviceLayer, x_to_device
from sparse_moe_layer_fwd_amd.workloads import Workload

pytestmark = pytest.mark.gpu


class _Relabelled(Workload):
    """Expert e of `base` becomes expert pi[e]."""

    def __init__(self, base: Workload, pi: np.ndarray):
        super().__init__(base.cfg, base.seed)
        self.base, self.pi = base, pi
        self.inv = np.argsort(pi)
        self.set_x(base.x())

    def w_router(self):
        return np.ascontiguousarray(self.base.w_router()[self.inv])

    def b_router(self):
        b = self.base.b_router()
        return None if b is None else np.ascontiguousarray(b[self.inv])

    def w1(self, e):
        return self.base.w1(int(self.inv[e]))

    def w2(self, e):
        return self.base.w2(int(self.inv[e]))


def _cols(a, perm):
    return np.ascontiguousarray(a[..., perm])


class _LatentPermuted(Workload):
    """The latent basis permuted by `perm` (a permutation of whole 16-element blocks)."""

    def __init__(self, base: Workload, perm: np.ndarray):
        super().__init__(base.cfg, base.seed)
        self.base, self.perm = base, perm
        self.set_x(base.x())

    def w_down(self):
        return np.ascontiguousarray(self.base.w_down()[self.perm])

    def w_up(self):
        return _cols(self.base.w_up(), self.perm)

    def w_router(self):
        w = self.base.w_router()
        return w if self.cfg.router_on_x else _cols(w, self.perm)

    def _nvfp4_cols(self, m):             # permute blocks along the reduction (latent) dimension
        codes, scales, g = m
        bperm = self.perm[::16] // 16
        c = codes.reshape(codes.shape[0], -1, 8)[:, bperm].reshape(codes.shape)
        return np.ascontiguousarray(c), np.ascontiguousarray(scales[:, bperm]), g

    def w1(self, e):                      # [m][l]: latent columns
        w = self.base.w1(e)
        return self._nvfp4_cols(w) if self.cfg.expert == "nvfp4" else _cols(w, self.perm)

    def w2(self, e):                      # [l][m]: latent rows
        w = self.base.w2(e)
        if self.cfg.expert == "nvfp4":
            codes, scales, g = w
            return np.ascontiguousarray(codes[self.perm]), np.ascontiguousarray(scales[self.perm]), g
        return np.ascontiguousarray(w[self.perm])


def _run(wl):
    y, idx, gate, counts = DeviceLayer.from_workload(wl).forward(x_to_device(wl), routing=True)
    torch.cuda.synchronize()
    return y, idx.cpu().numpy(), gate.cpu().numpy(), counts.cpu().numpy()


CASES = ["hot_cold_nvfp4", "latent_bf16_prefill", "decode_bf16", "decode_nvfp4", "multi_item_256"]


@pytest.mark.parametrize("name", CASES)
def test_expert_relabel_bitwise(name):
    cfg = SMALL[name]
    log("case relabel %s" % name)
    base = Workload(cfg, 5)
    margin_filter(base, cfg)
    pi = np.random.default_rng(11).permutation(cfg.n_experts)
    y0, i0, g0, c0 = _run(base)
    y1, i1, g1, c1 = _run(_Relabelled(base, pi))
    assert np.array_equal(i1, pi[i0]), "relabelled routing differs"
    assert np.array_equal(g1, g0), "gates differ"
    assert np.array_equal(c1[pi], c0), "counts differ"
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16)), "y not bitwise equal"


@pytest.mark.parametrize("name", ["hot_cold_nvfp4", "latent_bf16_prefill", "decode_bf16",
                                  "router_on_x_shared"])
def test_latent_block_permutation(name):
    cfg = SMALL[name]
    log("case latent permutation %s" % name)
    base = Workload(cfg, 7)
    margin_filter(base, cfg)
    nb = cfg.latent // 16
    bperm = np.random.default_rng(13).permutation(nb)
    perm = (bperm[:, None] * 16 + np.arange(16)[None, :]).ravel()
    y0, i0, g0, c0 = _run(base)
    y1, i1, g1, c1 = _run(_LatentPermuted(base, perm))
    assert np.array_equal(np.sort(i1, 1), np.sort(i0, 1)) and np.array_equal(c1, c0)
    assert np.max(np.abs(g1 - g0)) <= GATE_TOL
    if cfg.router_on_x:                   # the router reads x: logits are the same sums
        assert np.array_equal(i1, i0) and np.array_equal(g1, g0)
    err = rel_err(y1.float().cpu().numpy().astype(np.float64), y0.float().cpu().numpy().astype(np.float64))
    log("  y rel diff %.3e" % err)
    assert err <= TOL[cfg.expert]
