"""Test-side helpers: small hand-built layers and the margin filter."""
from __future__ import annotations

import json
import os

import numpy as np

from sparse_moe_layer_fwd_amd.workloads import MoEConfig

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


class ArrayLayer:
    """A layer whose stored tensors are given as arrays (for pins and invariances)."""

    def __init__(self, cfg: MoEConfig, x, w_router, w1, w2, w_down=None, w_up=None,
                 b_router=None, ws1=None, ws2=None, act_scales=None, shared_act_scales=None):
        self.cfg = cfg
        self._x, self._wr, self._w1, self._w2 = x, w_router, w1, w2
        self._wd, self._wu, self._br, self._ws1, self._ws2 = w_down, w_up, b_router, ws1, ws2
        self._as, self._sas = act_scales, shared_act_scales

    def act_scales(self):
        return self._as

    def shared_act_scales(self):
        return self._sas

    def x(self):
        return self._x

    def w_down(self):
        return self._wd

    def w_up(self):
        return self._wu

    def w_router(self):
        return self._wr

    def b_router(self):
        return self._br

    def w1(self, e):
        return self._w1[e]

    def w2(self, e):
        return self._w2[e]

    def ws1(self):
        return self._ws1

    def ws2(self):
        return self._ws2


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def f64_layer(cfg: MoEConfig, rng: np.random.Generator, T=None):
    """Random float64 layer of shape ``cfg`` (act/expert dtype 'f64'), for pins."""
    T = cfg.T if T is None else T
    d, l, N, m = cfg.d, cfg.latent, cfg.n_experts, cfg.ffn
    c = cfg.replace(act="f64", expert="f64", T=T)
    x = rng.standard_normal((T, d))
    wd = rng.standard_normal((l, d)) / np.sqrt(d) if cfg.has_latent_proj else None
    wu = rng.standard_normal((d, l)) / np.sqrt(l) if cfg.has_latent_proj else None
    kr = d if cfg.router_on_x else l
    wr = rng.standard_normal((N, kr)) / np.sqrt(kr)
    w1 = rng.standard_normal((N, m, l)) / np.sqrt(l)
    w2 = rng.standard_normal((N, l, m)) / np.sqrt(m)
    ws1 = ws2 = None
    if cfg.n_shared:
        ws1 = rng.standard_normal((cfg.n_shared, cfg.shared_ffn, d)) / np.sqrt(d)
        ws2 = rng.standard_normal((cfg.n_shared, d, cfg.shared_ffn)) / np.sqrt(cfg.shared_ffn)
    return c, ArrayLayer(c, x, wr, w1, w2, wd, wu, None, ws1, ws2)


from oracle.margin import margin_filter  # noqa: E402,F401
