"""Parity at the full sizes of the layer configurations, in the launch
configuration the benchmark times.

Routing (index sets, counts, gates) is checked on every token.  y is checked
on every token for layers of up to 8192 tokens.  The two 16384-token
Ultra-like NVFP4 layers check y on a cover set the oracle picks from its own
routing: the first and the last token routed to every touched expert, plus 48
seeded random tokens.  Within an expert the expert-sorted rows follow token
order, so the first token lands in the expert's first row tile and the last
token in its last one (the remainder tile, or the partial full-height tile),
and every touched expert's weights are used by at least one checked output.
"""
import numpy as np
import pytest
import torch

import oracle
from test_gpu_parity import TOL, check_routing, log, prepare, rel_err
from sparse_moe_layer_fwd_amd.workloads import CONFIGS

pytestmark = pytest.mark.gpu

SAMPLE = 48
ALL_TOKENS_MAX_T = 8192


def cover_tokens(idx: np.ndarray, n_experts: int, seed: int) -> np.ndarray:
    """First and last token routed to each touched expert, plus SAMPLE random tokens."""
    T = idx.shape[0]
    tok = np.repeat(np.arange(T), idx.shape[1])
    e = idx.ravel()
    first = np.full(n_experts, T, dtype=np.int64)
    last = np.full(n_experts, -1, dtype=np.int64)
    np.minimum.at(first, e, tok)
    np.maximum.at(last, e, tok)
    touched = last >= 0
    rnd = np.random.default_rng(seed).choice(T, size=min(SAMPLE, T), replace=False)
    return np.unique(np.concatenate([first[touched], last[touched], rnd]))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg_id", [2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13])
def test_full_size_config(cfg_id):
    cfg = CONFIGS[cfg_id]
    log("full config %d %s: preparing" % (cfg_id, cfg.name))
    wl, dl, x = prepare(cfg, 0)
    log("  forward")
    y, idx, gate, counts = dl.forward(x, routing=True)
    torch.cuda.synchronize()
    if cfg.T <= ALL_TOKENS_MAX_T:
        tokens = None
    else:
        r = oracle.route(wl, cfg)
        tokens = cover_tokens(r.idx, cfg.n_experts, cfg_id)
        covered = np.unique(r.idx[tokens])
        assert np.array_equal(covered, np.flatnonzero(r.counts)), "cover set misses an expert"
    log("  oracle on %s tokens" % ("all %d" % cfg.T if tokens is None else "%d cover" % len(tokens)))
    ref = oracle.forward(wl, cfg, tokens=tokens)
    check_routing(cfg, ref, idx, gate, counts)
    yg = y.float().cpu().numpy().astype(np.float64)
    if tokens is not None:
        yg = yg[tokens]
    err = rel_err(yg, ref.y)
    log("  y rel err %.3e (tol %.0e) over %d tokens; max count %d, experts touched %d" % (
        err, TOL[cfg.expert], len(ref.tokens), ref.counts.max(), int((ref.counts > 0).sum())))
    assert err <= TOL[cfg.expert]
