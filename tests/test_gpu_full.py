"""Parity at the full sizes of the layer configurations, in the launch
configuration the benchmark times: routing (index sets, counts, gates) on every
token, y on a seeded sample of tokens the oracle computes one by one."""
import numpy as np
import pytest
import torch

import oracle
from test_gpu_parity import TOL, check_routing, log, prepare, rel_err
from sparse_moe_layer_fwd_amd.workloads import CONFIGS

pytestmark = pytest.mark.gpu

SAMPLE = 48


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cfg_id", [2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13])
def test_full_size_config(cfg_id):
    cfg = CONFIGS[cfg_id]
    log("full config %d %s: preparing" % (cfg_id, cfg.name))
    wl, dl, x = prepare(cfg, 0)
    log("  forward")
    y, idx, gate, counts = dl.forward(x, routing=True)
    torch.cuda.synchronize()
    tokens = np.sort(np.random.default_rng(cfg_id).choice(cfg.T, size=min(SAMPLE, cfg.T),
                                                          replace=False))
    log("  oracle")
    ref = oracle.forward(wl, cfg, tokens=tokens)
    check_routing(cfg, ref, idx, gate, counts)
    yg = y[torch.from_numpy(tokens).to(y.device)].float().cpu().numpy().astype(np.float64)
    err = rel_err(yg, ref.y)
    log("  y rel err %.3e (tol %.0e); max count %d, experts touched %d" % (
        err, TOL[cfg.expert], ref.counts.max(), int((ref.counts > 0).sum())))
    assert err <= TOL[cfg.expert]
