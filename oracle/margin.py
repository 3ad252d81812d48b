"""Margin filter for routing inputs (test infrastructure, like the rest of oracle/).

The layer configurations ask for routing inputs without near-ties at the top-K
boundary (a top-K margin).  This redraws every token whose fp64 gap between the
K-th and (K+1)-th logit is below ``cfg.margin``, using the oracle's own routing
steps and the generator's per-(token, attempt) redraw streams.
"""
import numpy as np

from .moe import decode_expert, latent_down, router_logits


def margin_filter(wl, cfg, max_rounds=20):
    """Redraw tokens whose fp64 top-K gap is below cfg.margin (the configs ask for
    routing inputs without near-ties).  Uses the oracle's routing; returns the
    number of rows redrawn.  The redraws come from the generator's per-(token,
    attempt) streams, so the result is reproducible."""
    if cfg.top_k >= cfg.n_experts:
        return 0
    x = np.array(wl.x(), copy=True)
    wd = wl.w_down()
    wd64 = None if wd is None else decode_expert(wd, cfg.act)
    wr, br = wl.w_router(), wl.b_router()
    redrawn = 0
    attempt = np.zeros(cfg.T, dtype=np.int64)
    bad = np.arange(cfg.T)
    for _ in range(max_rounds):
        xb = decode_expert(x[bad], cfg.act)
        lg = router_logits(xb if cfg.router_on_x else latent_down(xb, wd64), wr, br)
        srt = -np.sort(-lg, axis=1)
        gap = srt[:, cfg.top_k - 1] - srt[:, cfg.top_k]
        bad = bad[gap < cfg.margin]
        if bad.size == 0:
            break
        for t in bad:
            attempt[t] += 1
            x[t] = wl.x_redraw(int(t), int(attempt[t]))
            redrawn += 1
    else:
        raise RuntimeError("margin filter did not converge")
    wl.set_x(x)
    return redrawn
