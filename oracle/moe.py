"""fp64 reference of the LatentMoE layer forward (test infrastructure only).

The method is exact (no approximation), so every function here is the plain
definition written out in float64 on the exact stored input values (bf16, fp32
or NVFP4 bit patterns decoded to float64).  Nothing is rounded in between.
Library primitives used as steps: numpy matmul (fp64 BLAS), numpy stable sort,
numpy exp.

Method, per token (sources in ``oracle/__init__.py``):
  1. z = W_d x                (latent down-projection d -> l; [KO 2.2], [JA note])
     z = x                    (standard MoE: no projection, l = d)
  2. logits_e = W_r[e] . z + b_r[e]      (router GEMV on the latent; linear router)
     logits_e = W_r[e] . x + b_r[e]      (router_on_x: routing at d as [KO 2.2] draws it)
  3. sel = the K experts of largest logit; ties go to the lower expert id
  4. g_k = softmax over the K selected logits
  5. u = sum_k g_k W2[sel_k] sqrelu(W1[sel_k] z),  sqrelu(h) = max(h, 0)^2
     (expert FFN l -> m -> l; m is the expert FFN width in [KO 2.2])
  6. y = W_u u                (latent up-projection l -> d; [KO 2.2])
  7. y += sum_s Ws2[s] sqrelu(Ws1[s] x)  (always-on shared experts at d; [Nano],
     kept outside the latent compression per [KO 2.2])
FP8 layers ([Nano] FP8 post-training quantisation of weights and activations;
[Ultra] FP8 shared experts): weights are E4M3 codes times a per-matrix scale;
every GEMM input is replaced by q(v) = a * e4m3(Q(v, a)) with its static
per-tensor scale a (z or x before the first expert GEMM, the squared-ReLU
hidden rows before the second), Q as in ``e4m3_quantize``.
Readings where the pages are silent (router on the latent, softmax over the
selected K, squared-ReLU, no biases in the FFN, tie rule, Zipf bias added to the
logits) are listed with reasons in the repository's design notes.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np


# ----------------------------------------------------------------- storage decode
def bf16_to_f64(u16: np.ndarray) -> np.ndarray:
    """bfloat16 bits -> float64.  bf16 is the upper half of an IEEE binary32.

    Pinned: tests compare with torch's own bfloat16 -> float64 conversion.
    """
    u = np.ascontiguousarray(u16, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code (1 sign, 2 exponent bits with bias 1, 1 mantissa bit).

    NVFP4 elements are E2M1 ([KO 2.4]).  The element format is the OCP
    Microscaling FP4 one: exponent field 0 is subnormal (0 or 0.5), no Inf/NaN.
    Pinned: golden table of the format's 16 values in tests/golden.
    """
    sign = -1.0 if (code >> 3) & 1 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        mag = 0.5 * m                       # subnormal: 2^(1-1) * (m / 2)
    else:
        mag = 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return sign * mag


def e4m3_value(byte: int) -> float:
    """Value of an 8-bit E4M3 code (1 sign, 4 exponent bits with bias 7, 3 mantissa bits).

    NVFP4 block scales are E4M3 ([KO 2.4]); OCP FP8 E4M3 has no infinities,
    S.1111.111 is NaN, largest finite 448.  Pinned against torch.float8_e4m3fn.
    """
    sign = -1.0 if (byte >> 7) & 1 else 1.0
    e = (byte >> 3) & 0xF
    m = byte & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        mag = 2.0 ** (1 - 7) * (m / 8.0)    # subnormal
    else:
        mag = 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return sign * mag


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3_TABLE = np.array([e4m3_value(b) for b in range(256)], dtype=np.float64)


def e4m3_quantize(v, scale) -> np.ndarray:
    """E4M3 codes of v / scale: the FP8 activation rule of the layer.

    The decision is taken in fp32, the precision of the kernels' accumulators:
    t = fp32(fp32(v) * r) with r = 1 / scale correctly rounded to fp32; t is
    clamped to [-448, 448] (E4M3 has no infinities; 448 is its largest finite
    value) and rounded to the nearest E4M3 value, ties to the even mantissa.
    The sign bit is t's (a negative t that rounds to 0 gives code 0x80).
    Pinned: torch.float8_e4m3fn's rounding on in-range values, hand-worked
    ties, saturation, and code -> value -> code round trips.
    """
    r = np.float32(1.0) / np.float32(scale)
    t = np.asarray(v, dtype=np.float32) * r                    # fp32 product (IEEE, RNE)
    t = np.clip(t, np.float32(-448.0), np.float32(448.0)).astype(np.float64)
    sign = np.signbit(t).astype(np.uint8) << 7
    a = np.abs(t)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6                                        # below the smallest normal
    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)    # multiples of 2^-9; 8 -> 0x08
    nrm = ~sub
    mant, ex = np.frexp(a[nrm])                                # a = mant * 2^ex, mant in [0.5, 1)
    e = ex - 1
    q = np.rint((mant * 2.0 - 1.0) * 8.0).astype(np.int64)     # 3 mantissa bits, ties to even
    e = np.where(q == 8, e + 1, e)
    q = np.where(q == 8, 0, q)
    code[nrm] = ((e + 7) << 3) | q
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def e4m3_qdq(v, scale) -> np.ndarray:
    """The value an FP8 GEMM input v stands for: scale * e4m3(Q(v, scale))."""
    return E4M3_TABLE[e4m3_quantize(v, scale)] * float(np.float32(scale))


def decode_nvfp4(codes: np.ndarray, scales: np.ndarray, gscale) -> np.ndarray:
    """Two-level NVFP4 decode: w[r][c] = e2m1(code[r][c]) * e4m3(scale[r][c//16]) * g.

    [KO 2.4]: E2M1 elements, one E4M3 scale per 16-element micro-block, one FP32
    global scale.  Blocks run along a row (the reduction dimension); element 2j
    sits in the low nibble of byte j, 2j+1 in the high nibble (a reading: the
    pages give no packing).  Pinned: hand-packed golden example.
    """
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    rows, half = codes.shape
    cols = 2 * half
    el = np.empty((rows, cols), dtype=np.uint8)
    el[:, 0::2] = codes & 0x0F
    el[:, 1::2] = codes >> 4
    vals = E2M1_TABLE[el]
    s = E4M3_TABLE[np.ascontiguousarray(scales, dtype=np.uint8)]
    if s.shape != (rows, cols // 16):
        raise ValueError("scale shape %r does not match %r" % (s.shape, (rows, cols // 16)))
    vals = vals * np.repeat(s, 16, axis=1)
    return vals * float(np.float32(gscale))


def decode_expert(stored, dtype: str) -> np.ndarray:
    """Any stored weight -> float64."""
    if dtype == "nvfp4":
        codes, scales, g = stored
        return decode_nvfp4(codes, scales, g)
    if dtype == "fp8":                      # (E4M3 codes, per-matrix fp32 scale)
        codes, sc = stored
        return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)] * float(np.float32(sc))
    if dtype == "bf16":
        return bf16_to_f64(stored)
    if dtype == "f32":
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    if dtype == "f64":                      # exact test tensors (pins only)
        return np.asarray(stored, dtype=np.float64)
    raise ValueError(dtype)


def _act(a, dtype: str) -> np.ndarray:
    return decode_expert(a, dtype)


# ----------------------------------------------------------------- method steps
def sqrelu(h: np.ndarray) -> np.ndarray:
    """Squared ReLU, max(h, 0)^2: the expert nonlinearity."""
    r = np.maximum(h, 0.0)
    return r * r


def latent_down(x64: np.ndarray, wd64: Optional[np.ndarray]) -> np.ndarray:
    """z = W_d x for every token ([KO 2.2]: project d -> l before routing)."""
    if wd64 is None:
        return x64
    return x64 @ wd64.T


def router_logits(z: np.ndarray, wr: np.ndarray, br: Optional[np.ndarray]) -> np.ndarray:
    """logits[t][e] = sum_i W_r[e][i] z[t][i] + b_r[e]: a linear router on its
    input z (the latent, or x at d when the layer routes on x)."""
    lg = z @ np.asarray(wr, dtype=np.float64).T
    if br is not None:
        lg = lg + np.asarray(br, dtype=np.float64)[None, :]
    return lg


def select_top_k(logits: np.ndarray, k: int) -> np.ndarray:
    """Indices of the K largest logits per row, ordered by descending logit,
    equal logits ordered by ascending expert id (brute force: a full stable sort)."""
    order = np.argsort(-logits, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def gates_softmax(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """g[t][k] = exp(l_sel_k - l_max) / sum_j exp(l_sel_j - l_max) over the K selected."""
    sel = np.take_along_axis(logits, idx.astype(np.int64), axis=1)
    w = np.exp(sel - sel.max(axis=1, keepdims=True))
    return w / w.sum(axis=1, keepdims=True)


def expert_ffn(z_rows: np.ndarray, w1: np.ndarray, w2: np.ndarray, h_scale=None) -> np.ndarray:
    """W2 sqrelu(W1 z) for each row z (W1 [m][l], W2 [l][m], float64).  With
    h_scale (FP8 layers) the hidden rows enter W2 as their FP8 values q(h)."""
    h = sqrelu(z_rows @ w1.T)
    if h_scale is not None:
        h = e4m3_qdq(h, h_scale)
    return h @ w2.T


@dataclasses.dataclass
class OracleResult:
    y: Optional[np.ndarray]       # [len(tokens)][d] float64 (None if route_only)
    tokens: np.ndarray            # token ids y rows belong to
    logits: np.ndarray            # [T][N] float64
    idx: np.ndarray               # [T][K] int32, descending logit
    gate: np.ndarray              # [T][K] float64
    counts: np.ndarray            # [N] int64
    gap: np.ndarray               # [T] l_(K) - l_(K+1) (inf if K == N)
    z: np.ndarray                 # [T][l] float64 latent


def route(layer, cfg) -> OracleResult:
    """Steps 1-4 for every token plus the per-expert counts."""
    x64 = _act(layer.x(), cfg.act)
    wd = layer.w_down()
    z = latent_down(x64, None if wd is None else _act(wd, cfg.act))
    # [KO 2.2] places the router at d (on x); the latent variant routes on z
    logits = router_logits(x64 if cfg.router_on_x else z,
                           layer.w_router(), layer.b_router())
    K = cfg.top_k
    idx = select_top_k(logits, K)
    gate = gates_softmax(logits, idx)
    counts = np.bincount(idx.ravel(), minlength=cfg.n_experts).astype(np.int64)
    if K < cfg.n_experts:
        srt = -np.sort(-logits, axis=1)
        gap = srt[:, K - 1] - srt[:, K]
    else:
        gap = np.full(logits.shape[0], np.inf)
    return OracleResult(None, np.arange(logits.shape[0]), logits, idx, gate, counts, gap, z)


def forward(layer, cfg, tokens: Optional[Sequence[int]] = None) -> OracleResult:
    """The whole layer: routing over all T tokens, y for ``tokens`` (default all).

    ``layer`` supplies stored tensors through x(), w_down(), w_router(),
    b_router(), w1(e), w2(e), w_up(), ws1(), ws2().  Each expert's weights are
    decoded to float64 one expert at a time.
    """
    r = route(layer, cfg)
    T = r.idx.shape[0]
    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    u = np.zeros((len(tok), cfg.latent), dtype=np.float64)
    idx_sub = r.idx[tok]
    gate_sub = r.gate[tok]
    zin, h_scale = r.z[tok], None
    if cfg.expert == "fp8":                          # FP8 expert inputs
        a_z, h_scale = layer.act_scales()
        zin = e4m3_qdq(zin, a_z)
    for e in np.unique(idx_sub):
        rows, ks = np.nonzero(idx_sub == e)          # each token picks e at most once
        w1 = decode_expert(layer.w1(int(e)), cfg.expert)
        w2 = decode_expert(layer.w2(int(e)), cfg.expert)
        out = expert_ffn(zin[rows], w1, w2, h_scale)
        u[rows] += gate_sub[rows, ks][:, None] * out
    wu = layer.w_up()
    y = u if wu is None else u @ _act(wu, cfg.act).T
    if cfg.n_shared:
        x64 = _act(layer.x(), cfg.act)[tok]
        sdt = "fp8" if cfg.shared_fp8 else cfg.act
        ws1 = decode_expert(layer.ws1(), sdt)
        ws2 = decode_expert(layer.ws2(), sdt)
        hs_scale = None
        if cfg.shared_fp8:
            a_x, hs_scale = layer.shared_act_scales()
            x64 = e4m3_qdq(x64, a_x)
        for s in range(cfg.n_shared):
            y = y + expert_ffn(x64, ws1[s], ws2[s], hs_scale)
    r.y = y
    r.tokens = tok
    return r


def forward_scalar(layer, cfg) -> OracleResult:
    """The same layer in pure-Python loops (no BLAS, no numpy sort) for tiny shapes.

    Used to cross-check ``forward``'s vectorised gather/scatter bookkeeping.
    """
    X = _act(layer.x(), cfg.act).tolist()
    wd = layer.w_down()
    Wd = None if wd is None else _act(wd, cfg.act).tolist()
    Wr = np.asarray(layer.w_router(), dtype=np.float64).tolist()
    br = layer.b_router()
    Br = [0.0] * cfg.n_experts if br is None else np.asarray(br, dtype=np.float64).tolist()
    wu = layer.w_up()
    Wu = None if wu is None else _act(wu, cfg.act).tolist()
    W1 = [decode_expert(layer.w1(e), cfg.expert).tolist() for e in range(cfg.n_experts)]
    W2 = [decode_expert(layer.w2(e), cfg.expert).tolist() for e in range(cfg.n_experts)]
    T, K, N, L, M = len(X), cfg.top_k, cfg.n_experts, cfg.latent, cfg.ffn
    fp8 = cfg.expert == "fp8"
    a_z, a_h = layer.act_scales() if fp8 else (None, None)

    def q(vec, a):                           # an FP8 GEMM input's value (identity if a is None)
        return vec if a is None else [float(v) for v in e4m3_qdq(np.array(vec), a)]

    def matvec(W, v):
        return [math.fsum(wi * vi for wi, vi in zip(row, v)) for row in W]

    ys, idxs, gates, lgs, zs = [], [], [], [], []
    for t in range(T):
        z = X[t] if Wd is None else matvec(Wd, X[t])
        lg = [a + b for a, b in zip(matvec(Wr, X[t] if cfg.router_on_x else z), Br)]
        chosen = []
        for _ in range(K):                   # repeated selection of the best remaining
            best = None
            for e in range(N):
                if e in chosen:
                    continue
                if best is None or lg[e] > lg[best]:
                    best = e
            chosen.append(best)
        mx = lg[chosen[0]]
        ex = [math.exp(lg[e] - mx) for e in chosen]
        s = math.fsum(ex)
        g = [v / s for v in ex]
        u = [0.0] * L
        zq = q(z, a_z)
        for k, e in enumerate(chosen):
            h = q([max(v, 0.0) ** 2 for v in matvec(W1[e], zq)], a_h)
            o = matvec(W2[e], h)
            u = [ui + g[k] * oi for ui, oi in zip(u, o)]
        y = u if Wu is None else matvec(Wu, u)
        if cfg.n_shared:
            sdt = "fp8" if cfg.shared_fp8 else cfg.act
            S1 = decode_expert(layer.ws1(), sdt).tolist()
            S2 = decode_expert(layer.ws2(), sdt).tolist()
            a_x, a_s = layer.shared_act_scales() if cfg.shared_fp8 else (None, None)
            xq = q(X[t], a_x)
            for sidx in range(cfg.n_shared):
                h = q([max(v, 0.0) ** 2 for v in matvec(S1[sidx], xq)], a_s)
                o = matvec(S2[sidx], h)
                y = [a + b for a, b in zip(y, o)]
        ys.append(y)
        idxs.append(chosen)
        gates.append(g)
        lgs.append(lg)
        zs.append(z)
    idx = np.array(idxs, dtype=np.int32)
    counts = np.bincount(idx.ravel(), minlength=N).astype(np.int64)
    return OracleResult(np.array(ys), np.arange(T), np.array(lgs), idx, np.array(gates),
                        counts, np.full(T, np.nan), np.array(zs))
