"""Pins of the fp64 oracle against values and facts fixed outside it.

Each test names what it pins: a hand-worked golden example, a format table, a
library routine on a special case, a closed form or an invariance.  A plausible
mistake in the oracle (dropped term, wrong sign or index, transposed operand,
wrong nonlinearity, wrong tie rule, wrong nibble order) fails at least one.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from helpers import GOLDEN, ArrayLayer, f64_layer, load_golden
from sparse_moe_layer_fwd_amd.workloads import CONFIGS, MoEConfig

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------- formats
def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b = line.split()
            rows.append((int(a, 0), float(b)))
    return rows


def test_e2m1_table_matches_golden():
    for code, val in _read_table("e2m1_values.txt"):
        got = oracle.E2M1_TABLE[code]
        assert got == val and math.copysign(1, got) == math.copysign(1, val), code


def test_e4m3_golden_points():
    for byte, val in _read_table("e4m3_points.txt"):
        got = oracle.E4M3_TABLE[byte]
        if math.isnan(val):
            assert math.isnan(got), hex(byte)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(byte)


def test_e4m3_all_codes_match_torch():
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.E4M3_TABLE
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(1)
    u = rng.integers(0, 1 << 16, size=100000, dtype=np.uint32).astype(np.uint16)
    u = u[(u & 0x7F80) != 0x7F80]                        # drop Inf/NaN patterns
    ref = torch.from_numpy(u.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.bf16_to_f64(u), ref)


def test_nvfp4_hand_packed_example():
    g = load_golden("nvfp4_hand.json")
    codes = np.array([int(h, 16) for h in g["codes_hex"]], dtype=np.uint8).reshape(g["rows"], -1)
    scales = np.array([int(h, 16) for h in g["scales_hex"]], dtype=np.uint8).reshape(g["rows"], -1)
    w = oracle.decode_nvfp4(codes, scales, np.float32(g["gscale"]))
    exp = np.array(g["expected"], dtype=np.float64).reshape(g["rows"], g["cols"])
    assert np.array_equal(w, exp)
    assert np.array_equal(np.signbit(w), np.signbit(exp))


def test_nvfp4_products_are_bf16_exact():
    """Every finite e2m1 * e4m3 product is a bf16 value (so dequantising to bf16 loses
    nothing before the fp32 global scale).  Checked with torch's bf16 rounding."""
    prod = np.outer(oracle.E2M1_TABLE, oracle.E4M3_TABLE).ravel()
    prod = prod[np.isfinite(prod)]
    rt = torch.from_numpy(prod).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(rt, prod)


# ---------------------------------------------------------------- routing
def _brute_top_k(row, k):
    chosen = []
    for _ in range(k):
        best = None
        for e, v in enumerate(row):
            if e in chosen:
                continue
            if best is None or v > row[best]:
                best = e
        chosen.append(best)
    return chosen


def test_top_k_brute_force_with_ties():
    rng = np.random.default_rng(2)
    lg = rng.integers(-3, 4, size=(200, 12)).astype(np.float64)   # many exact ties
    for k in (1, 3, 5, 12):
        idx = oracle.select_top_k(lg, k)
        for t in range(lg.shape[0]):
            assert list(idx[t]) == _brute_top_k(list(lg[t]), k)
            sel = lg[t, idx[t]]
            rest = np.delete(lg[t], idx[t])
            if rest.size:
                assert sel.min() >= rest.max()


def test_top_k_engineered_tie_prefers_lower_id():
    lg = np.array([[1.0, 5.0, 5.0, 0.0, 5.0]])
    assert list(oracle.select_top_k(lg, 2)[0]) == [1, 2]
    assert list(oracle.select_top_k(lg, 3)[0]) == [1, 2, 4]


def test_top_k_matches_torch_topk_without_ties():
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((500, 64))
    idx = oracle.select_top_k(lg, 7)
    ref = torch.topk(torch.from_numpy(lg), 7, dim=1, largest=True, sorted=True).indices.numpy()
    assert np.array_equal(idx, ref)


def test_gates_closed_forms():
    rng = np.random.default_rng(4)
    lg = rng.standard_normal((300, 16)) * 3
    for k in (1, 4, 16):
        idx = oracle.select_top_k(lg, k)
        g = oracle.gates_softmax(lg, idx)
        assert np.allclose(g.sum(axis=1), 1.0, atol=1e-15, rtol=0)
        assert np.all(np.diff(g, axis=1) <= 0)         # descending logit -> descending gate
        if k == 1:
            assert np.all(g == 1.0)
        if k == 16:                                   # K = N: the full softmax
            full = torch.softmax(torch.from_numpy(lg), dim=1).numpy()
            assert np.allclose(np.take_along_axis(full, idx.astype(np.int64), 1), g,
                               atol=1e-15, rtol=1e-13)


# ---------------------------------------------------------------- hand examples
def test_hand_worked_latent_example():
    g = load_golden("tiny_hand.json")
    cfg = MoEConfig("hand", T=1, d=g["d"], latent=g["latent"], n_experts=g["n_experts"],
                    top_k=g["top_k"], ffn=g["ffn"], act="f64", expert="f64")
    arr = lambda k: np.array(g[k], dtype=np.float64)
    layer = ArrayLayer(cfg, arr("x"), arr("w_router"), arr("w1"), arr("w2"), arr("w_down"),
                       arr("w_up"), arr("b_router"))
    for fwd in (oracle.forward, oracle.forward_scalar):
        r = fwd(layer, cfg)
        assert np.array_equal(r.idx, np.array(g["expected_idx"]))
        assert np.allclose(r.gate, arr("expected_gate"), rtol=0, atol=1e-15)
        assert np.allclose(r.logits, arr("expected_logits"), rtol=0, atol=0)
        assert np.allclose(r.y, arr("expected_y"), rtol=1e-15, atol=1e-14)
    r = oracle.forward(layer, cfg)
    assert np.array_equal(r.z, arr("expected_z"))
    assert np.array_equal(r.gap, arr("expected_gap"))
    assert list(r.counts) == [0, 1, 1]


def test_hand_worked_standard_moe_with_shared_expert():
    g = load_golden("std_shared_hand.json")
    cfg = MoEConfig("hand_std", T=1, d=g["d"], latent=g["latent"], n_experts=g["n_experts"],
                    top_k=g["top_k"], ffn=g["ffn"], n_shared=g["n_shared"],
                    shared_ffn=g["shared_ffn"], has_latent_proj=False, act="f64", expert="f64")
    arr = lambda k: np.array(g[k], dtype=np.float64)
    layer = ArrayLayer(cfg, arr("x"), arr("w_router"), arr("w1"), arr("w2"),
                       ws1=arr("ws1"), ws2=arr("ws2"))
    for fwd in (oracle.forward, oracle.forward_scalar):
        r = fwd(layer, cfg)
        assert np.array_equal(r.idx, np.array(g["expected_idx"]))
        assert np.array_equal(r.gate, arr("expected_gate"))
        assert np.array_equal(r.y, arr("expected_y"))


# ---------------------------------------------------------------- reductions / invariances
SMALL = MoEConfig("small", T=40, d=24, latent=8, n_experts=6, top_k=3, ffn=10,
                  act="f64", expert="f64")


def _textbook_moe_torch(layer, cfg):
    """Classic sparsely-gated top-K MoE computed densely in torch fp64: run every
    expert on every token, then mask with torch.topk and torch.softmax."""
    x = torch.from_numpy(np.asarray(layer.x(), dtype=np.float64))
    wr = torch.from_numpy(np.asarray(layer.w_router(), dtype=np.float64))
    lg = x @ wr.T
    top = torch.topk(lg, cfg.top_k, dim=1)
    g = torch.softmax(top.values, dim=1)
    y = torch.zeros_like(x)
    for e in range(cfg.n_experts):
        w1 = torch.from_numpy(np.asarray(layer.w1(e)))
        w2 = torch.from_numpy(np.asarray(layer.w2(e)))
        out = torch.nn.functional.linear(torch.relu(torch.nn.functional.linear(x, w1)) ** 2, w2)
        ge = (g * (top.indices == e)).sum(dim=1, keepdim=True)
        y = y + ge * out
    return y.numpy(), top.indices.numpy()


def test_identity_projections_reduce_to_standard_moe():
    rng = np.random.default_rng(5)
    std = MoEConfig("std", T=50, d=12, latent=12, n_experts=7, top_k=2, ffn=9,
                    has_latent_proj=False)
    c_std, lstd = f64_layer(std, rng)
    c_lat = c_std.replace(has_latent_proj=True)
    eye = np.eye(12)
    llat = ArrayLayer(c_lat, lstd.x(), lstd.w_router(), lstd._w1, lstd._w2, eye, eye)
    a = oracle.forward(lstd, c_std)
    b = oracle.forward(llat, c_lat)
    assert np.array_equal(a.idx, b.idx)
    assert np.allclose(a.y, b.y, rtol=1e-13, atol=1e-13)
    y_t, idx_t = _textbook_moe_torch(lstd, c_std)
    assert np.array_equal(a.idx, idx_t)
    assert np.allclose(a.y, y_t, rtol=1e-12, atol=1e-12)


def test_single_expert_is_a_dense_squared_relu_mlp():
    rng = np.random.default_rng(6)
    cfg = MoEConfig("dense", T=30, d=16, latent=8, n_experts=1, top_k=1, ffn=12)
    c, layer = f64_layer(cfg, rng)
    r = oracle.forward(layer, c)
    F = torch.nn.functional
    x = torch.from_numpy(layer.x())
    z = F.linear(x, torch.from_numpy(layer.w_down()))
    h = F.relu(F.linear(z, torch.from_numpy(layer.w1(0)))).pow(2)
    y = F.linear(F.linear(h, torch.from_numpy(layer.w2(0))), torch.from_numpy(layer.w_up()))
    assert np.allclose(r.y, y.numpy(), rtol=1e-12, atol=1e-12)


def test_homogeneity_degree_two():
    """K = 1, no router bias: the gate is 1 and routing is scale-invariant, so
    y(2x) = 4 y(x) exactly (squared ReLU is homogeneous of degree 2)."""
    rng = np.random.default_rng(7)
    c, layer = f64_layer(SMALL.replace(top_k=1), rng)
    r1 = oracle.forward(layer, c)
    layer._x = 2.0 * layer._x
    r2 = oracle.forward(layer, c)
    assert np.array_equal(r1.idx, r2.idx)
    assert np.array_equal(r2.y, 4.0 * r1.y)


def test_orthogonal_latent_rotation_invariance():
    """Rotating the latent basis by an orthogonal Q (W_d -> Q W_d, W_r -> W_r Q^T,
    W1 -> W1 Q^T, W2 -> Q W2, W_u -> W_u Q^T) leaves y unchanged; a transposed
    operand anywhere breaks it for a non-symmetric Q."""
    rng = np.random.default_rng(8)
    c, layer = f64_layer(SMALL, rng)
    q, _ = np.linalg.qr(rng.standard_normal((c.latent, c.latent)))
    assert not np.allclose(q, q.T)
    rot = ArrayLayer(c, layer.x(), layer.w_router() @ q.T,
                     np.einsum("eml,kl->emk", layer._w1, q), np.einsum("kl,elm->ekm", q, layer._w2),
                     q @ layer.w_down(), layer.w_up() @ q.T)
    a = oracle.forward(layer, c)
    b = oracle.forward(rot, c)
    assert np.array_equal(a.idx, b.idx)
    assert np.allclose(a.y, b.y, rtol=1e-11, atol=1e-11)


def test_expert_relabel_invariance():
    rng = np.random.default_rng(9)
    c, layer = f64_layer(SMALL, rng)
    br = rng.standard_normal(c.n_experts)
    layer._br = br
    p = rng.permutation(c.n_experts)          # new expert j is old expert p[j]
    rel = ArrayLayer(c, layer.x(), layer.w_router()[p], layer._w1[p], layer._w2[p],
                     layer.w_down(), layer.w_up(), br[p])
    a = oracle.forward(layer, c)
    b = oracle.forward(rel, c)
    assert np.array_equal(p[b.idx], a.idx)
    assert np.array_equal(a.gate, b.gate)
    assert np.allclose(a.y, b.y, rtol=1e-13, atol=1e-13)


def test_two_shared_experts_equal_one_of_double_width():
    rng = np.random.default_rng(10)
    cfg = MoEConfig("sh", T=20, d=10, latent=10, n_experts=4, top_k=2, ffn=6, n_shared=2,
                    shared_ffn=5, has_latent_proj=False)
    c, layer = f64_layer(cfg, rng)
    a = oracle.forward(layer, c)
    ws1 = np.concatenate([layer._ws1[0], layer._ws1[1]], axis=0)[None]
    ws2 = np.concatenate([layer._ws2[0], layer._ws2[1]], axis=1)[None]
    c1 = c.replace(n_shared=1, shared_ffn=10)
    one = ArrayLayer(c1, layer.x(), layer.w_router(), layer._w1, layer._w2, ws1=ws1, ws2=ws2)
    b = oracle.forward(one, c1)
    assert np.allclose(a.y, b.y, rtol=1e-13, atol=1e-13)


def test_router_bias_forces_an_expert():
    rng = np.random.default_rng(11)
    c, layer = f64_layer(SMALL, rng)
    br = np.zeros(c.n_experts)
    br[4] = 1e6
    layer._br = br
    r = oracle.forward(layer, c)
    assert np.all(r.idx[:, 0] == 4)
    assert r.counts[4] == c.T


def test_vectorised_matches_scalar_loops():
    rng = np.random.default_rng(12)
    c, layer = f64_layer(SMALL, rng)
    layer._br = rng.standard_normal(c.n_experts)
    a = oracle.forward(layer, c)
    b = oracle.forward_scalar(layer, c)
    assert np.array_equal(a.idx, b.idx)
    assert np.array_equal(a.counts, b.counts)
    assert np.allclose(a.gate, b.gate, rtol=1e-14, atol=1e-15)
    assert np.allclose(a.y, b.y, rtol=1e-12, atol=1e-12)


def test_router_on_x_equals_latent_router_through_inverse_projection():
    """Routing on x with W_r equals routing on z = W_d x with W_r W_d^-1 (l = d,
    W_d invertible and not symmetric): the router must read x, untransposed."""
    rng = np.random.default_rng(21)
    cfg = MoEConfig("rx", T=40, d=12, latent=12, n_experts=8, top_k=3, ffn=10, n_shared=1,
                    shared_ffn=6, router_on_x=True)
    c, layer = f64_layer(cfg, rng)
    wd = layer.w_down() + 0.5 * np.eye(12)
    assert not np.allclose(wd, wd.T)
    layer._wd = wd
    c_lat = c.replace(router_on_x=False)
    lat = ArrayLayer(c_lat, layer.x(), layer.w_router() @ np.linalg.inv(wd), layer._w1,
                     layer._w2, wd, layer.w_up(), None, layer._ws1, layer._ws2)
    a = oracle.forward(layer, c)
    b = oracle.forward(lat, c_lat)
    assert np.allclose(a.logits, b.logits, rtol=1e-11, atol=1e-11)
    assert np.array_equal(a.idx, b.idx)
    assert np.allclose(a.y, b.y, rtol=1e-11, atol=1e-11)
    # and the same layer routed on z instead picks different experts
    wrong = oracle.forward(ArrayLayer(c_lat, layer.x(), layer.w_router(), layer._w1, layer._w2,
                                      wd, layer.w_up(), None, layer._ws1, layer._ws2), c_lat)
    assert not np.array_equal(wrong.idx, a.idx)


def test_router_on_x_vectorised_matches_scalar_loops():
    rng = np.random.default_rng(22)
    cfg = MoEConfig("rx", T=24, d=16, latent=8, n_experts=6, top_k=2, ffn=10, n_shared=1,
                    shared_ffn=12, router_on_x=True)
    c, layer = f64_layer(cfg, rng)
    layer._br = rng.standard_normal(c.n_experts)
    a = oracle.forward(layer, c)
    b = oracle.forward_scalar(layer, c)
    assert np.array_equal(a.idx, b.idx)
    assert np.allclose(a.gate, b.gate, rtol=1e-14, atol=1e-15)
    assert np.allclose(a.y, b.y, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- FP8 (E4M3)
def _read_quant_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            v, sc, code = line.split()[:3]
            rows.append((float(v), float(sc), int(code, 16)))
    return rows


def test_e4m3_quantize_hand_worked_cases():
    rows = _read_quant_table("e4m3_quantize.txt")
    assert len(rows) >= 15
    for v, sc, code in rows:
        assert int(oracle.e4m3_quantize(np.array([v]), sc)[0]) == code, (v, sc)


def test_e4m3_quantize_matches_torch_float8_rounding():
    """torch's own fp32 -> float8_e4m3fn conversion (round to nearest even) on
    in-range values of every magnitude, with a non-power-of-two scale."""
    rng = np.random.default_rng(31)
    v = (rng.standard_normal(200000) * np.exp(rng.uniform(-14, 7, 200000))).astype(np.float32)
    for sc in (1.0, 0.0133928571, 3.0):
        r = np.float32(1.0) / np.float32(sc)
        t = np.clip(v * r, -448, 448).astype(np.float32)
        ref = torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(oracle.e4m3_quantize(v, sc), ref), sc


def test_e4m3_quantize_round_trips_every_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(oracle.e4m3_quantize(oracle.E4M3_TABLE[codes], 1.0), codes)
    # and quantise-dequantise is idempotent
    x = np.random.default_rng(32).standard_normal(5000) * 3
    once = oracle.e4m3_qdq(x, 0.02)
    assert np.array_equal(oracle.e4m3_qdq(once, 0.02), once)


def test_fp8_weight_decode_matches_torch_float8():
    from sparse_moe_layer_fwd_amd.workloads import Workload
    cfg = MoEConfig("f8", T=8, d=64, latent=32, n_experts=3, top_k=1, ffn=48, expert="fp8")
    codes, sc = Workload(cfg, seed=2).w1(1)
    assert codes.dtype == np.uint8 and codes.shape == (48, 32)
    assert not np.any((codes & 0x7F) == 0x7F)                 # no NaN codes drawn
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy() * float(sc)
    assert np.array_equal(oracle.decode_expert((codes, sc), "fp8"), ref)


def _fp8_layer_torch(wl, cfg):
    """The FP8 layer written independently in torch: float8_e4m3fn casts for
    every weight decode and activation quantisation, torch.topk routing."""
    f64 = torch.float64

    def dec(codes, sc):
        return torch.from_numpy(np.asarray(codes)).view(torch.float8_e4m3fn).to(f64) * float(np.float32(sc))

    def qdq(v, sc):
        r = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(sc, dtype=torch.float32)
        t = (v.to(torch.float32) * r).clamp(-448, 448)
        return t.to(torch.float8_e4m3fn).to(f64) * float(np.float32(sc))

    F = torch.nn.functional
    x = torch.from_numpy(oracle.bf16_to_f64(wl.x()))
    z = F.linear(x, torch.from_numpy(oracle.bf16_to_f64(wl.w_down())))
    logits = F.linear(x if cfg.router_on_x else z, torch.from_numpy(wl.w_router().astype(np.float64)))
    top = torch.topk(logits, cfg.top_k, dim=1)
    g = torch.softmax(top.values, dim=1)
    a_z, a_h = wl.act_scales()
    zq = qdq(z, a_z)
    u = torch.zeros_like(z)
    for e in range(cfg.n_experts):
        h = F.relu(F.linear(zq, dec(*wl.w1(e)))) ** 2
        out = F.linear(qdq(h, a_h), dec(*wl.w2(e)))
        u = u + (g * (top.indices == e)).sum(dim=1, keepdim=True) * out
    y = F.linear(u, torch.from_numpy(oracle.bf16_to_f64(wl.w_up())))
    if cfg.n_shared:
        c1, s1 = wl.ws1()
        c2, s2 = wl.ws2()
        a_x, a_s = wl.shared_act_scales()
        xq = qdq(x, a_x)
        for s in range(cfg.n_shared):
            h = F.relu(F.linear(xq, dec(c1[s], s1))) ** 2
            y = y + F.linear(qdq(h, a_s), dec(c2[s], s2))
    return y.numpy(), top.indices.numpy()


@pytest.mark.parametrize("router_on_x", [False, True])
def test_fp8_layer_matches_independent_torch_layer(router_on_x):
    from sparse_moe_layer_fwd_amd.workloads import Workload
    cfg = MoEConfig("f8", T=40, d=64, latent=32, n_experts=6, top_k=2, ffn=48, expert="fp8",
                    n_shared=2, shared_ffn=16, shared_fp8=True, router_on_x=router_on_x)
    wl = Workload(cfg, seed=4)
    r = oracle.forward(wl, cfg)
    y_t, idx_t = _fp8_layer_torch(wl, cfg)
    assert np.array_equal(np.sort(r.idx, axis=1), np.sort(idx_t, axis=1))
    assert np.allclose(r.y, y_t, rtol=1e-12, atol=1e-12)


def test_fp8_vectorised_matches_scalar_loops():
    from sparse_moe_layer_fwd_amd.workloads import Workload
    cfg = MoEConfig("f8", T=12, d=32, latent=16, n_experts=5, top_k=2, ffn=24, expert="fp8",
                    n_shared=1, shared_ffn=16, shared_fp8=True)
    wl = Workload(cfg, seed=5)
    a = oracle.forward(wl, cfg)
    b = oracle.forward_scalar(wl, cfg)
    assert np.array_equal(a.idx, b.idx)
    assert np.allclose(a.y, b.y, rtol=1e-12, atol=1e-12)


def test_token_subset_equals_full_rows():
    rng = np.random.default_rng(13)
    c, layer = f64_layer(SMALL, rng)
    full = oracle.forward(layer, c)
    sub = oracle.forward(layer, c, tokens=[3, 17, 0, 39])
    assert np.allclose(sub.y, full.y[[3, 17, 0, 39]], rtol=1e-14, atol=1e-14)


def test_counts_and_config1_routing_invariants():
    from sparse_moe_layer_fwd_amd.workloads import Workload
    from helpers import margin_filter
    cfg = CONFIGS[1]
    wl = Workload(cfg, seed=0)
    margin_filter(wl, cfg)
    r = oracle.route(wl, cfg)
    assert r.counts.sum() == cfg.T * cfg.top_k
    assert np.all(r.gap >= cfg.margin)
    assert np.allclose(r.gate.sum(axis=1), 1.0, atol=1e-14)
    for t in range(cfg.T):
        assert len(set(r.idx[t].tolist())) == cfg.top_k


def test_config1_vectorised_matches_scalar():
    from sparse_moe_layer_fwd_amd.workloads import Workload
    cfg = CONFIGS[1].replace(T=6)
    wl = Workload(cfg, seed=0)
    a = oracle.forward(wl, cfg)
    b = oracle.forward_scalar(wl, cfg)
    assert np.array_equal(a.idx, b.idx)
    assert np.allclose(a.y, b.y, rtol=1e-12, atol=1e-12)


def test_nvfp4_forward_equals_decoded_dense_forward():
    """An NVFP4 layer is the same layer with its weights decoded to fp64."""
    from sparse_moe_layer_fwd_amd.workloads import Workload
    cfg = MoEConfig("fp4", T=16, d=64, latent=32, n_experts=4, top_k=2, ffn=48, expert="nvfp4")
    wl = Workload(cfg, seed=3)
    a = oracle.forward(wl, cfg)
    dense = ArrayLayer(cfg.replace(act="bf16", expert="f64"), wl.x(), wl.w_router(),
                       [oracle.decode_expert(wl.w1(e), "nvfp4") for e in range(4)],
                       [oracle.decode_expert(wl.w2(e), "nvfp4") for e in range(4)],
                       wl.w_down(), wl.w_up())
    b = oracle.forward(dense, dense.cfg)
    assert np.array_equal(a.y, b.y)
