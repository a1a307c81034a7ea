"""GPU parity: the HIP library against the CPU oracle, through the C ABI.

Small shapes are compared element by element (all tokens, all rows); they span several tiles
of every kernel and end on ragged tails. Full workload sizes are checked on sampled tokens
(every routed row of each sampled token, the shared row, the combined output) plus properties
that hold at any size. Routing integers are compared bit-exactly from the same fp32 logits.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sparse_moe_layer_softmax_amd as moe
from sparse_moe_layer_softmax_amd.workloads import WORKLOADS, Workload, as_u16, capacity_for, from_u16, generate
from tests import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


BASE = WORKLOADS["tiny_t128_h512_e32_k2"]
SMALL = {
    "tiny_t128_h512_e32_k2": BASE,
    "ragged_t130_h256_e256_k8": Workload("ragged_t130_h256_e256_k8", T=130, H=256, E=256, K=8, I=256,
                                         scale=2.827, w_std=0.02, router_std=0.02, seed=11),
    "single_token_t1_e256_k8": Workload("single_token_t1_e256_k8", T=1, H=256, E=256, K=8, I=512,
                                        scale=2.827, w_std=0.02, router_std=0.02, seed=12),
    "t3_e64_k6": Workload("t3_e64_k6", T=3, H=512, E=64, K=6, I=256, scale=2.827, seed=13),
    "dense_e1_k1_t100": Workload("dense_e1_k1_t100", T=100, H=512, E=1, K=1, I=256, n_shared=0,
                                 seed=14),
    "no_shared_t128": BASE.with_(name="no_shared_t128", n_shared=0, seed=15),
    "no_renorm_t128": BASE.with_(name="no_renorm_t128", norm_topk=False, scale=2.827, seed=16),
    "capacity_drops_t200_e8_k2": Workload("capacity_drops_t200_e8_k2", T=200, H=256, E=8, K=2, I=256,
                                          capacity=30, zipf=0.3, seed=17),
    "capacity_t256_h512_e32_k2": Workload("capacity_t256_h512_e32_k2", T=256, H=512, E=32, K=2, I=512,
                                          limit=0.0, capacity=capacity_for(256, 2, 32),
                                          w_std=0.006, router_std=0.006, seed=18),
    "clamp_forced_t128": BASE.with_(name="clamp_forced_t128", x_std=30.0, seed=19),
    "multi_tile_t300_e16_k4": Workload("multi_tile_t300_e16_k4", T=300, H=512, E=16, K=4, I=256,
                                       scale=2.827, seed=20),
    # several 8-tile bands in one group (about 1500 rows per expert), ragged last tiles
    "bands_t3000_e4_k2": Workload("bands_t3000_e4_k2", T=3000, H=256, E=4, K=2, I=256, scale=2.827,
                                  seed=22),
    # a few hundred rows per expert on the tiled kernel: one and two row tiles per expert (skewed
    # router), partly filled tiles
    "midsize_t1000_h512_e16_k4": Workload("midsize_t1000_h512_e16_k4", T=1000, H=512, E=16, K=4, I=256,
                                         scale=2.827, zipf=0.4, seed=26),
    "midsize_t640_h256_e32_k8": Workload("midsize_t640_h256_e32_k8", T=640, H=256, E=32, K=8, I=512,
                                        scale=2.827, seed=27),
    # a dense SwiGLU FFN (E = 1, k = 1, no shared expert) with a wide intermediate on the tiled path
    "dense_ffn_t700_h512_i2304": Workload("dense_ffn_t700_h512_i2304", T=700, H=512, E=1, K=1,
                                          I=2304, n_shared=0, seed=25),
    # router on the tiled MFMA path (T >= 1024, E = 256), ragged T
    "tiled_router_t1030_e256_k8": Workload("tiled_router_t1030_e256_k8", T=1030, H=256, E=256, K=8,
                                           I=256, scale=2.827, seed=23),
}

# FP8 expert weights (E4M3 codes, per-row fp32 scales); every FFN shape runs the weight-streaming
# kernel, so these span one and many 64-row tiles per group, ragged tails and the clamp
SMALL.update({
    "fp8_tiny_t128_h512_e32_k2": BASE.with_(name="fp8_tiny_t128_h512_e32_k2", fp8=True, seed=40),
    "fp8_ragged_t130_h256_e256_k8": SMALL["ragged_t130_h256_e256_k8"].with_(
        name="fp8_ragged_t130_h256_e256_k8", fp8=True, seed=41),
    "fp8_no_shared_t128": BASE.with_(name="fp8_no_shared_t128", n_shared=0, fp8=True, seed=42),
    "fp8_multi_tile_t300_e16_k4": SMALL["multi_tile_t300_e16_k4"].with_(
        name="fp8_multi_tile_t300_e16_k4", fp8=True, seed=43),
    "fp8_bands_t3000_e4_k2": SMALL["bands_t3000_e4_k2"].with_(name="fp8_bands_t3000_e4_k2",
                                                              fp8=True, seed=44),
    "fp8_clamp_forced_t128": BASE.with_(name="fp8_clamp_forced_t128", x_std=30.0, fp8=True, seed=45),
    "fp8_capacity_drops_t200_e8_k2": SMALL["capacity_drops_t200_e8_k2"].with_(
        name="fp8_capacity_drops_t200_e8_k2", fp8=True, seed=46),
})

# routing only: the tiled router with its hidden dimension split 12 ways (2 K-tiles per split)
ROUTE_ONLY = {
    "tiled_router_t2000_h1536_e256_k8": Workload("tiled_router_t2000_h1536_e256_k8", T=2000, H=1536,
                                                 E=256, K=8, I=256, scale=2.827, seed=24),
}


# ----------------------------------------------------------------------------- end to end, small
@pytest.mark.parametrize("name", list(SMALL))
def test_layer_forward_small(name):
    _require_gpu()
    wl = SMALL[name]
    dev = generate(wl, DEV)
    hw = P.host(dev)
    g, _, _ = P.run_layer_gpu(wl, dev)
    # logits against the oracle's own projection
    lo = oracle.router_logits(hw["x"], hw["w_router"], hw["router_bias"])
    P.assert_logits_close(g["logits"], lo)
    # same-logits mode: every routing integer bit-exact, every tensor in tolerance
    r = P.oracle_same_logits(wl, hw, g["logits"])
    P.compare_layer(wl, hw, g, r)
    # independent logits: indices agree on every token with a clear k-th / (k+1)-th margin
    idx_i, _, probs = oracle.route_from_logits(lo, wl.K, wl.scale, wl.norm_topk, want_probs=True)
    ok = P.margin_ok(probs, wl.K)
    np.testing.assert_array_equal(g["topk_idx"][ok], idx_i[ok])
    if name.endswith("capacity_drops_t200_e8_k2"):
        assert (g["slot_to_row"] < 0).sum() > 0, "this case must drop slots"
    if name.endswith("clamp_forced_t128"):
        hv = P.f64(g["h_routed"][: int(g["offsets"][-1])])
        assert np.abs(hv).max() > 50, "this case must reach the clamp"


def test_layer_is_deterministic():
    _require_gpu()
    wl = SMALL["ragged_t130_h256_e256_k8"]
    dev = generate(wl, DEV)
    g1, layer, _ = P.run_layer_gpu(wl, dev)
    outs = []
    for _ in range(3):
        outs.append(as_u16(layer.forward(dev["x"])))
    torch.cuda.synchronize()
    for o in outs:
        np.testing.assert_array_equal(o, g1["out"])


def test_exact_logit_ties_go_to_lower_expert():
    _require_gpu()
    wl = SMALL["ragged_t130_h256_e256_k8"].with_(name="ties", seed=21)
    dev = generate(wl, DEV)
    # duplicate router rows: expert 2e+1 gets expert 2e's row, so their logits are bit-equal
    wr = dev["w_router"].clone()
    wr[1::2] = wr[0::2]
    dev["w_router"] = wr
    hw = P.host(dev)
    g, _, _ = P.run_layer_gpu(wl, dev)
    np.testing.assert_array_equal(g["logits"][:, 0::2], g["logits"][:, 1::2])
    r = P.oracle_same_logits(wl, hw, g["logits"])
    P.compare_layer(wl, hw, g, r)
    # each selected odd expert is preceded by its even twin
    for t in range(wl.T):
        sel = list(g["topk_idx"][t])
        for e in sel:
            if e % 2 == 1:
                assert e - 1 in sel and sel.index(e - 1) < sel.index(e)


def test_zero_input():
    _require_gpu()
    wl = SMALL["t3_e64_k6"].with_(name="zero", T=5)
    dev = generate(wl, DEV)
    dev["x"] = torch.zeros_like(dev["x"])
    g, _, _ = P.run_layer_gpu(wl, dev)
    assert np.all(g["topk_idx"] == np.arange(wl.K))
    np.testing.assert_allclose(g["topk_w"], wl.scale / wl.K, rtol=1e-6)
    assert np.all((g["out"] & 0x7FFF) == 0)


# ----------------------------------------------------------------------------- per entry point
def _ws(n):
    return torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)


@pytest.mark.parametrize("name", ["tiny_t128_h512_e32_k2", "ragged_t130_h256_e256_k8", "no_renorm_t128",
                                  "tiled_router_t1030_e256_k8", "tiled_router_t2000_h1536_e256_k8"])
def test_moe_route(name):
    _require_gpu()
    wl = {**SMALL, **ROUTE_ONLY}[name]
    dev = generate(wl, DEV)
    hw = P.host(dev)
    s = moe.Shape.of(wl)
    logits = torch.empty((wl.T, wl.E), dtype=torch.float32, device=DEV)
    w = torch.empty((wl.T, wl.K), dtype=torch.float32, device=DEV)
    idx = torch.empty((wl.T, wl.K), dtype=torch.int32, device=DEV)
    moe.moe_route(s, dev["x"], dev["w_router"], dev["router_bias"], logits, w, idx,
                  _ws(moe.moe_route_workspace_size(s)))
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    P.assert_logits_close(lg, oracle.router_logits(hw["x"], hw["w_router"], hw["router_bias"]))
    ri, rw = oracle.route_from_logits(lg, wl.K, wl.scale, wl.norm_topk)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=0, atol=1e-5 * wl.scale)
    # logits pointer is optional
    w2 = torch.empty_like(w)
    idx2 = torch.empty_like(idx)
    moe.moe_route(s, dev["x"], dev["w_router"], dev["router_bias"], None, w2, idx2,
                  _ws(moe.moe_route_workspace_size(s)))
    torch.cuda.synchronize()
    assert torch.equal(idx2, idx) and torch.equal(w2, w)


# up to 1024 slots one single-wavefront launch does the dispatch, above it three launches; the
# cases cover both forms, their boundary (1024 and 1040 slots) and capacity drops in each
@pytest.mark.parametrize("T,K,E,C", [(128, 2, 32, 0), (130, 8, 256, 0), (1, 8, 256, 0),
                                     (200, 2, 8, 30), (64, 8, 256, 0), (128, 8, 256, 3),
                                     (512, 2, 16, 40), (4096, 2, 32, 320), (65536, 8, 256, 0),
                                     (40000, 8, 256, 1200)])
def test_moe_permute(T, K, E, C):
    _require_gpu()
    rng = np.random.default_rng(T + K + E + C)
    pop = np.exp(-0.08 * np.arange(E))  # skewed popularity, empty experts likely when E is large
    pop /= pop.sum()
    # k distinct experts per token, drawn without replacement by Gumbel-top-k on log popularity
    keys = np.log(pop)[None, :] + rng.gumbel(size=(T, E))
    idx = np.argsort(-keys, axis=1)[:, :K].astype(np.int32)
    s = moe.Shape(T=T, H=256, E=E, K=K, I=256, capacity=C)
    d_idx = torch.from_numpy(idx).to(DEV)
    counts = torch.empty(E, dtype=torch.int32, device=DEV)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    r2s = torch.full((T * K,), 7, dtype=torch.int32, device=DEV)
    s2r = torch.full((T * K,), 7, dtype=torch.int32, device=DEV)
    moe.moe_permute(s, d_idx, counts, offsets, r2s, s2r, _ws(moe.moe_permute_workspace_size(s)))
    torch.cuda.synchronize()
    rc, ro, rr, rs = oracle.dispatch(idx, E, C)
    np.testing.assert_array_equal(counts.cpu().numpy(), rc)
    np.testing.assert_array_equal(offsets.cpu().numpy(), ro)
    np.testing.assert_array_equal(r2s.cpu().numpy(), rr)
    np.testing.assert_array_equal(s2r.cpu().numpy(), rs)
    if C:
        assert rc.max() <= C


def _expert_ffn(s, n_groups, rows_max, x, r2s, offsets, w3, h, y, ws):
    """moe_expert_ffn or moe_expert_ffn_fp8, by the weights' type; w3 = (gate, up, down) as
    device tensors, each a bf16 tensor or a (uint8 codes, fp32 scales) pair."""
    if isinstance(w3[0], tuple):
        (qg, cg), (qu, cu), (qd, cd) = w3
        moe.moe_expert_ffn_fp8(s, n_groups, rows_max, x, r2s, offsets, qg, cg, qu, cu, qd, cd, h, y, ws)
    else:
        moe.moe_expert_ffn(s, n_groups, rows_max, x, r2s, offsets, *w3, h, y, ws)


def _dev_weights(dev, names, lead=False):
    def one(n):
        t = dev[n][None] if lead else dev[n]
        if t.dtype == torch.uint8:
            sc = dev[n + "_scale"]
            return (t, sc[None] if lead else sc)
        return t
    return tuple(one(n) for n in names)


@pytest.mark.parametrize("name", ["tiny_t128_h512_e32_k2", "ragged_t130_h256_e256_k8",
                                  "clamp_forced_t128", "multi_tile_t300_e16_k4", "bands_t3000_e4_k2",
                                  "midsize_t1000_h512_e16_k4", "midsize_t640_h256_e32_k8",
                                  "fp8_tiny_t128_h512_e32_k2", "fp8_ragged_t130_h256_e256_k8",
                                  "fp8_clamp_forced_t128", "fp8_multi_tile_t300_e16_k4",
                                  "fp8_bands_t3000_e4_k2"])
def test_moe_expert_ffn_routed_and_identity(name):
    _require_gpu()
    wl = SMALL[name]
    dev = generate(wl, DEV)
    hw = P.host(dev)
    s = moe.Shape.of(wl)
    lo = oracle.router_logits(hw["x"], hw["w_router"], hw["router_bias"])
    idx, w = oracle.route_from_logits(lo, wl.K, wl.scale, wl.norm_topk)
    counts, offsets, r2s, s2r = oracle.dispatch(idx, wl.E, wl.capacity)
    TK = wl.T * wl.K
    h = torch.empty((TK, wl.I), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((TK, wl.H), dtype=torch.bfloat16, device=DEV)
    _expert_ffn(s, wl.E, TK, dev["x"], torch.from_numpy(r2s).to(DEV),
                torch.from_numpy(offsets).to(DEV), _dev_weights(dev, ("w_gate", "w_up", "w_down")),
                h, y, _ws(moe.moe_expert_ffn_workspace_size(s, wl.E, TK)))
    torch.cuda.synchronize()
    R = int(offsets[-1])
    hg, yg = as_u16(h)[:R], as_u16(y)[:R]
    for e in range(wl.E):
        a, b = offsets[e], offsets[e + 1]
        if a == b:
            continue
        xr = hw["x"][r2s[a:b] // wl.K]
        w3 = P.routed_weights(hw, e)
        rh, ry = P.ffn_rows(xr, w3, wl.limit)
        P.assert_bf16_close(hg[a:b], rh, "h expert %d" % e)
        P.assert_bf16_close(yg[a:b], P.down_rows(hg[a:b], w3[2]), "y expert %d (chained)" % e)
        P.assert_bf16_close(yg[a:b], ry, "y expert %d (end to end)" % e,
                            extra=P.propagated_h_diff(hg[a:b], rh, w3[2]))
    # identity rows, one group, no offsets: the shared-expert form, once with h kept in the
    # workspace and once with h returned; both runs must agree bit for bit
    sw = _dev_weights(dev, ("s_gate", "s_up", "s_down"), lead=True)
    ys = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=DEV)
    _expert_ffn(s, 1, wl.T, dev["x"], None, None, sw, None, ys,
                _ws(moe.moe_expert_ffn_workspace_size(s, 1, wl.T)))
    hs = torch.empty((wl.T, wl.I), dtype=torch.bfloat16, device=DEV)
    ys2 = torch.empty_like(ys)
    _expert_ffn(s, 1, wl.T, dev["x"], None, None, sw, hs, ys2,
                _ws(moe.moe_expert_ffn_workspace_size(s, 1, wl.T)))
    torch.cuda.synchronize()
    assert torch.equal(ys, ys2)
    s3 = P.shared_weights(hw)
    rhs, rys = P.ffn_rows(hw["x"], s3, wl.limit)
    P.assert_bf16_close(as_u16(hs), rhs, "identity-row h")
    P.assert_bf16_close(as_u16(ys), P.down_rows(as_u16(hs), s3[2]), "identity-row y (chained)")
    P.assert_bf16_close(as_u16(ys), rys, "identity-row y (end to end)",
                        extra=P.propagated_h_diff(as_u16(hs), rhs, s3[2]))


@pytest.mark.parametrize("name", ["tiny_t128_h512_e32_k2", "capacity_drops_t200_e8_k2", "no_shared_t128"])
def test_moe_combine(name):
    _require_gpu()
    wl = SMALL[name]
    rng = np.random.default_rng(31)
    lo = (rng.standard_normal((wl.T, wl.E)) * 0.5).astype(np.float32)
    idx, w = oracle.route_from_logits(lo, wl.K, 2.827)
    counts, offsets, r2s, s2r = oracle.dispatch(idx, wl.E, wl.capacity)
    R = int(offsets[-1])
    yr = as_u16((torch.randn(max(R, 1), wl.H) * 0.3).to(torch.bfloat16))
    ysh = as_u16((torch.randn(wl.T, wl.H) * 0.3).to(torch.bfloat16)) if wl.n_shared else None
    s = moe.Shape.of(wl)
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=DEV)
    moe.moe_combine(s, from_u16(yr, DEV), torch.from_numpy(w).to(DEV), torch.from_numpy(s2r).to(DEV),
                    None if ysh is None else from_u16(ysh, DEV), out)
    torch.cuda.synchronize()
    P.assert_bf16_close(as_u16(out), oracle.combine(w, s2r, yr, ysh), "combine")


# ----------------------------------------------------------------------------- full sizes, sampled
FULL = ["hy4_decode_t64", "hy4_prefill_t8192", "capacity_t4096_h7168_e32_k2", "hy4_skew_t65536",
        "hy4_decode_t64_fp8", "dense_ffn_t8192_h6144_i18432", "hy4_prefill_t8192_fp8"]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    _require_gpu()
    wl = WORKLOADS[name]
    print("\n[full-size] %s T=%d H=%d E=%d K=%d I=%d" % (name, wl.T, wl.H, wl.E, wl.K, wl.I), flush=True)
    dev = generate(wl, DEV)
    shape = moe.Shape.of(wl)
    layer = moe.MoELayer.from_inputs(shape, dev)
    out = layer.forward(dev["x"])
    torch.cuda.synchronize()
    T, E, K, H, I = wl.T, wl.E, wl.K, wl.H, wl.I
    n_id = T if wl.n_shared else 0
    logits = layer.intermediate("logits", torch.float32, (T, E)).cpu().numpy()
    g_idx = layer.intermediate("topk_idx", torch.int32, (T, K)).cpu().numpy()
    g_w = layer.intermediate("topk_w", torch.float32, (T, K)).cpu().numpy()
    g_counts = layer.intermediate("counts", torch.int32, (E,)).cpu().numpy()
    g_off = layer.intermediate("offsets", torch.int32, (E + 1,)).cpu().numpy()
    g_r2s = layer.intermediate("row_to_slot", torch.int32, (T * K,)).cpu().numpy()
    g_s2r = layer.intermediate("slot_to_row", torch.int32, (T * K,)).cpu().numpy()
    h_all = layer.intermediate("h", torch.bfloat16, (n_id + T * K, I))
    y_all = layer.intermediate("y", torch.bfloat16, (n_id + T * K, H))

    # routing from the same fp32 logits: bit-exact on every token
    r_idx, r_w = oracle.route_from_logits(logits, K, wl.scale, wl.norm_topk)
    np.testing.assert_array_equal(g_idx, r_idx)
    np.testing.assert_allclose(g_w, r_w, rtol=0, atol=1e-5 * wl.scale)
    rc, ro, rr, rs = oracle.dispatch(r_idx, E, wl.capacity)
    np.testing.assert_array_equal(g_counts, rc)
    np.testing.assert_array_equal(g_off, ro)
    np.testing.assert_array_equal(g_r2s, rr)
    np.testing.assert_array_equal(g_s2r, rs)
    # properties at any size
    np.testing.assert_allclose(g_w.astype(np.float64).sum(1), wl.scale, rtol=1e-5)
    R = int(g_off[-1])
    assert R == T * K - int((g_s2r < 0).sum())
    np.testing.assert_array_equal(np.sort(g_r2s[:R]), np.sort(np.nonzero(g_s2r >= 0)[0]))

    # sampled tokens: logits, every routed row, the shared row and the output
    rng = np.random.default_rng(1234)
    n_s = 8 if T <= 64 else 5
    toks = np.sort(rng.choice(T, n_s, replace=False))
    if wl.capacity:
        dropped_tok = np.nonzero((g_s2r < 0).reshape(T, K).any(1))[0]
        if len(dropped_tok):
            toks = np.unique(np.concatenate([toks, dropped_tok[:1]]))
    x_s = as_u16(dev["x"][torch.from_numpy(toks).to(DEV)])
    bias = None if dev["router_bias"] is None else dev["router_bias"].cpu().numpy()
    lo_s = oracle.router_logits(x_s, as_u16(dev["w_router"]), bias)
    P.assert_logits_close(logits[toks], lo_s, "sampled logits")
    _, _, probs = oracle.route_from_logits(lo_s, K, wl.scale, wl.norm_topk, want_probs=True)
    ok = P.margin_ok(probs, K)
    idx_i, _ = oracle.route_from_logits(lo_s, K, wl.scale, wl.norm_topk)
    np.testing.assert_array_equal(g_idx[toks][ok], idx_i[ok])

    cache = {}

    def host_w(n, e=None):
        t = dev[n] if e is None else dev[n][e]
        if t.dtype == torch.uint8:
            sc = dev[n + "_scale"] if e is None else dev[n + "_scale"][e]
            return oracle.Fp8(t.cpu().numpy(), sc.cpu().numpy())
        return as_u16(t)

    def expert(e):
        if e not in cache:
            cache[e] = tuple(host_w(n, e) for n in ("w_gate", "w_up", "w_down"))
        return cache[e]

    for i, t in enumerate(toks):
        rows = g_s2r[t * K:(t + 1) * K]
        kept = [j for j in range(K) if rows[j] >= 0]
        sel = torch.from_numpy((n_id + rows[kept]).astype(np.int64)).to(DEV)
        gh = as_u16(h_all[sel])
        gy = as_u16(y_all[sel])
        ry = np.zeros((max(R, 1), H), np.uint16)
        for n, j in enumerate(kept):
            wg_, wu_, wd_ = expert(int(g_idx[t, j]))
            rh1, ry1 = P.ffn_rows(x_s[i:i + 1], (wg_, wu_, wd_), wl.limit)
            P.assert_bf16_close(gh[n:n + 1], rh1, "h token %d slot %d" % (t, j))
            P.assert_bf16_close(gy[n:n + 1], P.down_rows(gh[n:n + 1], wd_),
                                "y token %d slot %d (chained)" % (t, j))
            P.assert_bf16_close(gy[n:n + 1], ry1, "y token %d slot %d (end to end)" % (t, j),
                                extra=P.propagated_h_diff(gh[n:n + 1], rh1, wd_))
            ry[rows[j]] = ry1[0]
        ys_r = None
        if wl.n_shared:
            if "shared" not in cache:
                cache["shared"] = tuple(host_w(n) for n in ("s_gate", "s_up", "s_down"))
            sd_ = cache["shared"][2]
            rhs, ys_r = P.ffn_rows(x_s[i:i + 1], cache["shared"], wl.limit)
            ghs = as_u16(h_all[int(t):int(t) + 1])
            gys = as_u16(y_all[int(t):int(t) + 1])
            P.assert_bf16_close(ghs, rhs, "h_shared token %d" % t)
            P.assert_bf16_close(gys, P.down_rows(ghs, sd_), "y_shared token %d (chained)" % t)
            P.assert_bf16_close(gys, ys_r, "y_shared token %d (end to end)" % t,
                                extra=P.propagated_h_diff(ghs, rhs, sd_))
        g_out = as_u16(out[int(t):int(t) + 1])
        w1 = g_w[t:t + 1]
        s2r1 = g_s2r[t * K:(t + 1) * K]
        # chained: oracle combine of the GPU rows
        gy_full = np.zeros((max(R, 1), H), np.uint16)
        gy_full[rows[kept]] = gy
        if not wl.n_shared:
            gys = None
        P.assert_bf16_close(g_out, oracle.combine(w1, s2r1, gy_full, gys), "out (chained) token %d" % t)
        # independent: oracle rows, with the measured y differences propagated
        r_out = oracle.combine(w1, s2r1, ry, ys_r)
        extra = P.propagated_y_diff(w1, s2r1, gy_full, ry, gys, ys_r)
        P.assert_bf16_close(g_out, r_out, "out (end to end) token %d" % t, extra=extra)
