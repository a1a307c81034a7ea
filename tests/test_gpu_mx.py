"""GPU parity of the MX form (OCP MXFP8: E4M3 codes with one E8M0 scale per 32 elements along K,
on weights and on the activations the layer quantises) against the CPU oracle, through the C ABI.

The block quantisation is integer work decided by exact arithmetic on both sides (a power-of-two
scale from the block maximum's exponent, a nearest-even E4M3 code of an exact product), so codes
and scale bytes are compared bit for bit: x's against the oracle's quantisation of x (placed at
every GEMM row that reads the token), h's against the oracle's quantisation of the GPU's own h.
Every bf16 tensor must lie in its a-priori rounding interval (tests/parity.py), chained and end
to end, as in the W8A8 tests.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
import sparse_moe_layer_softmax_amd as moe
from sparse_moe_layer_softmax_amd.workloads import WORKLOADS, Workload, as_u16, generate
from tests import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda"
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mx_blocks.txt")


def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def _bf16_rows(a):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.float32))).to(torch.bfloat16)


def _bf16_exact(a):
    """float64 values that are bf16 numbers, as a bf16 tensor (through float64, no double rounding)."""
    return torch.tensor(np.asarray(a, np.float64), dtype=torch.float64).to(torch.bfloat16)


# ----------------------------------------------------------------------------- the quantiser
def _golden_rows():
    rows = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        els = [float(eval(e, {"__builtins__": {}})) for e in line.split("#")[0].split("|")[1].split(",")]
        rows.append(els + [0.0] * (32 - len(els)))
    # four blocks per 128-element row
    while len(rows) % 4:
        rows.append([0.0] * 32)
    return np.array(rows).reshape(-1, 128)


def _quant_cases():
    rng = np.random.default_rng(78)
    cases = {}
    v = rng.standard_normal((37, 6144)) * np.exp(rng.uniform(-6, 6, size=(37, 1)))
    v *= np.exp(rng.standard_normal((37, 6144 // 32, 1)) * 2).repeat(32, axis=2).reshape(37, 6144)
    v[3] = 0.0
    v[4, :100] = -0.0
    cases["random_6144"] = v
    cases["golden_blocks"] = _golden_rows()
    # block maxima across the whole E8M0 range: tiny (bf16 subnormal) to near the bf16 maximum
    mags = 2.0 ** np.array([-133, -130, -126, -120, -100, -20, 0, 20, 100, 120, 126, 127])
    cases["magnitudes_128"] = rng.standard_normal((12, 128)) * mags[:, None] / 4
    cases["narrow_128"] = rng.standard_normal((5, 128))
    return cases


@pytest.mark.parametrize("case", list(_quant_cases()))
def test_quantize_rows_mx_bit_exact(case):
    _require_gpu()
    v = _quant_cases()[case]
    x = (_bf16_exact(v) if case == "golden_blocks" else _bf16_rows(v)).to(DEV)
    rows, cols = x.shape
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=DEV)
    planes = torch.empty((cols // 128, rows, 4), dtype=torch.uint8, device=DEV)
    moe.moe_quantize_rows_mx(x, codes, planes)
    torch.cuda.synchronize()
    rc, rs = oracle.mx_quant_rows(as_u16(x))
    np.testing.assert_array_equal(P.mx_planes_to_rows(planes.cpu().numpy(), rows), rs)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)


def test_quantize_rows_mx_rejects_bad_arguments():
    _require_gpu()
    x = torch.zeros((4, 256), dtype=torch.bfloat16, device=DEV)
    c = torch.empty((4, 256), dtype=torch.uint8, device=DEV)
    s = torch.empty((2, 4, 4), dtype=torch.uint8, device=DEV)
    lib = moe.library()
    assert lib.moe_quantize_rows_mx(x.data_ptr(), 4, 192, c.data_ptr(), s.data_ptr(), None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_rows_mx(x.data_ptr(), 0, 256, c.data_ptr(), s.data_ptr(), None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_rows_mx(x.data_ptr() + 2, 4, 256, c.data_ptr(), s.data_ptr(), None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_rows_mx(x.data_ptr(), 4, 256, c.data_ptr(), s.data_ptr() + 1, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_rows_mx(None, 4, 256, c.data_ptr(), s.data_ptr(), None) == moe.MOE_ERR_INVALID_ARG


# ----------------------------------------------------------------------------- the layer
def _mx(wl: Workload, name: str, seed: int) -> Workload:
    return wl.with_(name=name, fp8=True, act_fp8=True, mx=True, seed=seed)


_BASE = WORKLOADS["tiny_t128_h512_e32_k2"]
SMALL = {
    # weight-streaming (decode) kernel: 16- and 64-row tiles, ragged tails
    "mx_tiny_t128_h512_e32_k2": _mx(_BASE, "mx_tiny_t128_h512_e32_k2", 80),
    "mx_ragged_t130_h256_e256_k8": _mx(
        Workload("r", T=130, H=256, E=256, K=8, I=256, scale=2.827), "mx_ragged_t130_h256_e256_k8", 81),
    "mx_single_token_t1_e256_k8": _mx(
        Workload("s", T=1, H=256, E=256, K=8, I=512, scale=2.827), "mx_single_token_t1_e256_k8", 82),
    "mx_no_shared_t128": _mx(_BASE.with_(n_shared=0), "mx_no_shared_t128", 83),
    "mx_capacity_drops_t200_e8_k2": _mx(
        Workload("c", T=200, H=256, E=8, K=2, I=256, capacity=30, zipf=0.3),
        "mx_capacity_drops_t200_e8_k2", 84),
    "mx_clamp_forced_t128": _mx(_BASE.with_(x_std=30.0), "mx_clamp_forced_t128", 85),
    # LDS-tiled kernel (scaled FP8 MFMA): one and two row tiles per expert, bands, partly
    # filled tiles, a wide dense FFN, the Hy4 width
    "mx_multi_tile_t300_e16_k4": _mx(
        Workload("m", T=300, H=512, E=16, K=4, I=256, scale=2.827), "mx_multi_tile_t300_e16_k4", 86),
    "mx_bands_t3000_e4_k2": _mx(
        Workload("b", T=3000, H=256, E=4, K=2, I=256, scale=2.827), "mx_bands_t3000_e4_k2", 87),
    "mx_midsize_t1000_h512_e16_k4": _mx(
        Workload("d", T=1000, H=512, E=16, K=4, I=256, scale=2.827, zipf=0.4),
        "mx_midsize_t1000_h512_e16_k4", 88),
    "mx_no_shared_tiled_t640_e8_k2": _mx(
        Workload("n", T=640, H=512, E=8, K=2, I=256, n_shared=0), "mx_no_shared_tiled_t640_e8_k2", 89),
    "mx_dense_ffn_t700_h512_i2304": _mx(
        Workload("f", T=700, H=512, E=1, K=1, I=2304, n_shared=0), "mx_dense_ffn_t700_h512_i2304", 90),
    "mx_hy4_width_t512_e8_k2": _mx(
        Workload("w", T=512, H=6144, E=8, K=2, I=2048, scale=2.827, w_std=0.006, router_std=0.006),
        "mx_hy4_width_t512_e8_k2", 91),
}


def _mxw(hw, n, e=None):
    q = hw[n] if e is None else hw[n][e]
    s = hw[n + "_mx"] if e is None else hw[n + "_mx"][e]
    return oracle.Mx(q, s)


def check_mx_layer(wl, hw, g):
    T, K, E, H, I = wl.T, wl.K, wl.E, wl.H, wl.I
    n_id = T if wl.n_shared else 0
    r_idx, r_w = oracle.route_from_logits(g["logits"], K, wl.scale, wl.norm_topk)
    np.testing.assert_array_equal(g["topk_idx"], r_idx)
    np.testing.assert_allclose(g["topk_w"], r_w, rtol=0, atol=1e-5 * wl.scale)
    rc, ro, rr, rs = oracle.dispatch(r_idx, E, wl.capacity)
    for k, ref in (("counts", rc), ("offsets", ro), ("row_to_slot", rr), ("slot_to_row", rs)):
        np.testing.assert_array_equal(g[k], ref, err_msg=k)
    R = int(ro[-1])
    # x codes (token order) and scale bytes at every GEMM row that reads the token: bit-exact
    xq, xs = oracle.mx_quant_rows(hw["x"])
    np.testing.assert_array_equal(g["xq"], xq)
    tok_of_row = np.concatenate([np.arange(n_id), rr[:R] // K]).astype(np.int64)
    np.testing.assert_array_equal(g["x_scale"][:n_id + R], xs[tok_of_row])
    # h codes and scale bytes of every valid row: bit-exact from the GPU's own h
    h_all = np.concatenate([g["h_shared"], g["h_routed"][:R]]) if n_id else g["h_routed"][:R]
    hq, hs = oracle.mx_quant_rows(h_all)
    np.testing.assert_array_equal(g["hq"][:n_id + R], hq)
    np.testing.assert_array_equal(g["h_scale"][:n_id + R], hs)
    r = oracle.layer_forward_mx(hw["x"], hw["w_router"], _mxw(hw, "w_gate"), _mxw(hw, "w_up"),
                                _mxw(hw, "w_down"), K, bias=hw["router_bias"],
                                sg=_mxw(hw, "s_gate") if n_id else None,
                                su=_mxw(hw, "s_up") if n_id else None,
                                sd=_mxw(hw, "s_down") if n_id else None, scale=wl.scale,
                                limit=wl.limit, capacity=wl.capacity, norm_topk=wl.norm_topk,
                                logits=g["logits"])
    h_orc = np.concatenate([r["h_shared"], r["h_routed"][:R]]) if n_id else r["h_routed"][:R]
    hq_o, hs_o = oracle.mx_quant_rows(h_orc)
    G = E + (1 if n_id else 0)
    chain = P.chain_for(P.kernel_of(n_id + T * K, G), True, True, mx=True)
    stats = P.Stats()
    groups = [("shared", None, 0, np.arange(T))] if n_id else []
    groups += [("expert %d" % e, e, n_id + int(ro[e]), g["row_to_slot"][ro[e]:ro[e + 1]] // K)
               for e in range(E) if ro[e] < ro[e + 1]]
    y_orc_all = np.concatenate([r["y_shared"], r["y_routed"][:R]]) if n_id else r["y_routed"][:R]
    y_gpu_all = np.concatenate([g["y_shared"], g["y_routed"][:R]]) if n_id else g["y_routed"][:R]
    for label, key, a, tok in groups:
        b = a + len(tok)
        w3 = tuple(_mxw(hw, n, key) for n in (("s_gate", "s_up", "s_down") if key is None
                                               else ("w_gate", "w_up", "w_down")))
        P.check_mx_rows(label, xq[tok], xs[tok], w3, wl.limit, chain, h_all[a:b], g["hq"][a:b],
                        g["h_scale"][a:b], y_gpu_all[a:b], h_orc[a:b], hq_o[a:b], hs_o[a:b],
                        y_orc_all[a:b], stats)
    s2r = g["slot_to_row"].reshape(T, K)
    P.check_out("layer", g["topk_w"], r["topk_w"], s2r, g["y_routed"][:max(R, 1)],
                r["y_routed"][:max(R, 1)], g["y_shared"], r.get("y_shared"), g["out"], r["out"],
                stats)
    print("[parity] %s: %s" % (wl.name, stats.line()), flush=True)


@pytest.mark.parametrize("name", list(SMALL))
def test_mx_layer_small(name):
    _require_gpu()
    wl = SMALL[name]
    dev = generate(wl, DEV)
    hw = P.host(dev)
    g, _, _ = P.run_layer_gpu(wl, dev)
    P.assert_logits_close(g["logits"], oracle.router_logits(hw["x"], hw["w_router"], hw["router_bias"]))
    check_mx_layer(wl, hw, g)
    if name.endswith("capacity_drops_t200_e8_k2"):
        assert (g["slot_to_row"] < 0).sum() > 0, "this case must drop slots"
    if name.endswith("clamp_forced_t128"):
        assert np.abs(P.f64(g["h_routed"][: int(g["offsets"][-1])])).max() > 50


def test_small_cases_reach_both_kernels():
    kinds = {P.kernel_of(wl.T * wl.K + (wl.T if wl.n_shared else 0), wl.E + wl.n_shared)
             for wl in SMALL.values()}
    assert kinds == {"skinny", "tiled"}


def test_mx_layer_is_deterministic():
    _require_gpu()
    wl = SMALL["mx_midsize_t1000_h512_e16_k4"]
    dev = generate(wl, DEV)
    g, layer, _ = P.run_layer_gpu(wl, dev)
    for _ in range(2):
        np.testing.assert_array_equal(as_u16(layer.forward(dev["x"])), g["out"])


# ----------------------------------------------------------------------------- full size, sampled
FULL = ["hy4_decode_t64_mx", "hy4_prefill_t8192_mx", "hy4_skew_t65536_mx"]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", FULL)
def test_mx_full_size_sampled(name):
    _require_gpu()
    wl = WORKLOADS[name]
    print("\n[full-size] %s T=%d H=%d E=%d K=%d I=%d" % (name, wl.T, wl.H, wl.E, wl.K, wl.I), flush=True)
    dev = generate(wl, DEV)
    layer = moe.MoELayer.from_inputs(moe.Shape.of(wl), dev)
    out = layer.forward(dev["x"])
    torch.cuda.synchronize()
    T, E, K, H, I = wl.T, wl.E, wl.K, wl.H, wl.I
    n_id = T if wl.n_shared else 0
    rows_all = n_id + T * K
    rd = lambda n, dt, shp: layer.intermediate(n, dt, shp)
    logits = rd("logits", torch.float32, (T, E)).cpu().numpy()
    g_idx = rd("topk_idx", torch.int32, (T, K)).cpu().numpy()
    g_w = rd("topk_w", torch.float32, (T, K)).cpu().numpy()
    g_off = rd("offsets", torch.int32, (E + 1,)).cpu().numpy()
    g_s2r = rd("slot_to_row", torch.int32, (T * K,)).cpu().numpy()
    r_idx, r_w = oracle.route_from_logits(logits, K, wl.scale, wl.norm_topk)
    np.testing.assert_array_equal(g_idx, r_idx)
    rc, ro, rr, rs = oracle.dispatch(r_idx, E, wl.capacity)
    np.testing.assert_array_equal(g_off, ro)
    np.testing.assert_array_equal(g_s2r, rs)
    h_all = rd("h", torch.bfloat16, (rows_all, I))
    y_all = rd("y", torch.bfloat16, (rows_all, H))
    xq_all = rd("xq", torch.uint8, (T, H))
    hq_all = rd("hq", torch.uint8, (rows_all, I))
    sr = layer.layout["scale_rows"]
    xs_planes = rd("x_scale", torch.uint8, (H // 128, sr, 4)).cpu().numpy()
    hs_planes = rd("h_scale", torch.uint8, (I // 128, sr, 4)).cpu().numpy()
    row_scales = lambda planes, row: np.ascontiguousarray(planes[:, row, :].reshape(1, -1))
    rng = np.random.default_rng(4322)
    toks = np.sort(rng.choice(T, 8 if T <= 64 else 5, replace=False))
    cache = {}

    def w(n, e=None):
        key = (n, e)
        if key not in cache:
            t = dev[n] if e is None else dev[n][e]
            sc = dev[n + "_mx"] if e is None else dev[n + "_mx"][e]
            cache[key] = oracle.Mx(t.cpu().numpy(), sc.cpu().numpy())
        return cache[key]

    kern = P.kernel_of(rows_all, E + (1 if n_id else 0))
    chain = P.chain_for(kern, True, True, mx=True)
    stats = P.Stats()
    yg_rows, yo_rows, ysg, yso = {}, {}, [], []
    qs, items = {}, []
    for t in toks:
        t = int(t)
        q_t, s_t = oracle.mx_quant_rows(as_u16(dev["x"][t:t + 1]))
        np.testing.assert_array_equal(xq_all[t:t + 1].cpu().numpy(), q_t, err_msg="xq token %d" % t)
        qs[t] = (q_t, s_t)
        rows = g_s2r[t * K:(t + 1) * K]
        items += [(t, j, int(g_idx[t, j]), n_id + int(rows[j])) for j in range(K) if rows[j] >= 0]
        if n_id:
            items.append((t, -1, None, t))  # the shared row

    def prepare(it):
        t, j, e, row = it
        w3 = (w("s_gate"), w("s_up"), w("s_down")) if e is None else \
            (w("w_gate", e), w("w_up", e), w("w_down", e))
        return (t, j, e, row, w3, as_u16(h_all[row:row + 1]), hq_all[row:row + 1].cpu().numpy(),
                as_u16(y_all[row:row + 1]))

    def check(prep):
        t, j, e, row, w3, gh, hq_g, gy = prep
        q_t, s_t = qs[t]
        np.testing.assert_array_equal(row_scales(xs_planes, row), s_t, err_msg="x scales row %d" % row)
        hs_g = row_scales(hs_planes, row)
        hq_r, hs_r = oracle.mx_quant_rows(gh)  # the GPU's codes from its own h: bit-exact
        np.testing.assert_array_equal(hq_g, hq_r, err_msg="hq row %d" % row)
        np.testing.assert_array_equal(hs_g, hs_r, err_msg="h scales row %d" % row)
        h_o = oracle.gateup_rows_mx(q_t, s_t, w3[0], w3[1], wl.limit)
        hq_o, hs_o = oracle.mx_quant_rows(h_o)
        y_o = oracle.down_rows_mx(hq_o, hs_o, w3[2])
        st = P.Stats()
        P.check_mx_rows("token %d slot %d" % (t, j), q_t, s_t, w3, wl.limit, chain, gh, hq_g,
                        hs_g, gy, h_o, hq_o, hs_o, y_o, st)
        return e, row, gy[0], y_o[0], st

    for e, row, gy0, yo0, st in P.run_pipelined(prepare, check, items):
        stats.merge(st)
        if e is None:
            ysg.append(gy0)
            yso.append(yo0)
        else:
            yg_rows[row], yo_rows[row] = gy0, yo0
    s2r_t = g_s2r.reshape(T, K)[toks]
    uniq = sorted(yg_rows)
    pos = {r: i for i, r in enumerate(uniq)}
    loc = np.array([[pos[n_id + int(r)] if r >= 0 else -1 for r in rr] for rr in s2r_t], np.int32)
    yg = np.stack([yg_rows[r] for r in uniq])
    yo = np.stack([yo_rows[r] for r in uniq])
    ysg = np.stack(ysg) if n_id else None
    yso = np.stack(yso) if n_id else None
    out_orc = oracle.combine(r_w[toks], loc.ravel(), yo, yso)
    P.check_out("tokens %s" % toks.tolist(), g_w[toks], r_w[toks], loc, yg, yo, ysg, yso,
                as_u16(out[torch.from_numpy(toks).to(DEV)]), out_orc, stats)
    print("[parity] %s: %s" % (name, stats.line()), flush=True)


# ----------------------------------------------------------------------------- operands past 4 GiB
@pytest.mark.timeout(300)
@pytest.mark.parametrize("case", ["h_codes_past_4gib", "x_codes_past_4gib"])
def test_mx_operands_past_4_gib(case):
    """An FP8 operand of more than 4 GiB takes the tiled kernel's 64-bit-address DMA form: the h
    codes [2.2M, 2048] of the down projection, or the x codes [2.2M, 2048] of gate/up (E = 1,
    k = 1, no shared expert, so GEMM row t is token t). Checked against the oracle on the rows
    around the 2^32-byte boundary of that operand and on the last rows."""
    _require_gpu()
    T = 2_200_000
    H, I = (256, 2048) if case.startswith("h_") else (2048, 256)
    width = I if case.startswith("h_") else H  # bytes per row of the large operand
    assert T * width > (1 << 32)
    wl = Workload(case, T=T, H=H, E=1, K=1, I=I, n_shared=0, scale=1.0, limit=10.0, seed=95,
                  fp8=True, act_fp8=True, mx=True)
    print("\n[large] mx %s T=%d H=%d I=%d" % (case, T, H, I), flush=True)
    dev = generate(wl, DEV)
    layer = moe.MoELayer.from_inputs(moe.Shape.of(wl), dev)
    out = layer.forward(dev["x"])
    torch.cuda.synchronize()
    boundary = (1 << 32) // width  # first row that starts past 2^32 bytes
    rows = np.unique(np.concatenate([np.arange(boundary - 40, boundary + 300), np.arange(T - 300, T)]))
    sel = torch.from_numpy(rows.astype(np.int64)).to(DEV)
    rd = lambda n, dt, shp: layer.intermediate(n, dt, shp)
    np.testing.assert_array_equal(rd("slot_to_row", torch.int32, (T,))[sel].cpu().numpy(), rows)
    sr = layer.layout["scale_rows"]
    plane_rows = lambda name, k: np.ascontiguousarray(
        rd(name, torch.uint8, (k // 128, sr, 4))[:, sel, :].cpu().numpy().transpose(1, 0, 2)
        .reshape(len(rows), -1))
    xq, xs = oracle.mx_quant_rows(as_u16(dev["x"][sel]))
    np.testing.assert_array_equal(rd("xq", torch.uint8, (T, H))[sel].cpu().numpy(), xq)
    np.testing.assert_array_equal(plane_rows("x_scale", H), xs)
    gh = as_u16(rd("h", torch.bfloat16, (T, I))[sel])
    hq_g = rd("hq", torch.uint8, (T, I))[sel].cpu().numpy()
    hs_g = plane_rows("h_scale", I)
    hq_r, hs_r = oracle.mx_quant_rows(gh)  # the GPU's codes from its own h: bit-exact
    np.testing.assert_array_equal(hq_g, hq_r)
    np.testing.assert_array_equal(hs_g, hs_r)
    w3 = tuple(oracle.Mx(dev[n][0].cpu().numpy(), dev[n + "_mx"][0].cpu().numpy())
               for n in ("w_gate", "w_up", "w_down"))
    h_o = oracle.gateup_rows_mx(xq, xs, w3[0], w3[1], wl.limit)
    hq_o, hs_o = oracle.mx_quant_rows(h_o)
    y_o = oracle.down_rows_mx(hq_o, hs_o, w3[2])
    gy = as_u16(rd("y", torch.bfloat16, (T, H))[sel])
    assert P.kernel_of(T, 1) == "tiled"
    stats = P.Stats()
    P.check_mx_rows(case, xq, xs, w3, wl.limit, P.chain_for("tiled", True, True, mx=True), gh, hq_g,
                    hs_g, gy, h_o, hq_o, hs_o, y_o, stats)
    # one expert, weight 1: the output rows are the y rows
    np.testing.assert_array_equal(as_u16(out[sel]), gy)
    print("[parity] mx %s: %s" % (case, stats.line()), flush=True)
