"""GPU parity of the W8A8 form (FP8 expert weights and per-row FP8 activations) against the CPU
oracle, through the C ABI.

The quantised activations are integers decided by fp32 arithmetic that both sides carry out
in the same precision, so they are compared bit for bit: the codes and scales of x against the
oracle's quantisation of x, and those of h against the oracle's quantisation of the GPU's own h.
Every bf16 tensor must lie in its a-priori rounding interval (tests/parity.py), chained (from
the GPU's own inputs of the stage) and against the oracle's own chain, where the interval is
widened only by the checked differences upstream: an h element on a bf16 rounding boundary can
round differently on the two sides and then quantise one E4M3 step apart (and a row maximum
moves the row's scale), so y's interval adds sum_i |dequantised h difference|_i |Wd[c, i]|,
and out's the weighted y differences.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sparse_moe_layer_softmax_amd as moe
from sparse_moe_layer_softmax_amd.workloads import WORKLOADS, Workload, as_u16, generate
from tests import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def _bf16_rows(a):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.float32))).to(torch.bfloat16)


# ----------------------------------------------------------------------------- the quantiser
def _quant_cases():
    rng = np.random.default_rng(77)
    cases = {}
    v = rng.standard_normal((37, 6144)) * np.exp(rng.uniform(-6, 6, size=(37, 1)))
    v[3] = 0.0                       # zero row: scale 1, zero codes
    v[4, :100] = -0.0                # signed zeros in a live row
    cases["random_6144"] = v
    # rows whose maximum is 448 (scale exactly 1): every E4M3 midpoint (ties to even), the
    # subnormal range and its ties, values just around the saturation point
    vals = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mids = (vals[:-1] + vals[1:]) / 2
    row = np.concatenate([mids, -mids, [448.0], 2.0 ** -10 * np.arange(1, 17), -(2.0 ** -10) * np.arange(1, 17)])
    row = np.concatenate([row, np.zeros((-len(row)) % 8)])
    cases["ties_%d" % len(row)] = np.stack([row, -row, row * 0.5 + 0.0])
    cases["narrow_8"] = rng.standard_normal((5, 8))
    # rows so small that 448 / amax overflows fp32 (quantised unscaled to signed-zero codes),
    # rows around that threshold and rows whose scale amax / 448 is an fp32 subnormal
    tiny = rng.standard_normal((6, 64))
    tiny *= np.array([1e-37, 1e-36, 1.3e-36, 1.4e-36, 3e-36, 1e-35])[:, None] / np.abs(tiny).max(1, keepdims=True)
    cases["tiny_rows_64"] = tiny
    cases["odd_520"] = rng.standard_normal((9, 520)) * 3.0
    return cases


@pytest.mark.parametrize("case", list(_quant_cases()))
def test_quantize_rows_bit_exact(case):
    _require_gpu()
    v = _quant_cases()[case]
    x = _bf16_rows(v).to(DEV)
    rows, cols = x.shape
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=DEV)
    scales = torch.empty(rows, dtype=torch.float32, device=DEV)
    moe.moe_quantize_rows_e4m3(x, codes, scales)
    torch.cuda.synchronize()
    rc, rs = oracle.quant_rows_e4m3(as_u16(x))
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)


def test_quantize_rows_rejects_bad_arguments():
    _require_gpu()
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device=DEV)
    c = torch.empty((4, 64), dtype=torch.uint8, device=DEV)
    s = torch.empty(4, dtype=torch.float32, device=DEV)
    lib = moe.library()
    assert lib.moe_quantize_rows_e4m3(x.data_ptr(), 4, 60, c.data_ptr(), s.data_ptr(), None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_rows_e4m3(x.data_ptr(), 0, 64, c.data_ptr(), s.data_ptr(), None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_rows_e4m3(x.data_ptr() + 2, 4, 64, c.data_ptr(), s.data_ptr(), None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_rows_e4m3(None, 4, 64, c.data_ptr(), s.data_ptr(), None) == moe.MOE_ERR_INVALID_ARG


# ----------------------------------------------------------------------------- the layer
def _w8a8(wl: Workload, name: str, seed: int) -> Workload:
    return wl.with_(name=name, fp8=True, act_fp8=True, seed=seed)


_BASE = WORKLOADS["tiny_t128_h512_e32_k2"]
SMALL = {
    # weight-streaming (decode) kernel: one and several 64-row tiles, ragged tails
    "w8a8_tiny_t128_h512_e32_k2": _w8a8(_BASE, "w8a8_tiny_t128_h512_e32_k2", 60),
    "w8a8_ragged_t130_h256_e256_k8": _w8a8(
        Workload("r", T=130, H=256, E=256, K=8, I=256, scale=2.827), "w8a8_ragged_t130_h256_e256_k8", 61),
    "w8a8_single_token_t1_e256_k8": _w8a8(
        Workload("s", T=1, H=256, E=256, K=8, I=512, scale=2.827), "w8a8_single_token_t1_e256_k8", 62),
    "w8a8_no_shared_t128": _w8a8(_BASE.with_(n_shared=0), "w8a8_no_shared_t128", 63),
    "w8a8_capacity_drops_t200_e8_k2": _w8a8(
        Workload("c", T=200, H=256, E=8, K=2, I=256, capacity=30, zipf=0.3),
        "w8a8_capacity_drops_t200_e8_k2", 64),
    "w8a8_clamp_forced_t128": _w8a8(_BASE.with_(x_std=30.0), "w8a8_clamp_forced_t128", 65),
    # LDS-tiled MFMA kernel (FP8 MFMA): one and two row tiles per expert, bands of row tiles,
    # partly filled tiles, a wide dense FFN
    "w8a8_multi_tile_t300_e16_k4": _w8a8(
        Workload("m", T=300, H=512, E=16, K=4, I=256, scale=2.827), "w8a8_multi_tile_t300_e16_k4", 66),
    "w8a8_bands_t3000_e4_k2": _w8a8(
        Workload("b", T=3000, H=256, E=4, K=2, I=256, scale=2.827), "w8a8_bands_t3000_e4_k2", 67),
    "w8a8_midsize_t1000_h512_e16_k4": _w8a8(
        Workload("d", T=1000, H=512, E=16, K=4, I=256, scale=2.827, zipf=0.4),
        "w8a8_midsize_t1000_h512_e16_k4", 68),
    "w8a8_midsize_t640_h256_e32_k8": _w8a8(
        Workload("e", T=640, H=256, E=32, K=8, I=512, scale=2.827), "w8a8_midsize_t640_h256_e32_k8", 69),
    "w8a8_dense_ffn_t700_h512_i2304": _w8a8(
        Workload("f", T=700, H=512, E=1, K=1, I=2304, n_shared=0), "w8a8_dense_ffn_t700_h512_i2304", 70),
    # the Hy4 width element by element on the tiled FP8 MFMA path (gate/up K-loop of 48 tiles of
    # 128 codes, down of 16): 128 tokens, 4 experts of about 64 rows, top-2, the shared expert
    "w8a8_hy4_width_t128_e4_k2": _w8a8(
        Workload("w", T=128, H=6144, E=4, K=2, I=2048, scale=2.827, w_std=0.006, router_std=0.006),
        "w8a8_hy4_width_t128_e4_k2", 71),
}


def _fp8(hw, n, e=None):
    q = hw[n] if e is None else hw[n][e]
    s = hw[n + "_scale"] if e is None else hw[n + "_scale"][e]
    return oracle.Fp8(q, s)


def check_w8a8_layer(wl, hw, g):
    T, K, E, H, I = wl.T, wl.K, wl.E, wl.H, wl.I
    n_id = T if wl.n_shared else 0
    # routing from the GPU's fp32 logits: bit-exact
    r_idx, r_w = oracle.route_from_logits(g["logits"], K, wl.scale, wl.norm_topk)
    np.testing.assert_array_equal(g["topk_idx"], r_idx)
    np.testing.assert_allclose(g["topk_w"], r_w, rtol=0, atol=1e-5 * wl.scale)
    rc, ro, rr, rs = oracle.dispatch(r_idx, E, wl.capacity)
    for k, ref in (("counts", rc), ("offsets", ro), ("row_to_slot", rr), ("slot_to_row", rs)):
        np.testing.assert_array_equal(g[k], ref, err_msg=k)
    R = int(ro[-1])
    # x codes and scales: bit-exact
    xq, sx = oracle.quant_rows_e4m3(hw["x"])
    np.testing.assert_array_equal(g["x_scale"], sx)
    np.testing.assert_array_equal(g["xq"], xq)
    # h codes and scales of every valid row (shared rows first): bit-exact from the GPU's own h
    h_all = np.concatenate([g["h_shared"], g["h_routed"][:R]]) if n_id else g["h_routed"][:R]
    hq, sh = oracle.quant_rows_e4m3(h_all)
    np.testing.assert_array_equal(g["h_scale"][:n_id + R], sh)
    np.testing.assert_array_equal(g["hq"][:n_id + R], hq)
    # the oracle's own chain from the same logits
    r = oracle.layer_forward_w8a8(hw["x"], hw["w_router"], _fp8(hw, "w_gate"), _fp8(hw, "w_up"),
                                  _fp8(hw, "w_down"), K, bias=hw["router_bias"],
                                  sg=_fp8(hw, "s_gate") if n_id else None,
                                  su=_fp8(hw, "s_up") if n_id else None,
                                  sd=_fp8(hw, "s_down") if n_id else None, scale=wl.scale,
                                  limit=wl.limit, capacity=wl.capacity, norm_topk=wl.norm_topk,
                                  logits=g["logits"])
    h_orc = np.concatenate([r["h_shared"], r["h_routed"][:R]]) if n_id else r["h_routed"][:R]
    hq_o, sh_o = oracle.quant_rows_e4m3(h_orc)
    G = E + (1 if n_id else 0)
    chain = P.chain_for(P.kernel_of(n_id + T * K, G), True, True)
    stats = P.Stats()
    groups = [("shared", None, 0, np.arange(T))] if n_id else []
    groups += [("expert %d" % e, e, n_id + int(ro[e]), g["row_to_slot"][ro[e]:ro[e + 1]] // K)
               for e in range(E) if ro[e] < ro[e + 1]]
    y_orc_all = np.concatenate([r["y_shared"], r["y_routed"][:R]]) if n_id else r["y_routed"][:R]
    y_gpu_all = np.concatenate([g["y_shared"], g["y_routed"][:R]]) if n_id else g["y_routed"][:R]
    for label, key, a, tok in groups:
        b = a + len(tok)
        w3 = tuple(_fp8(hw, n, key) for n in (("s_gate", "s_up", "s_down") if key is None
                                               else ("w_gate", "w_up", "w_down")))
        P.check_w8a8_rows(label, g["xq"][tok], g["x_scale"][tok], w3, wl.limit, chain,
                          h_all[a:b], g["hq"][a:b], g["h_scale"][a:b], y_gpu_all[a:b],
                          h_orc[a:b], hq_o[a:b], sh_o[a:b], y_orc_all[a:b], stats)
    s2r = g["slot_to_row"].reshape(T, K)
    P.check_out("layer", g["topk_w"], r["topk_w"], s2r, g["y_routed"][:max(R, 1)],
                r["y_routed"][:max(R, 1)], g["y_shared"], r.get("y_shared"), g["out"], r["out"],
                stats)
    print("[parity] %s: %s" % (wl.name, stats.line()), flush=True)


_E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


@pytest.mark.parametrize("name", list(SMALL))
def test_w8a8_layer_small(name):
    _require_gpu()
    wl = SMALL[name]
    dev = generate(wl, DEV)
    hw = P.host(dev)
    g, _, _ = P.run_layer_gpu(wl, dev)
    P.assert_logits_close(g["logits"], oracle.router_logits(hw["x"], hw["w_router"], hw["router_bias"]))
    check_w8a8_layer(wl, hw, g)
    if name.endswith("capacity_drops_t200_e8_k2"):
        assert (g["slot_to_row"] < 0).sum() > 0, "this case must drop slots"
    if name.endswith("clamp_forced_t128"):
        assert np.abs(P.f64(g["h_routed"][: int(g["offsets"][-1])])).max() > 50


def test_w8a8_layer_is_deterministic():
    _require_gpu()
    wl = SMALL["w8a8_midsize_t640_h256_e32_k8"]
    dev = generate(wl, DEV)
    g, layer, _ = P.run_layer_gpu(wl, dev)
    for _ in range(2):
        np.testing.assert_array_equal(as_u16(layer.forward(dev["x"])), g["out"])


# ----------------------------------------------------------------------------- full size, sampled
FULL = ["hy4_decode_t64_w8a8", "hy4_prefill_t8192_w8a8", "hy4_skew_t65536_w8a8"]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", FULL)
def test_w8a8_full_size_sampled(name):
    _require_gpu()
    wl = WORKLOADS[name]
    print("\n[full-size] %s T=%d H=%d E=%d K=%d I=%d" % (name, wl.T, wl.H, wl.E, wl.K, wl.I), flush=True)
    dev = generate(wl, DEV)
    layer = moe.MoELayer.from_inputs(moe.Shape.of(wl), dev)
    out = layer.forward(dev["x"])
    torch.cuda.synchronize()
    T, E, K, H, I = wl.T, wl.E, wl.K, wl.H, wl.I
    n_id = T if wl.n_shared else 0
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
    R = int(ro[-1])
    h_all = rd("h", torch.bfloat16, (n_id + T * K, I))
    y_all = rd("y", torch.bfloat16, (n_id + T * K, H))
    xq_all = rd("xq", torch.uint8, (T, H))
    sx_all = rd("x_scale", torch.float32, (T,)).cpu().numpy()
    hq_all = rd("hq", torch.uint8, (n_id + T * K, I))
    sh_all = rd("h_scale", torch.float32, (n_id + T * K,)).cpu().numpy()
    rng = np.random.default_rng(4321)
    toks = np.sort(rng.choice(T, 8 if T <= 64 else 5, replace=False))
    cache = {}

    def w(n, e=None):
        key = (n, e)
        if key not in cache:
            t = dev[n] if e is None else dev[n][e]
            sc = dev[n + "_scale"] if e is None else dev[n + "_scale"][e]
            cache[key] = oracle.Fp8(t.cpu().numpy(), sc.cpu().numpy())
        return cache[key]

    kern = P.kernel_of(n_id + T * K, E + (1 if n_id else 0))
    chain = P.chain_for(kern, True, True)
    stats = P.Stats()
    yg_rows, yo_rows, ysg, yso = {}, {}, [], []
    qs, items = {}, []
    for t in toks:
        t = int(t)
        x_t = as_u16(dev["x"][t:t + 1])
        q_t, s_t = oracle.quant_rows_e4m3(x_t)
        np.testing.assert_array_equal(xq_all[t:t + 1].cpu().numpy(), q_t, err_msg="xq token %d" % t)
        np.testing.assert_array_equal(sx_all[t:t + 1], s_t)
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
                sh_all[row:row + 1], as_u16(y_all[row:row + 1]))

    def check(prep):
        t, j, e, row, w3, gh, hq_g, sh_g, gy = prep
        q_t, s_t = qs[t]
        hq_r, sh_r = oracle.quant_rows_e4m3(gh)  # the GPU's codes from its own h: bit-exact
        np.testing.assert_array_equal(hq_g, hq_r, err_msg="hq row %d" % row)
        np.testing.assert_array_equal(sh_g, sh_r)
        h_o = oracle.gateup_rows_w8a8(q_t, s_t, w3[0], w3[1], wl.limit)
        hq_o, sh_o = oracle.quant_rows_e4m3(h_o)
        y_o = oracle.down_rows_w8a8(hq_o, sh_o, w3[2])
        st = P.Stats()
        P.check_w8a8_rows("token %d slot %d" % (t, j), q_t, s_t, w3, wl.limit, chain, gh, hq_g,
                          sh_g, gy, h_o, hq_o, sh_o, y_o, st)
        return e, row, gy[0], y_o[0], st

    for e, row, gy0, yo0, st in P.run_pipelined(prepare, check, items):
        stats.merge(st)
        if e is None:
            ysg.append(gy0)
            yso.append(yo0)
        else:
            yg_rows[row], yo_rows[row] = gy0, yo0
    # the sampled tokens' outputs against the oracle's combine of its own rows
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
def test_w8a8_operands_past_4_gib(case):
    """An FP8 operand of more than 4 GiB takes the tiled kernel's 64-bit-address DMA form: the h
    codes [2.2M, 2048] of the down projection, or the x codes [2.2M, 2048] of gate/up (E = 1,
    k = 1, no shared expert, so GEMM row t is token t). Checked against the oracle on the rows
    around the 2^32-byte boundary of that operand and on the last rows."""
    _require_gpu()
    T = 2_200_000
    H, I = (256, 2048) if case.startswith("h_") else (2048, 256)
    width = I if case.startswith("h_") else H  # bytes per row of the large operand
    assert T * width > (1 << 32)
    wl = Workload(case, T=T, H=H, E=1, K=1, I=I, n_shared=0, scale=1.0, limit=10.0, seed=96,
                  fp8=True, act_fp8=True)
    print("\n[large] w8a8 %s T=%d H=%d I=%d" % (case, T, H, I), flush=True)
    dev = generate(wl, DEV)
    layer = moe.MoELayer.from_inputs(moe.Shape.of(wl), dev)
    out = layer.forward(dev["x"])
    torch.cuda.synchronize()
    boundary = (1 << 32) // width  # first row that starts past 2^32 bytes
    rows = np.unique(np.concatenate([np.arange(boundary - 40, boundary + 300), np.arange(T - 300, T)]))
    sel = torch.from_numpy(rows.astype(np.int64)).to(DEV)
    rd = lambda n, dt, shp: layer.intermediate(n, dt, shp)
    np.testing.assert_array_equal(rd("slot_to_row", torch.int32, (T,))[sel].cpu().numpy(), rows)
    xq, sx = oracle.quant_rows_e4m3(as_u16(dev["x"][sel]))
    np.testing.assert_array_equal(rd("xq", torch.uint8, (T, H))[sel].cpu().numpy(), xq)
    np.testing.assert_array_equal(rd("x_scale", torch.float32, (T,))[sel].cpu().numpy(), sx)
    gh = as_u16(rd("h", torch.bfloat16, (T, I))[sel])
    hq_g = rd("hq", torch.uint8, (T, I))[sel].cpu().numpy()
    sh_g = rd("h_scale", torch.float32, (T,))[sel].cpu().numpy()
    hq_r, sh_r = oracle.quant_rows_e4m3(gh)  # the GPU's codes from its own h: bit-exact
    np.testing.assert_array_equal(hq_g, hq_r)
    np.testing.assert_array_equal(sh_g, sh_r)
    w3 = tuple(oracle.Fp8(dev[n][0].cpu().numpy(), dev[n + "_scale"][0].cpu().numpy())
               for n in ("w_gate", "w_up", "w_down"))
    h_o = oracle.gateup_rows_w8a8(xq, sx, w3[0], w3[1], wl.limit)
    hq_o, sh_o = oracle.quant_rows_e4m3(h_o)
    y_o = oracle.down_rows_w8a8(hq_o, sh_o, w3[2])
    gy = as_u16(rd("y", torch.bfloat16, (T, H))[sel])
    assert P.kernel_of(T, 1) == "tiled"
    stats = P.Stats()
    P.check_w8a8_rows(case, xq, sx, w3, wl.limit, P.chain_for("tiled", True, True), gh, hq_g, sh_g,
                      gy, h_o, hq_o, sh_o, y_o, stats)
    # one expert, weight 1: the output rows are the y rows
    np.testing.assert_array_equal(as_u16(out[sel]), gy)
    print("[parity] w8a8 %s: %s" % (case, stats.line()), flush=True)
