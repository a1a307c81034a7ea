"""GPU parity of the W8A8 form (FP8 expert weights and per-row FP8 activations) against the CPU
oracle, through the C ABI.

The quantised activations are integers decided by fp32 arithmetic that both sides carry out
in the same precision, so they are compared bit for bit: the codes and scales of x against the
oracle's quantisation of x, and those of h against the oracle's quantisation of the GPU's own h.
Every bf16 tensor is compared, chained, with the oracle applied to the same inputs the GPU stage
consumed (h from the GPU's x codes, y from the GPU's h codes, out from the GPU's rows), within
|gpu - oracle| <= 1e-2*|oracle| + 1e-3*rms(oracle). Against the oracle's own chain from x the
same bound holds with the measured upstream differences propagated: an h element on a bf16
rounding boundary can round differently on the two sides and then quantise one E4M3 step apart
(and a row maximum moves the row's scale), so y's bound adds sum_i |dequantised h difference|_i
* |Wd[c, i]|, and out's the weighted y differences.
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
}


def _fp8(hw, n, e=None):
    q = hw[n] if e is None else hw[n][e]
    s = hw[n + "_scale"] if e is None else hw[n + "_scale"][e]
    return oracle.Fp8(q, s)


def check_w8a8_layer(wl, hw, g, check_end_to_end=True):
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
    # per expert, chained: h from the GPU's x codes, y from the GPU's h codes
    for e in range(E):
        a, b = int(ro[e]), int(ro[e + 1])
        if a == b:
            continue
        tok = g["row_to_slot"][a:b] // K
        h_ref = oracle.gateup_rows_w8a8(g["xq"][tok], g["x_scale"][tok], _fp8(hw, "w_gate", e),
                                        _fp8(hw, "w_up", e), wl.limit)
        P.assert_bf16_close(g["h_routed"][a:b], h_ref, "h expert %d (chained)" % e)
        y_ref = oracle.down_rows_w8a8(g["hq"][n_id + a:n_id + b], g["h_scale"][n_id + a:n_id + b],
                                      _fp8(hw, "w_down", e))
        P.assert_bf16_close(g["y_routed"][a:b], y_ref, "y expert %d (chained)" % e)
    ys = None
    if n_id:
        hs_ref = oracle.gateup_rows_w8a8(g["xq"], g["x_scale"], _fp8(hw, "s_gate"), _fp8(hw, "s_up"),
                                         wl.limit)
        P.assert_bf16_close(g["h_shared"], hs_ref, "h_shared (chained)")
        ys = oracle.down_rows_w8a8(g["hq"][:n_id], g["h_scale"][:n_id], _fp8(hw, "s_down"))
        P.assert_bf16_close(g["y_shared"], ys, "y_shared (chained)")
    out_ref = oracle.combine(g["topk_w"], g["slot_to_row"], g["y_routed"], g["y_shared"])
    P.assert_bf16_close(g["out"], out_ref, "out (chained)")
    if check_end_to_end:
        # the oracle's own chain from the same logits. Where its h rounds one ulp away from the
        # GPU's, the h codes can differ by one E4M3 step (and a row maximum moves the whole row's
        # scale), so y gets the measured difference of the dequantised h propagated through the
        # down weights, and out the measured y differences, as in the bf16 layer's check
        r = oracle.layer_forward_w8a8(hw["x"], hw["w_router"], _fp8(hw, "w_gate"), _fp8(hw, "w_up"),
                                      _fp8(hw, "w_down"), K, bias=hw["router_bias"],
                                      sg=_fp8(hw, "s_gate") if n_id else None,
                                      su=_fp8(hw, "s_up") if n_id else None,
                                      sd=_fp8(hw, "s_down") if n_id else None, scale=wl.scale,
                                      limit=wl.limit, capacity=wl.capacity, norm_topk=wl.norm_topk,
                                      logits=g["logits"])
        P.assert_bf16_close(g["h_routed"][:R], r["h_routed"][:R], "h_routed (end to end)")

        def deq_diff(hq_g, sh_g, h_orc):
            hq_o, sh_o = oracle.quant_rows_e4m3(h_orc)
            return np.abs(_E4M3[hq_g] * sh_g.astype(np.float64)[:, None]
                          - _E4M3[hq_o] * sh_o.astype(np.float64)[:, None])

        for e in range(E):
            a, b = int(ro[e]), int(ro[e + 1])
            if a == b:
                continue
            wd = _fp8(hw, "w_down", e)
            extra = deq_diff(g["hq"][n_id + a:n_id + b], g["h_scale"][n_id + a:n_id + b],
                             r["h_routed"][a:b]) @ np.abs(P.weight_f64(wd)).T
            P.assert_bf16_close(g["y_routed"][a:b], r["y_routed"][a:b],
                                "y expert %d (end to end)" % e, extra=extra)
        if n_id:
            extra = deq_diff(g["hq"][:n_id], g["h_scale"][:n_id], r["h_shared"]) @ \
                np.abs(P.weight_f64(_fp8(hw, "s_down"))).T
            P.assert_bf16_close(g["y_shared"], r["y_shared"], "y_shared (end to end)", extra=extra)
        extra = P.propagated_y_diff(g["topk_w"], g["slot_to_row"], g["y_routed"], r["y_routed"],
                                    g["y_shared"], r.get("y_shared"))
        P.assert_bf16_close(g["out"], r["out"], "out (end to end)", extra=extra)


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

    for t in toks:
        t = int(t)
        x_t = as_u16(dev["x"][t:t + 1])
        q_t, s_t = oracle.quant_rows_e4m3(x_t)
        np.testing.assert_array_equal(xq_all[t:t + 1].cpu().numpy(), q_t, err_msg="xq token %d" % t)
        np.testing.assert_array_equal(sx_all[t:t + 1], s_t)
        rows = g_s2r[t * K:(t + 1) * K]
        kept = [j for j in range(K) if rows[j] >= 0]
        gy_full = np.zeros((max(R, 1), H), np.uint16)
        for j in kept:
            e, row = int(g_idx[t, j]), n_id + int(rows[j])
            gh = as_u16(h_all[row:row + 1])
            P.assert_bf16_close(gh, oracle.gateup_rows_w8a8(q_t, s_t, w("w_gate", e), w("w_up", e), wl.limit),
                                "h token %d slot %d (chained)" % (t, j))
            hq_r, sh_r = oracle.quant_rows_e4m3(gh)
            np.testing.assert_array_equal(hq_all[row:row + 1].cpu().numpy(), hq_r)
            np.testing.assert_array_equal(sh_all[row:row + 1], sh_r)
            gy = as_u16(y_all[row:row + 1])
            P.assert_bf16_close(gy, oracle.down_rows_w8a8(hq_r, sh_r, w("w_down", e)),
                                "y token %d slot %d (chained)" % (t, j))
            gy_full[rows[j]] = gy[0]
        gys = None
        if n_id:
            ghs = as_u16(h_all[t:t + 1])
            P.assert_bf16_close(ghs, oracle.gateup_rows_w8a8(q_t, s_t, w("s_gate"), w("s_up"), wl.limit),
                                "h_shared token %d (chained)" % t)
            hq_r, sh_r = oracle.quant_rows_e4m3(ghs)
            np.testing.assert_array_equal(hq_all[t:t + 1].cpu().numpy(), hq_r)
            gys = as_u16(y_all[t:t + 1])
            P.assert_bf16_close(gys, oracle.down_rows_w8a8(hq_r, sh_r, w("s_down")),
                                "y_shared token %d (chained)" % t)
        P.assert_bf16_close(as_u16(out[t:t + 1]),
                            oracle.combine(g_w[t:t + 1], g_s2r[t * K:(t + 1) * K], gy_full, gys),
                            "out token %d (chained)" % t)
