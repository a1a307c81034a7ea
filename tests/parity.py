"""Helpers shared by the GPU parity tests: tolerance checks and GPU/oracle runners.

Tolerances (stated where the pages and the layer's definition leave them open):
  * bf16 tensors h, y, y_shared, out: |gpu - oracle| <= 1e-2*|oracle| + 1e-3*rms(oracle),
    element-wise, rms over the whole compared tensor.
  * Chained checks (the bar): every bf16 tensor is compared with the oracle applied to the SAME
    bf16 inputs the GPU stage consumed (h from x; y from the GPU's h; out from the GPU's y and
    y_shared), with the bare tolerance above.
  * Independent checks (consistency): the oracle's own chain from x. An element that lies on a
    bf16 rounding boundary can round one ulp apart on the two sides (fp32 vs fp64 accumulation),
    and the next linear map carries that difference on. So the bound for y adds
    sum_i |h_gpu - h_oracle|_i * |Wd[c,i]|, and the bound for out adds
    sum_j |w_j| * |y_gpu - y_oracle|_j + |y_shared_gpu - y_shared_oracle|: the measured upstream
    differences propagated through the layer's own maps.
  * fp32 router logits: |gpu - oracle| <= 1e-4 * rms(oracle) + 1e-5 * |oracle| (fp32
    accumulation over H terms against a double sum).
  * fp32 routing weights: |gpu - oracle| <= 1e-5 * routed_scaling.
  * Integers (indices, counts, offsets, permutation): bit-exact.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import sparse_moe_layer_softmax_amd as moe
from sparse_moe_layer_softmax_amd.workloads import as_u16

f64 = oracle.bf16_to_f64


def ulp_bf16(u16: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at each element (2^(e-7), fixed below the smallest normal)."""
    e = (np.asarray(u16, np.uint16).astype(np.int64) >> 7) & 0xFF
    return np.ldexp(1.0, np.maximum(e, 1) - 127 - 7)


def bf16_close(got_u16, ref_u16, extra=None):
    g, r = f64(got_u16), f64(ref_u16)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    tol = 1e-2 * np.abs(r) + 1e-3 * rms
    if extra is not None:
        tol = tol + extra
    ok = np.abs(g - r) <= tol
    return ok, g, r, tol


def assert_bf16_close(got_u16, ref_u16, what, extra=None):
    got_u16 = np.asarray(got_u16)
    ref_u16 = np.asarray(ref_u16)
    assert got_u16.shape == ref_u16.shape, (what, got_u16.shape, ref_u16.shape)
    ok, g, r, tol = bf16_close(got_u16, ref_u16, extra)
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError("%s: %d/%d elements out of tolerance; first at %s: gpu=%r oracle=%r tol=%r"
                             % (what, len(bad), ok.size, i, g[i], r[i], tol[i]))


def assert_logits_close(got, ref, what="logits"):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    tol = 1e-4 * rms + 1e-5 * np.abs(ref)
    err = np.abs(got - ref)
    assert np.all(err <= tol), "%s: max err %g (tol at worst %g)" % (what, err.max(), tol.flat[err.argmax()])


def margin_ok(probs: np.ndarray, K: int, thresh: float = 1e-4) -> np.ndarray:
    """Tokens whose k-th / (k+1)-th largest probabilities differ by at least `thresh`."""
    E = probs.shape[1]
    if K >= E:
        return np.ones(probs.shape[0], bool)
    srt = -np.sort(-probs, axis=1)
    return (srt[:, K - 1] - srt[:, K]) >= thresh


_E4M3 = None


def weight_f64(w) -> np.ndarray:
    """Float64 values of a weight matrix: bf16 bit patterns, or an oracle.Fp8 (scale * e4m3)."""
    global _E4M3
    if isinstance(w, oracle.Fp8):
        if _E4M3 is None:
            _E4M3 = np.array([oracle.double_from_e4m3(c) for c in range(256)])
        return _E4M3[w.q] * w.scale.astype(np.float64)[..., None]
    return f64(w)


def is_fp8(hw: dict) -> bool:
    return hw["w_gate"].dtype == np.uint8


def routed_weights(hw: dict, e: int):
    """(gate, up, down) of routed expert e in the oracle's form (bf16 arrays or oracle.Fp8)."""
    names = ("w_gate", "w_up", "w_down")
    if is_fp8(hw):
        return tuple(oracle.Fp8(hw[n][e], hw[n + "_scale"][e]) for n in names)
    return tuple(hw[n][e] for n in names)


def shared_weights(hw: dict):
    names = ("s_gate", "s_up", "s_down")
    if hw["s_gate"] is None:
        return None, None, None
    if is_fp8(hw):
        return tuple(oracle.Fp8(hw[n], hw[n + "_scale"]) for n in names)
    return tuple(hw[n] for n in names)


def all_routed(hw: dict):
    names = ("w_gate", "w_up", "w_down")
    if is_fp8(hw):
        return tuple(oracle.Fp8(hw[n], hw[n + "_scale"]) for n in names)
    return tuple(hw[n] for n in names)


def ffn_rows(x_rows, w3, limit):
    """Oracle expert FFN of the given rows: (h, y)."""
    if isinstance(w3[0], oracle.Fp8):
        return oracle.expert_ffn_rows_fp8(x_rows, *w3, limit)
    return oracle.expert_ffn_rows(x_rows, *w3, limit)


def down_rows(h, wd):
    if isinstance(wd, oracle.Fp8):
        return oracle.down_rows_fp8(h, wd)
    return oracle.down_rows(h, wd)


def propagated_h_diff(h_gpu_u16, h_orc_u16, wd):
    """sum_i |h_gpu - h_oracle|_i * |Wd[c, i]| for each row and output column c."""
    dh = np.abs(f64(h_gpu_u16) - f64(h_orc_u16))
    return dh @ np.abs(weight_f64(wd)).T


def propagated_y_diff(topk_w, slot_to_row, y_gpu_u16, y_orc_u16, ys_gpu_u16=None, ys_orc_u16=None):
    """sum over kept slots of |w_j| * |y_gpu - y_oracle| (row of slot j), plus the shared row's."""
    T, K = topk_w.shape
    H = y_gpu_u16.shape[1]
    acc = np.zeros((T, H))
    dy = np.abs(f64(y_gpu_u16) - f64(y_orc_u16))
    for j in range(K):
        rows = slot_to_row.reshape(T, K)[:, j]
        kept = rows >= 0
        acc[kept] += np.abs(topk_w[kept, j:j + 1].astype(np.float64)) * dy[rows[kept]]
    if ys_gpu_u16 is not None:
        acc += np.abs(f64(ys_gpu_u16) - f64(ys_orc_u16))
    return acc


def host(wts: dict) -> dict:
    """Host copies (uint16 / float32 numpy) of a generated input dict."""
    out = {}
    for k, v in wts.items():
        if v is None or not isinstance(v, torch.Tensor):
            out[k] = v
        elif v.dtype == torch.bfloat16:
            out[k] = as_u16(v)
        else:
            out[k] = v.detach().cpu().numpy()
    return out


def run_layer_gpu(wl, dev: dict, train: bool = False):
    """moe_layer_forward (train: moe_layer_forward_train) on the GPU; returns host copies of out
    and every intermediate."""
    shape = moe.Shape.of(wl)
    layer = moe.MoELayer.from_inputs(shape, dev)
    out = layer.forward(dev["x"], train=train)
    torch.cuda.synchronize()
    T, E, K, H, I = wl.T, wl.E, wl.K, wl.H, wl.I
    n_id = T if wl.n_shared else 0
    rows = n_id + T * K
    g = dict(
        out=as_u16(out),
        logits=layer.intermediate("logits", torch.float32, (T, E)).cpu().numpy(),
        topk_w=layer.intermediate("topk_w", torch.float32, (T, K)).cpu().numpy(),
        topk_idx=layer.intermediate("topk_idx", torch.int32, (T, K)).cpu().numpy(),
        counts=layer.intermediate("counts", torch.int32, (E,)).cpu().numpy(),
        offsets=layer.intermediate("offsets", torch.int32, (E + 1,)).cpu().numpy(),
        row_to_slot=layer.intermediate("row_to_slot", torch.int32, (T * K,)).cpu().numpy(),
        slot_to_row=layer.intermediate("slot_to_row", torch.int32, (T * K,)).cpu().numpy(),
    )
    h = layer.intermediate("h", torch.int16, (rows, I)).cpu().numpy().view(np.uint16)
    y = layer.intermediate("y", torch.int16, (rows, H)).cpu().numpy().view(np.uint16)
    g["h_shared"], g["h_routed"] = (h[:n_id], h[n_id:]) if n_id else (None, h)
    g["y_shared"], g["y_routed"] = (y[:n_id], y[n_id:]) if n_id else (None, y)
    if layer.act_fp8:  # the quantised activations (W8A8)
        g["xq"] = layer.intermediate("xq", torch.uint8, (T, H)).cpu().numpy()
        g["x_scale"] = layer.intermediate("x_scale", torch.float32, (T,)).cpu().numpy()
        g["hq"] = layer.intermediate("hq", torch.uint8, (rows, I)).cpu().numpy()
        g["h_scale"] = layer.intermediate("h_scale", torch.float32, (rows,)).cpu().numpy()
    return g, layer, out


def oracle_same_logits(wl, hw: dict, logits: np.ndarray) -> dict:
    """Oracle steps 2-9 from the given fp32 logits (router projection skipped)."""
    fwd = oracle.layer_forward_fp8 if is_fp8(hw) else oracle.layer_forward
    sg, su, sd = shared_weights(hw)
    return fwd(hw["x"], hw["w_router"], *all_routed(hw), wl.K, bias=hw["router_bias"], sg=sg, su=su,
               sd=sd, scale=wl.scale, limit=wl.limit, capacity=wl.capacity,
               norm_topk=wl.norm_topk, logits=logits)


def compare_layer(wl, hw: dict, g: dict, r: dict, check_routing_bits: bool = True):
    """Element-wise comparison of a GPU layer run with the oracle run from the same logits."""
    if check_routing_bits:
        np.testing.assert_array_equal(g["topk_idx"], r["topk_idx"], err_msg="topk_idx")
        np.testing.assert_array_equal(g["counts"], r["counts"], err_msg="counts")
        np.testing.assert_array_equal(g["offsets"], r["offsets"], err_msg="offsets")
        np.testing.assert_array_equal(g["row_to_slot"], r["row_to_slot"], err_msg="row_to_slot")
        np.testing.assert_array_equal(g["slot_to_row"], r["slot_to_row"], err_msg="slot_to_row")
    np.testing.assert_allclose(g["topk_w"], r["topk_w"], rtol=0, atol=1e-5 * max(wl.scale, 1e-30))
    R = int(r["offsets"][-1])
    off = r["offsets"]
    # h from x: both sides start from the same bf16 x
    assert_bf16_close(g["h_routed"][:R], r["h_routed"][:R], "h_routed")
    # y, chained (oracle down projection of the GPU's h) and independent (oracle's own h)
    for e in range(wl.E):
        a, b = int(off[e]), int(off[e + 1])
        if a == b:
            continue
        wd = routed_weights(hw, e)[2]
        assert_bf16_close(g["y_routed"][a:b], down_rows(g["h_routed"][a:b], wd),
                          "y_routed expert %d (chained)" % e)
        assert_bf16_close(g["y_routed"][a:b], r["y_routed"][a:b], "y_routed expert %d (end to end)" % e,
                          extra=propagated_h_diff(g["h_routed"][a:b], r["h_routed"][a:b], wd))
    if wl.n_shared:
        assert_bf16_close(g["h_shared"], r["h_shared"], "h_shared")
        sd = shared_weights(hw)[2]
        assert_bf16_close(g["y_shared"], down_rows(g["h_shared"], sd), "y_shared (chained)")
        assert_bf16_close(g["y_shared"], r["y_shared"], "y_shared (end to end)",
                          extra=propagated_h_diff(g["h_shared"], r["h_shared"], sd))
    # out, chained: the oracle's combine of the GPU's own rows, bare tolerance
    chained = oracle.combine(g["topk_w"], g["slot_to_row"], g["y_routed"], g["y_shared"])
    assert_bf16_close(g["out"], chained, "out (chained)")
    # out, independent: the oracle's own rows plus the propagated y differences
    extra = propagated_y_diff(r["topk_w"], r["slot_to_row"], g["y_routed"], r["y_routed"],
                              g.get("y_shared"), r.get("y_shared"))
    assert_bf16_close(g["out"], r["out"], "out (end to end)", extra=extra)
