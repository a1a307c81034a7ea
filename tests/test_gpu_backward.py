"""GPU parity of the layer backward (moe_layer_backward) against the oracle, through the C ABI.

The forward runs first (moe_layer_forward, or moe_layer_forward_train, which also stores the
fp32 gate/up sums for the backward); the backward reads its workspace. Comparisons are
chained, as for the forward: every stage of the GPU backward is compared with the oracle's step
applied to the same inputs the GPU stage consumed (its own dy, dh, dg/du, d logits):
  * bf16 tensors (dy, dh, dg, du, per-row dx, dx): |gpu - oracle| <= 1e-2 |oracle| + 1e-3 rms.
  * fp32 sums of n products (routing-weight gradients over H, weight gradients over an expert's
    rows, dWr over T, dx_router over E): the accumulation bound n_steps * 2^-24 * sum|terms|,
    n_steps = n/16 + 16 for the MFMA weight gradients (16-wide partial sums), n for the others.
  * logit gradients: |gpu - oracle| <= 1e-5 * max|row| + 1e-6 |oracle| (fp32 softmax).
Integers (routing) are the forward's, already checked bit-exactly by the forward tests. The
oracle's own rounded backward from the same routing is compared end to end on the final
gradients by relative norm (<= 2e-2): a consistency check, since single bf16 rounding flips
propagate through the chain; the chained comparisons are the bar.
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
BASE = WORKLOADS["tiny_t128_h512_e32_k2"]
CASES = {
    "tiny_t128_h512_e32_k2": (BASE, 0.0),
    "aux_ragged_t130_h256_e256_k8": (Workload("ragged_t130_h256_e256_k8", T=130, H=256, E=256, K=8,
                                              I=256, scale=2.827, w_std=0.02, router_std=0.02,
                                              seed=51), 0.7),
    "no_shared_t128": (BASE.with_(name="no_shared_t128", n_shared=0, seed=52), 0.0),
    "no_renorm_t128": (BASE.with_(name="no_renorm_t128", norm_topk=False, scale=2.827, seed=53), 0.2),
    "capacity_drops_t200_e8_k2": (Workload("capacity_drops_t200_e8_k2", T=200, H=256, E=8, K=2,
                                           I=256, capacity=30, zipf=0.3, seed=54), 0.5),
    "clamp_forced_t128": (BASE.with_(name="clamp_forced_t128", x_std=30.0, seed=55), 0.0),
    "multi_tile_t300_e16_k4": (Workload("multi_tile_t300_e16_k4", T=300, H=512, E=16, K=4, I=256,
                                        scale=2.827, seed=56), 0.1),
    "bands_t3000_e4_k2": (Workload("bands_t3000_e4_k2", T=3000, H=256, E=4, K=2, I=256,
                                   scale=2.827, seed=57), 0.0),
    "dense_e1_k1_t100": (Workload("dense_e1_k1_t100", T=100, H=512, E=1, K=1, I=256, n_shared=0,
                                  seed=58), 0.0),
}

f64 = oracle.bf16_to_f64


def _u16(v):
    """float64 values that are bf16 values -> bf16 bit patterns."""
    return (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _close_sum(got, ref, abs_sum, steps, what):
    tol = steps * 2.0 ** -24 * abs_sum + 1e-30
    err = np.abs(np.asarray(got, np.float64) - ref)
    bad = err > tol
    assert not bad.any(), "%s: %d/%d out of tolerance; worst err %g tol %g" % (
        what, bad.sum(), bad.size, err[bad].max(), tol[bad][np.argmax(err[bad])])


def _dout(wl):
    gen = torch.Generator(device=DEV)
    gen.manual_seed(1000 * wl.seed + 77)
    return torch.randn(wl.T, wl.H, generator=gen, device=DEV).to(torch.bfloat16)


def _run(wl, d_aux, train=False):
    """Forward (train: moe_layer_forward_train, whose stored gate/up sums the backward then
    reads), backward, and host copies of every stage."""
    dev = generate(wl, DEV)
    s = moe.Shape.of(wl)
    layer = moe.MoELayer.from_inputs(s, dev)
    layer.forward(dev["x"], train=train)
    dout = _dout(wl)
    g = layer.backward(dout, d_aux)
    torch.cuda.synchronize()
    T, E, K, H, I = wl.T, wl.E, wl.K, wl.H, wl.I
    n_id = T if wl.n_shared else 0
    rows = n_id + T * K
    fw = dict(
        logits=layer.intermediate("logits", torch.float32, (T, E)).cpu().numpy(),
        topk_w=layer.intermediate("topk_w", torch.float32, (T, K)).cpu().numpy(),
        topk_idx=layer.intermediate("topk_idx", torch.int32, (T, K)).cpu().numpy(),
        counts=layer.intermediate("counts", torch.int32, (E,)).cpu().numpy(),
        offsets=layer.intermediate("offsets", torch.int32, (E + 1,)).cpu().numpy(),
        row_to_slot=layer.intermediate("row_to_slot", torch.int32, (T * K,)).cpu().numpy(),
        slot_to_row=layer.intermediate("slot_to_row", torch.int32, (T * K,)).cpu().numpy(),
        h=as_u16(layer.intermediate("h", torch.bfloat16, (rows, I))),
        y=as_u16(layer.intermediate("y", torch.bfloat16, (rows, H))),
    )
    bw = dict(
        dy=as_u16(layer.bwd_intermediate("dy", torch.bfloat16, (rows, H))),
        dh=as_u16(layer.bwd_intermediate("dh", torch.bfloat16, (rows, I))),
        dgu=as_u16(layer.bwd_intermediate("dgu", torch.bfloat16, (rows, 2 * I))),
        dx_rows=as_u16(layer.bwd_intermediate("dx_rows", torch.bfloat16, (rows, H))),
        dx_router=layer.bwd_intermediate("dx_router", torch.float32, (T, H)).cpu().numpy(),
    )
    gg = {k: (as_u16(v) if v.dtype == torch.bfloat16 else v.cpu().numpy()) for k, v in g.items()}
    return dev, P.host(dev), as_u16(dout), fw, bw, gg


@pytest.mark.parametrize("name", list(CASES))
def test_layer_backward_small(name):
    assert torch.cuda.is_available()
    wl, d_aux = CASES[name]
    dev, hw, dout, fw, bw, gg = _run(wl, d_aux)
    check_backward(wl, d_aux, hw, dout, fw, bw, gg)


@pytest.mark.parametrize("name", list(CASES))
def test_layer_backward_small_stored_gate_up(name):
    """The same chained checks with the gate/up sums that moe_layer_forward_train stored."""
    assert torch.cuda.is_available()
    wl, d_aux = CASES[name]
    dev, hw, dout, fw, bw, gg = _run(wl, d_aux, train=True)
    check_backward(wl, d_aux, hw, dout, fw, bw, gg)


@pytest.mark.parametrize("name", ["tiny_t128_h512_e32_k2", "aux_ragged_t130_h256_e256_k8",
                                  "capacity_drops_t200_e8_k2", "clamp_forced_t128",
                                  "dense_e1_k1_t100"])
def test_stored_gate_up_equals_recompute(name):
    """moe_layer_forward_train: its output passes the forward's parity checks against the oracle
    (it takes the tiled kernel at every shape), and the backward's gradients from its stored
    gate/up sums equal, bit for bit, the gradients of the recompute on the same forward
    workspace: the stored sums are the recompute's own."""
    assert torch.cuda.is_available()
    wl, d_aux = CASES[name]
    dev = generate(wl, DEV)
    hw = P.host(dev)
    g, layer, _ = P.run_layer_gpu(wl, dev, train=True)
    P.compare_layer(wl, hw, g, P.oracle_same_logits(wl, hw, g["logits"]), train=True)
    assert layer._gu is not None
    # the stored sums against their definition g = x Wg^T, u = x Wu^T (fp64), within the bound
    # of 16-wide fp32 partial sums over H
    gu = layer.gu.cpu().numpy()
    n_id, I, K = (wl.T if wl.n_shared else 0), wl.I, wl.K
    x = f64(hw["x"])
    groups = [(np.arange(n_id), np.arange(wl.T), P.shared_weights(hw))] if n_id else []
    off, r2s = g["offsets"], g["row_to_slot"]
    for e in range(wl.E):
        a, b = int(off[e]), int(off[e + 1])
        if a < b:
            groups.append((n_id + np.arange(a, b), r2s[a:b] // K, P.routed_weights(hw, e)))
    for rows, tok, (wg, wu, _) in groups:
        for w, cols, what in ((wg, slice(0, I), "g"), (wu, slice(I, 2 * I), "u")):
            wf = f64(w)
            _close_sum(gu[rows, cols], x[tok] @ wf.T, np.abs(x[tok]) @ np.abs(wf).T,
                       wl.H / 16 + 16, "stored %s" % what)
    dout = _dout(wl)
    rows = wl.T * wl.K + (wl.T if wl.n_shared else 0)
    host = lambda gr: {k: (as_u16(v) if v.dtype == torch.bfloat16 else v.cpu().numpy())
                       for k, v in gr.items()}
    stored = host(layer.backward(dout, d_aux))
    dgu_stored = as_u16(layer.bwd_intermediate("dgu", torch.bfloat16, (rows, 2 * wl.I)))
    layer._gu = None  # the same workspace, g and u recomputed
    recomputed = host(layer.backward(dout, d_aux))
    dgu_re = as_u16(layer.bwd_intermediate("dgu", torch.bfloat16, (rows, 2 * wl.I)))
    R = int(g["offsets"][-1]) + (wl.T if wl.n_shared else 0)
    np.testing.assert_array_equal(dgu_stored[:R], dgu_re[:R], err_msg="dg | du")
    for k in stored:
        np.testing.assert_array_equal(stored[k], recomputed[k], err_msg=k)


@pytest.mark.timeout(600)
def test_stored_gate_up_equals_recompute_full_size():
    """hy4_prefill_t8192 at full size: the backward from moe_layer_forward_train's stored gate/up
    sums equals, bit for bit, the backward that recomputes them on the same forward workspace,
    and the training forward's output equals the plain forward's (both take the tiled kernel at
    this shape)."""
    assert torch.cuda.is_available()
    wl = WORKLOADS["hy4_prefill_t8192"]
    print("\n[stored gate/up, full size] %s T=%d" % (wl.name, wl.T), flush=True)
    dev = generate(wl, DEV)
    layer = moe.MoELayer.from_inputs(moe.Shape.of(wl), dev)
    plain = as_u16(layer.forward(dev["x"]))
    trained = as_u16(layer.forward(dev["x"], train=True))
    np.testing.assert_array_equal(trained, plain, err_msg="out")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(4243)
    dout = torch.randn(wl.T, wl.H, generator=gen, device=DEV).to(torch.bfloat16)
    bits = lambda v: v.view(torch.int16 if v.dtype == torch.bfloat16 else torch.int32)
    stored = layer.backward(dout, 0.01)
    layer._gu = None
    recomputed = layer.backward(dout, 0.01)
    for k in stored:  # bit patterns compared on the device (the weight gradients are 39 GB)
        assert torch.equal(bits(stored[k]), bits(recomputed[k])), k


def test_forward_train_rejects_null_gate_up():
    assert torch.cuda.is_available()
    wl = BASE
    dev = generate(wl, DEV)
    s = moe.Shape.of(wl)
    layer = moe.MoELayer.from_inputs(s, dev)
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=DEV)
    wr, b, wg, wu, wd, sg, su, sd = layer.w
    with pytest.raises(RuntimeError):
        moe.moe_layer_forward_train(s, dev["x"], wr, b, wg, wu, wd, sg, su, sd, out, None, layer.ws)


def check_backward(wl, d_aux, hw, dout, fw, bw, gg):
    T, E, K, H, I = wl.T, wl.E, wl.K, wl.H, wl.I
    n_id = T if wl.n_shared else 0
    off = fw["offsets"]
    R = int(off[-1])
    x = hw["x"]
    r2s = fw["row_to_slot"]

    # combine backward: routed dy rows and routing-weight gradients
    y_r = f64(fw["y"][n_id:n_id + R])
    dy_o, dw_o = oracle.combine_bwd(fw["topk_w"], fw["slot_to_row"], y_r, dout)
    P.assert_bf16_close(bw["dy"][n_id:n_id + R], _u16(dy_o), "dy (routed rows)")
    if n_id:
        np.testing.assert_array_equal(bw["dy"][:T], dout)
    absw = np.zeros((T, K))
    s2r = fw["slot_to_row"].reshape(T, K)
    for j in range(K):
        kept = s2r[:, j] >= 0
        absw[kept, j] = np.sum(np.abs(f64(dout[kept])) * np.abs(y_r[s2r[kept, j]]), axis=1)
    _close_sum(gg["d_topk_w"], dw_o, absw, H, "d_topk_w")

    # per group: dh, dg/du, per-row dx, weight gradients
    groups = [("shared", 0, n_id, hw["s_gate"], hw["s_up"], hw["s_down"], "d_s")] if n_id else []
    for e in range(E):
        groups.append(("expert %d" % e, n_id + off[e], n_id + off[e + 1], hw["w_gate"][e],
                       hw["w_up"][e], hw["w_down"][e], e))
    for label, a, b, wg, wu, wd, key in groups:
        gwd = gg["d_s_down"] if key == "d_s" else gg["d_w_down"][key]
        gwg = gg["d_s_gate"] if key == "d_s" else gg["d_w_gate"][key]
        gwu = gg["d_s_up"] if key == "d_s" else gg["d_w_up"][key]
        n = b - a
        if n == 0:
            assert not gwd.any() and not gwg.any() and not gwu.any(), label + ": no rows, zero grads"
            continue
        rows_x = x[np.arange(a, b)] if key == "d_s" else x[r2s[a - n_id:b - n_id] // K]
        dy_g = f64(bw["dy"][a:b])
        dh_o = oracle.down_bwd_rows(dy_g, wd)
        P.assert_bf16_close(bw["dh"][a:b], _u16(dh_o), "dh " + label)
        dh_g = f64(bw["dh"][a:b])
        dg_o, du_o = oracle.swiglu_bwd_rows(rows_x, wg, wu, dh_g, wl.limit)
        P.assert_bf16_close(bw["dgu"][a:b, :I], _u16(dg_o), "dg " + label)
        P.assert_bf16_close(bw["dgu"][a:b, I:], _u16(du_o), "du " + label)
        dg_g, du_g = f64(bw["dgu"][a:b, :I]), f64(bw["dgu"][a:b, I:])
        dx_o = oracle.gateup_dgrad_rows(dg_g, du_g, wg, wu)
        P.assert_bf16_close(bw["dx_rows"][a:b], _u16(dx_o), "dx rows " + label)
        h_g, xf = f64(fw["h"][a:b]), f64(rows_x)
        steps = n / 16 + 16
        _close_sum(gwd, oracle.wgrad(dy_g, h_g), oracle.wgrad(np.abs(dy_g), np.abs(h_g)), steps,
                   "dWd " + label)
        _close_sum(gwg, oracle.wgrad(dg_g, xf), oracle.wgrad(np.abs(dg_g), np.abs(xf)), steps,
                   "dWg " + label)
        _close_sum(gwu, oracle.wgrad(du_g, xf), oracle.wgrad(np.abs(du_g), np.abs(xf)), steps,
                   "dWu " + label)

    # router: logit gradients from the GPU's routing-weight gradients, then dWr and dx_router
    dl_o = oracle.router_bwd(fw["logits"], fw["topk_idx"], gg["d_topk_w"], wl.scale, wl.norm_topk,
                             d_aux)
    # fp32 rounding of dl_e = p_e (dp_e - sum_k p_k dp_k) is relative to the terms of dp, not to
    # dl (they cancel when the selected weights' gradients are close): bound the terms by A
    lg = fw["logits"].astype(np.float64)
    pr = np.exp(lg - lg.max(axis=1, keepdims=True))
    pr /= pr.sum(axis=1, keepdims=True)
    dwg = gg["d_topk_w"].astype(np.float64)
    if wl.norm_topk:
        pk = np.take_along_axis(pr, fw["topk_idx"].astype(np.int64), axis=1)
        Z = pk.sum(axis=1, keepdims=True)
        A = wl.scale * (np.abs(dwg) / Z + np.abs((dwg * pk).sum(axis=1, keepdims=True)) / Z ** 2)
    else:
        A = wl.scale * np.abs(dwg)
    A = A.max(axis=1, keepdims=True) + abs(d_aux) * E / T
    tol = 1e-5 * pr * A + 1e-6 * np.abs(dl_o) + 1e-12
    err = np.abs(gg["d_logits"] - dl_o)
    assert np.all(err <= tol), ("d_logits", err.max(), int(np.sum(err > tol)))
    dl_g = gg["d_logits"].astype(np.float64)
    xf = f64(x)
    _close_sum(gg["d_w_router"], oracle.wgrad(dl_g, xf), oracle.wgrad(np.abs(dl_g), np.abs(xf)),
               T + 16, "dWr")
    wr = f64(hw["w_router"])
    _close_sum(bw["dx_router"], dl_g @ wr, np.abs(dl_g) @ np.abs(wr), E + 16, "dx_router")

    # dx: the token's rows in slot order, the shared row, the router term
    acc = np.zeros((T, H))
    dxr = f64(bw["dx_rows"])
    for j in range(K):
        kept = s2r[:, j] >= 0
        acc[kept] += dxr[n_id + s2r[kept, j]]
    if n_id:
        acc += dxr[:T]
    acc += bw["dx_router"].astype(np.float64)
    P.assert_bf16_close(gg["d_x"], oracle.bf16_round_array(acc), "dx")

    # end to end: the oracle's own rounded backward from the same routing
    fwd = {k: fw[k] for k in ("logits", "topk_idx", "topk_w", "counts", "offsets", "row_to_slot",
                              "slot_to_row")}
    r = oracle.layer_backward(x, hw["w_router"], hw["w_gate"], hw["w_up"], hw["w_down"], fwd, dout,
                              sg=hw["s_gate"], su=hw["s_up"], sd=hw["s_down"], scale=wl.scale,
                              limit=wl.limit, norm_topk=wl.norm_topk, d_aux=d_aux)
    pairs = [("dx", f64(gg["d_x"]), r["dx"]), ("d_wr", gg["d_w_router"], r["d_wr"]),
             ("d_wg", gg["d_w_gate"], r["d_wg"]), ("d_wu", gg["d_w_up"], r["d_wu"]),
             ("d_wd", gg["d_w_down"], r["d_wd"])]
    if n_id:
        pairs += [("d_sg", gg["d_s_gate"], r["d_sg"]), ("d_su", gg["d_s_up"], r["d_su"]),
                  ("d_sd", gg["d_s_down"], r["d_sd"])]
    for k, a_, b_ in pairs:
        rel = np.linalg.norm(np.asarray(a_, np.float64) - b_) / (np.linalg.norm(b_) + 1e-300)
        assert rel <= 2e-2, (k, rel)


def test_layer_backward_is_deterministic():
    assert torch.cuda.is_available()
    wl, d_aux = CASES["multi_tile_t300_e16_k4"]
    outs = [_run(wl, d_aux)[5] for _ in range(2)]
    for k in outs[0]:
        np.testing.assert_array_equal(outs[0][k], outs[1][k], err_msg=k)


# ----------------------------------------------------------------------------- full sizes, sampled
FULL = ["hy4_decode_t64", "hy4_prefill_t8192"]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", FULL)
def test_layer_backward_full_size_sampled(name):
    """Full workload shapes: chained checks on sampled tokens (their routing-weight gradients,
    every row stage and dx), sampled weight-gradient blocks of sampled experts, and every logit
    gradient."""
    assert torch.cuda.is_available()
    wl = WORKLOADS[name]
    d_aux = 0.01
    print("\n[backward full-size] %s T=%d" % (name, wl.T), flush=True)
    dev = generate(wl, DEV)
    s = moe.Shape.of(wl)
    layer = moe.MoELayer.from_inputs(s, dev)
    layer.forward(dev["x"])
    gen = torch.Generator(device=DEV)
    gen.manual_seed(4242)
    dout_d = torch.randn(wl.T, wl.H, generator=gen, device=DEV).to(torch.bfloat16)
    g = layer.backward(dout_d, d_aux)
    torch.cuda.synchronize()
    T, E, K, H, I = wl.T, wl.E, wl.K, wl.H, wl.I
    n_id = T
    rows = n_id + T * K
    inter = lambda nm, dt, shp: layer.intermediate(nm, dt, shp)
    binter = lambda nm, dt, shp: layer.bwd_intermediate(nm, dt, shp)
    logits = inter("logits", torch.float32, (T, E)).cpu().numpy()
    topk_w = inter("topk_w", torch.float32, (T, K)).cpu().numpy()
    topk_idx = inter("topk_idx", torch.int32, (T, K)).cpu().numpy()
    off = inter("offsets", torch.int32, (E + 1,)).cpu().numpy()
    r2s = inter("row_to_slot", torch.int32, (T * K,)).cpu().numpy()
    s2r = inter("slot_to_row", torch.int32, (T * K,)).cpu().numpy().reshape(T, K)
    h_all, y_all = inter("h", torch.bfloat16, (rows, I)), inter("y", torch.bfloat16, (rows, H))
    dy_all, dh_all = binter("dy", torch.bfloat16, (rows, H)), binter("dh", torch.bfloat16, (rows, I))
    dgu_all, dxr_all = binter("dgu", torch.bfloat16, (rows, 2 * I)), binter("dx_rows", torch.bfloat16, (rows, H))
    dx_router = binter("dx_router", torch.float32, (T, H))
    take = lambda t_, idx: as_u16(t_[torch.from_numpy(np.asarray(idx, np.int64)).to(DEV)])
    wgt = lambda nm, e=None: as_u16(dev[nm] if e is None else dev[nm][e])

    rng = np.random.default_rng(9)
    toks = np.sort(rng.choice(T, 4, replace=False))
    dout = take(dout_d, toks)
    x_s = take(dev["x"], toks)
    for i, t in enumerate(toks):
        kept = [j for j in range(K) if s2r[t, j] >= 0]
        lrows = n_id + s2r[t, kept]
        y_rows = f64(take(y_all, lrows))
        s2r_local = np.full((1, K), -1, np.int32)
        s2r_local[0, kept] = np.arange(len(kept))
        dy_o, dw_o = oracle.combine_bwd(topk_w[t:t + 1], s2r_local, y_rows, dout[i:i + 1])
        dy_g = take(dy_all, lrows)
        P.assert_bf16_close(dy_g, _u16(dy_o), "dy token %d" % t)
        absw = np.array([np.sum(np.abs(f64(dout[i])) * np.abs(y_rows[n])) for n in range(len(kept))])
        _close_sum(g["d_topk_w"][t, kept].cpu().numpy(), dw_o[0, kept], absw, H, "d_topk_w token %d" % t)
        # each routed row and the shared row: dh, dg/du, dx rows
        row_list = [(lr, int(topk_idx[t, j]), "routed") for lr, j in zip(lrows, kept)] + [(t, -1, "shared")]
        for lr, e, kind in row_list:
            wg, wu, wd = ((wgt("s_gate"), wgt("s_up"), wgt("s_down")) if e < 0 else
                          (wgt("w_gate", e), wgt("w_up", e), wgt("w_down", e)))
            dy1 = f64(take(dy_all, [lr]))
            P.assert_bf16_close(take(dh_all, [lr]), _u16(oracle.down_bwd_rows(dy1, wd)), "dh %s %d" % (kind, t))
            dh1 = f64(take(dh_all, [lr]))
            dg_o, du_o = oracle.swiglu_bwd_rows(x_s[i:i + 1], wg, wu, dh1, wl.limit)
            dgu1 = take(dgu_all, [lr])
            P.assert_bf16_close(dgu1[:, :I], _u16(dg_o), "dg %s %d" % (kind, t))
            P.assert_bf16_close(dgu1[:, I:], _u16(du_o), "du %s %d" % (kind, t))
            dx_o = oracle.gateup_dgrad_rows(f64(dgu1[:, :I]), f64(dgu1[:, I:]), wg, wu)
            P.assert_bf16_close(take(dxr_all, [lr]), _u16(dx_o), "dx rows %s %d" % (kind, t))
        # dx of the token
        acc = f64(take(dxr_all, lrows)).sum(axis=0) + f64(take(dxr_all, [t]))[0]
        dr = dx_router[int(t)].cpu().numpy().astype(np.float64)
        P.assert_bf16_close(take(g["d_x"], [t]), oracle.bf16_round_array((acc + dr)[None]), "dx token %d" % t)
    # every logit gradient, from the GPU's routing-weight gradients
    dl_o = oracle.router_bwd(logits, topk_idx, g["d_topk_w"].cpu().numpy(), wl.scale, wl.norm_topk, d_aux)
    dl_g = g["d_logits"].cpu().numpy()
    lg = logits.astype(np.float64)
    pr = np.exp(lg - lg.max(axis=1, keepdims=True))
    pr /= pr.sum(axis=1, keepdims=True)
    dwg = g["d_topk_w"].cpu().numpy().astype(np.float64)
    pk = np.take_along_axis(pr, topk_idx.astype(np.int64), axis=1)
    Z = pk.sum(axis=1, keepdims=True)
    A = (wl.scale * (np.abs(dwg) / Z + np.abs((dwg * pk).sum(axis=1, keepdims=True)) / Z ** 2)).max(axis=1, keepdims=True)
    tol = 1e-5 * pr * (A + d_aux * E / T) + 1e-6 * np.abs(dl_o) + 1e-12
    assert np.all(np.abs(dl_g - dl_o) <= tol), "d_logits"
    # weight-gradient blocks: 8 x 8 entries of the busiest and one other expert, the shared expert
    cs, is_ = np.sort(rng.choice(H, 8, replace=False)), np.sort(rng.choice(I, 8, replace=False))
    busiest = int(np.argmax(np.diff(off)))
    for e in (busiest, int(rng.integers(E)), -1):
        a, b = (0, T) if e < 0 else (n_id + off[e], n_id + off[e + 1])
        if b == a:
            continue
        rws = np.arange(a, b)
        dyb = f64(take(dy_all, rws))[:, cs]
        hb = f64(take(h_all, rws))[:, is_]
        dgb = f64(take(dgu_all, rws))[:, is_]
        xrows = rws if e < 0 else r2s[rws - n_id] // K
        xb = f64(take(dev["x"], xrows))[:, cs]
        n = b - a
        gd = (g["d_s_down"] if e < 0 else g["d_w_down"][e]).cpu().numpy()[np.ix_(cs, is_)]
        gg_ = (g["d_s_gate"] if e < 0 else g["d_w_gate"][e]).cpu().numpy()[np.ix_(is_, cs)]
        _close_sum(gd, oracle.wgrad(dyb, hb), oracle.wgrad(np.abs(dyb), np.abs(hb)), n / 16 + 16, "dWd block %d" % e)
        _close_sum(gg_, oracle.wgrad(dgb, xb), oracle.wgrad(np.abs(dgb), np.abs(xb)), n / 16 + 16, "dWg block %d" % e)
    # router weight gradient columns and the router term of sampled tokens
    xc = f64(as_u16(dev["x"]))[:, cs]
    _close_sum(g["d_w_router"].cpu().numpy()[:, cs], oracle.wgrad(dl_g.astype(np.float64), xc),
               oracle.wgrad(np.abs(dl_g.astype(np.float64)), np.abs(xc)), T + 16, "dWr columns")
    wr = f64(wgt("w_router"))
    dls = dl_g[toks].astype(np.float64)
    _close_sum(dx_router[torch.from_numpy(toks).to(DEV)].cpu().numpy(), dls @ wr, np.abs(dls) @ np.abs(wr), E + 16,
               "dx_router tokens")
