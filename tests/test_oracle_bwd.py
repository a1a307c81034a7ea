"""Pins of the oracle's backward pass (CPU only).

The pages print no backward; the oracle differentiates its own forward. In exact mode (no bf16
rounding points) every gradient it returns must equal PyTorch's automatic differentiation of a
float64 implementation of the same forward: the same fixed top-k choice and capacity drops, the
renormalisation and routed scaling, the clamped SwiGLU experts, the shared expert, and the
load-balancing loss term. The rounded mode (the GPU's bf16 storage points) must stay within bf16
error of the exact one, and its stored tensors must be bf16 values.
"""
import numpy as np
import pytest
import torch

from tests.test_oracle_pins import _rand_bf16


def _t(u16):
    return torch.from_numpy((np.asarray(u16, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64))


def _case(seed, T=24, H=32, E=8, K=3, I=48, shared=True, w_std=0.3, capacity=0):
    rng = np.random.default_rng(seed)
    d = dict(x=_rand_bf16(rng, (T, H), 1.0), wr=_rand_bf16(rng, (E, H), 0.2),
             wg=_rand_bf16(rng, (E, I, H), w_std), wu=_rand_bf16(rng, (E, I, H), w_std),
             wd=_rand_bf16(rng, (E, H, I), 0.1), dout=_rand_bf16(rng, (T, H), 1.0))
    if shared:
        d.update(sg=_rand_bf16(rng, (I, H), w_std), su=_rand_bf16(rng, (I, H), w_std),
                 sd=_rand_bf16(rng, (H, I), 0.1))
    else:
        d.update(sg=None, su=None, sd=None)
    d["bias"] = (0.5 * np.log(1.0 / (np.arange(E) + 1.0))).astype(np.float32)
    return d


def _autograd(d, fwd, K, scale, limit, norm_topk, d_aux):
    """Gradients of sum(out * dout) + d_aux * E * sum_e P_e f_e by torch autograd, float64."""
    x = _t(d["x"]).requires_grad_()
    wr = _t(d["wr"]).requires_grad_()
    wg, wu, wd = (_t(d[k]).requires_grad_() for k in ("wg", "wu", "wd"))
    T, H = x.shape
    E = wr.shape[0]
    lg = x @ wr.T + torch.from_numpy(d["bias"].astype(np.float64))
    l32 = torch.from_numpy(fwd["logits"].astype(np.float64))
    lg = lg + (l32 - lg).detach()  # the value of the forward's fp32 logits, the gradient of x Wr^T
    lg.retain_grad()
    p = torch.softmax(lg, dim=-1)
    idx = torch.from_numpy(fwd["topk_idx"].astype(np.int64))
    pk = p.gather(1, idx)
    w = scale * pk / pk.sum(1, keepdim=True) if norm_topk else scale * pk
    w.retain_grad()
    # the combine uses the forward's fp32 routing weights (their value; the gradient is w's)
    w32 = torch.from_numpy(fwd["topk_w"].astype(np.float64))
    wv = w + (w32 - w).detach()

    def ffn(xr, g_, u_, d_):
        g, u = xr @ g_.T, xr @ u_.T
        if limit > 0:
            g, u = g.clamp(-limit, limit), u.clamp(-limit, limit)
        return (torch.nn.functional.silu(g) * u) @ d_.T

    s2r = fwd["slot_to_row"].reshape(T, K)
    rows = []
    for t in range(T):
        acc = torch.zeros(H, dtype=torch.float64)
        for j in range(K):
            if s2r[t, j] < 0:
                continue
            e = int(idx[t, j])
            acc = acc + wv[t, j] * ffn(x[t:t + 1], wg[e], wu[e], wd[e])[0]
        rows.append(acc)
    out = torch.stack(rows)
    grads = {}
    if d["sg"] is not None:
        sg, su, sd = (_t(d[k]).requires_grad_() for k in ("sg", "su", "sd"))
        out = out + ffn(x, sg, su, sd)
    f = torch.bincount(idx.reshape(-1), minlength=E).to(torch.float64) / (T * K)
    aux = E * (p.mean(0) * f).sum()
    loss = (out * _t(d["dout"])).sum() + d_aux * aux
    loss.backward()
    grads.update(dx=x.grad, d_wr=wr.grad, d_wg=wg.grad, d_wu=wu.grad, d_wd=wd.grad,
                 d_logits=lg.grad, d_topk_w=w.grad)
    if d["sg"] is not None:
        grads.update(d_sg=sg.grad, d_su=su.grad, d_sd=sd.grad)
    return {k: v.numpy() for k, v in grads.items()}


CASES = [
    dict(seed=1, scale=2.827, limit=10.0, norm_topk=True, d_aux=0.3, capacity=0, shared=True,
         w_std=2.0),
    dict(seed=2, scale=1.0, limit=0.0, norm_topk=False, d_aux=0.0, capacity=0, shared=False,
         w_std=0.3),
    dict(seed=3, scale=2.827, limit=2.0, norm_topk=True, d_aux=1.5, capacity=7, shared=True,
         w_std=0.3),
]


@pytest.mark.parametrize("c", CASES, ids=lambda c: "seed%d" % c["seed"])
def test_exact_backward_equals_autograd(orc, c):
    K = 3
    d = _case(c["seed"], shared=c["shared"], w_std=c["w_std"])
    fwd = orc.layer_forward(d["x"], d["wr"], d["wg"], d["wu"], d["wd"], K, bias=d["bias"],
                            sg=d["sg"], su=d["su"], sd=d["sd"], scale=c["scale"],
                            limit=c["limit"], capacity=c["capacity"], norm_topk=c["norm_topk"])
    if c["capacity"]:
        assert (fwd["slot_to_row"] < 0).any(), "the capacity case must drop slots"
    if c["limit"] > 0:  # the clamp must cut some pre-activations
        g = _t(d["x"]) @ _t(d["wg"][0]).T
        assert (g.abs() > c["limit"]).any()
    r = orc.layer_backward(d["x"], d["wr"], d["wg"], d["wu"], d["wd"], fwd, d["dout"], sg=d["sg"],
                           su=d["su"], sd=d["sd"], scale=c["scale"], limit=c["limit"],
                           norm_topk=c["norm_topk"], d_aux=c["d_aux"], round_bf16=False)
    ref = _autograd(d, fwd, K, c["scale"], c["limit"], c["norm_topk"], c["d_aux"])
    kept = (fwd["slot_to_row"] >= 0).reshape(-1, K)
    for k, v in ref.items():
        got = r[k]
        if k == "d_topk_w":  # dropped slots have no gradient path in either
            v, got = v[kept], got[kept]
        scale_k = np.abs(v).max() + 1e-300
        np.testing.assert_allclose(got, v, rtol=1e-9, atol=1e-12 * scale_k, err_msg=k)


def test_rounded_backward_is_bf16_close_to_exact(orc):
    K = 3
    d = _case(4)
    fwd = orc.layer_forward(d["x"], d["wr"], d["wg"], d["wu"], d["wd"], K, bias=d["bias"],
                            sg=d["sg"], su=d["su"], sd=d["sd"], scale=2.827, limit=10.0)
    kw = dict(sg=d["sg"], su=d["su"], sd=d["sd"], scale=2.827, limit=10.0, d_aux=0.2)
    ex = orc.layer_backward(d["x"], d["wr"], d["wg"], d["wu"], d["wd"], fwd, d["dout"],
                            round_bf16=False, **kw)
    rd = orc.layer_backward(d["x"], d["wr"], d["wg"], d["wu"], d["wd"], fwd, d["dout"],
                            round_bf16=True, **kw)
    # stored tensors are bf16 values
    for k in ("dx", "dh_rows", "dg_rows", "du_rows", "dx_rows"):
        v = rd[k].astype(np.float32)
        assert np.array_equal(v.view(np.uint32) & 0xFFFF, np.zeros_like(v.view(np.uint32))), k
        assert np.array_equal(v.astype(np.float64), rd[k]), k
    # and everything stays within a few bf16 roundings of the exact values
    for k in ("dx", "d_wr", "d_wg", "d_wu", "d_wd", "d_sg", "d_su", "d_sd", "d_logits", "d_topk_w"):
        a, b = rd[k], ex[k]
        rms = np.sqrt(np.mean(b * b))
        assert np.all(np.abs(a - b) <= 0.03 * np.abs(b) + 0.03 * rms), k


def test_sub_steps_compose_to_the_layer_backward(orc):
    """The per-step functions (used by the chained GPU comparisons) reproduce the composed
    backward on one expert's rows bit for bit."""
    K = 3
    d = _case(5)
    fwd = orc.layer_forward(d["x"], d["wr"], d["wg"], d["wu"], d["wd"], K, bias=d["bias"],
                            sg=d["sg"], su=d["su"], sd=d["sd"], scale=2.827, limit=10.0)
    rd = orc.layer_backward(d["x"], d["wr"], d["wg"], d["wu"], d["wd"], fwd, d["dout"], sg=d["sg"],
                            su=d["su"], sd=d["sd"], scale=2.827, limit=10.0)
    f64 = orc.bf16_to_f64
    dy, dw = orc.combine_bwd(fwd["topk_w"], fwd["slot_to_row"], f64(fwd["y_routed"]), d["dout"])
    np.testing.assert_array_equal(dw, rd["d_topk_w"])
    off = fwd["offsets"]
    e = int(np.argmax(np.diff(off)))
    a, b = off[e], off[e + 1]
    xr = d["x"][fwd["row_to_slot"][a:b] // K]
    dh = orc.down_bwd_rows(dy[a:b], d["wd"][e])
    np.testing.assert_array_equal(dh, rd["dh_rows"][a:b])
    dg, du = orc.swiglu_bwd_rows(xr, d["wg"][e], d["wu"][e], dh, 10.0)
    np.testing.assert_array_equal(dg, rd["dg_rows"][a:b])
    np.testing.assert_array_equal(du, rd["du_rows"][a:b])
    dxr = orc.gateup_dgrad_rows(dg, du, d["wg"][e], d["wu"][e])
    np.testing.assert_array_equal(dxr, rd["dx_rows"][a:b])
    np.testing.assert_array_equal(orc.wgrad(dy[a:b], f64(fwd["h_routed"][a:b])), rd["d_wd"][e])
    np.testing.assert_array_equal(orc.wgrad(dg, f64(xr)), rd["d_wg"][e])
    dl = orc.router_bwd(fwd["logits"], fwd["topk_idx"], rd["d_topk_w"], 2.827, True, 0.0)
    np.testing.assert_array_equal(dl, rd["d_logits"])
