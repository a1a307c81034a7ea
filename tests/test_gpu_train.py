"""GPU parity of the training-side router (moe_route_train) against the oracle, through the C ABI.

Score noise is drawn on the host side of the test (seeded N(0, 0.01^2), as the Hy4 deep-dive's
router draws it) and given to both sides. Routing integers are compared bit-exactly from the
GPU's own fp32 logits; the statistics within tolerances derived from the fp32 reductions:
  * prob_mean: each probability carries a few fp32 roundings (exp, the butterfly sum over E,
    the division); the token sum adds at most (16 + 2 + nb) roundings, nb = ceil(T/64) partial
    blocks. Bound: |dP| <= (1e-5 + 1.2e-7 * (nb + 20)) * P + 1e-9.
  * aux_loss: the same relative bound plus 1e-6 for the 8-level tree over experts.
  * load_frac: integer counts, one fp32 division: relative 1e-7.
  * EMAs: two fp32 products and a sum: relative 1e-6.
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

CASES = {
    "tiny_t128_h512_e32_k2": WORKLOADS["tiny_t128_h512_e32_k2"],
    "ragged_t130_h256_e256_k8": Workload("ragged_t130_h256_e256_k8", T=130, H=256, E=256, K=8,
                                         I=256, scale=2.827, w_std=0.02, router_std=0.02, seed=31),
    "one_token_t1_e64_k6": Workload("one_token_t1_e64_k6", T=1, H=512, E=64, K=6, I=256, seed=32),
    "bias_t3000_h512_e256_k8": Workload("bias_t3000_h512_e256_k8", T=3000, H=512, E=256, K=8,
                                        I=256, scale=2.827, zipf=1.2, seed=33),
    "e24_k3_t777": Workload("e24_k3_t777", T=777, H=256, E=24, K=3, I=256, seed=34),
}
FULL = ["hy4_prefill_t8192", "hy4_skew_t65536"]


def _noise(wl, scale=0.01):
    g = torch.Generator(device=DEV)
    g.manual_seed(1000 * wl.seed + 99)
    return torch.randn(wl.T, wl.E, generator=g, device=DEV, dtype=torch.float32) * scale


def _run(wl, dev, noise, ema_c=None, ema_t=None, decay=0.9):
    s = moe.Shape.of(wl)
    T, E, K = wl.T, wl.E, wl.K
    out = dict(
        logits=torch.empty((T, E), dtype=torch.float32, device=DEV),
        topk_w=torch.empty((T, K), dtype=torch.float32, device=DEV),
        topk_idx=torch.empty((T, K), dtype=torch.int32, device=DEV),
        prob_mean=torch.empty(E, dtype=torch.float32, device=DEV),
        load_frac=torch.empty(E, dtype=torch.float32, device=DEV),
        aux_loss=torch.empty(1, dtype=torch.float32, device=DEV),
    )
    ws = torch.empty(moe.moe_route_train_workspace_size(s), dtype=torch.uint8, device=DEV)
    moe.moe_route_train(s, dev["x"], dev["w_router"], dev["router_bias"], noise, out["logits"],
                        out["topk_w"], out["topk_idx"], out["prob_mean"], out["load_frac"],
                        out["aux_loss"], ema_c, ema_t, ws, ema_decay=decay)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def _check_stats(wl, g, decay=0.9, ema0=None, ema_t0=None, ema_g=None, ema_tg=None):
    # routing from the GPU's own logits: bit-exact integers
    idx, w = oracle.route_from_logits(g["logits"], wl.K, wl.scale, wl.norm_topk)
    np.testing.assert_array_equal(g["topk_idx"], idx)
    np.testing.assert_allclose(g["topk_w"], w, rtol=0, atol=1e-5 * wl.scale)
    r = oracle.router_train_stats(g["logits"], g["topk_idx"], decay, ema0, ema_t0)
    nb = -(-wl.T // 64)
    rel = 1e-5 + 1.2e-7 * (nb + 20)
    err = np.abs(g["prob_mean"] - r["prob_mean"])
    assert np.all(err <= rel * r["prob_mean"] + 1e-9), ("prob_mean", err.max())
    np.testing.assert_allclose(g["load_frac"], r["load_frac"], rtol=1e-7, atol=0)
    assert abs(g["aux_loss"][0] - r["aux_loss"]) <= (rel + 1e-6) * r["aux_loss"], (g["aux_loss"], r["aux_loss"])
    if ema0 is not None:
        np.testing.assert_allclose(ema_g, r["ema_counts"], rtol=1e-6, atol=1e-6)
        assert abs(ema_tg - r["ema_tokens"]) <= 1e-6 * abs(r["ema_tokens"]) + 1e-6
    return r


@pytest.mark.parametrize("name", list(CASES))
def test_route_train_small(name):
    assert torch.cuda.is_available()
    wl = CASES[name]
    dev = generate(wl, DEV, shared=False)
    noise = _noise(wl)
    g = _run(wl, dev, noise)
    # logits against the oracle's projection plus the same noise
    bias = None if dev["router_bias"] is None else dev["router_bias"].cpu().numpy()
    lo = oracle.router_logits_noisy(as_u16(dev["x"]), as_u16(dev["w_router"]), bias,
                                    noise.cpu().numpy())
    P.assert_logits_close(g["logits"], lo)
    _check_stats(wl, g)
    # the noise moved some decisions: without it the routing differs somewhere
    g0 = _run(wl, dev, None)
    if wl.T >= 100:
        assert not np.array_equal(g0["topk_idx"], g["topk_idx"])
    _check_stats(wl, g0)


def test_route_train_ema_and_determinism():
    assert torch.cuda.is_available()
    wl = CASES["bias_t3000_h512_e256_k8"]
    dev = generate(wl, DEV, shared=False)
    noise = _noise(wl)
    rng = np.random.default_rng(7)
    ema0 = rng.uniform(0, 50, wl.E).astype(np.float32)
    ec = torch.from_numpy(ema0).to(DEV)
    et = torch.tensor([123.0], dtype=torch.float32, device=DEV)
    g = _run(wl, dev, noise, ec, et, decay=0.9)
    _check_stats(wl, g, 0.9, ema0.astype(np.float64), 123.0, ec.cpu().numpy(), float(et.cpu()[0]))
    # every output is the same bits on a second run
    g2 = _run(wl, dev, noise)
    for k in g:
        np.testing.assert_array_equal(g[k], g2[k], err_msg=k)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", FULL)
def test_route_train_full_size(name):
    assert torch.cuda.is_available()
    wl = WORKLOADS[name]
    print("\n[route-train full-size] %s T=%d E=%d K=%d" % (name, wl.T, wl.E, wl.K), flush=True)
    dev = generate(wl, DEV, shared=False)
    noise = _noise(wl)
    g = _run(wl, dev, noise)
    r = _check_stats(wl, g)
    # sampled tokens: logits against the oracle's own projection plus the noise
    toks = np.sort(np.random.default_rng(5).choice(wl.T, 6, replace=False))
    sel = torch.from_numpy(toks).to(DEV)
    bias = None if dev["router_bias"] is None else dev["router_bias"].cpu().numpy()
    lo = oracle.router_logits_noisy(as_u16(dev["x"][sel]), as_u16(dev["w_router"]), bias,
                                    noise[sel].cpu().numpy())
    P.assert_logits_close(g["logits"][toks], lo, "sampled logits")
    assert abs(float(np.sum(g["load_frac"])) - 1.0) < 1e-5
    if name == "hy4_skew_t65536":
        assert r["aux_loss"] > 2.0  # the skewed router concentrates the load
