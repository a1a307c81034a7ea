"""Pins of the oracle's training-side router statistics (CPU only).

The Hy3 deep-dive's SparseMoERouter, in training, computes a load-balancing loss
E * sum_e P_e f_e (P: token mean of the routing probabilities, f: share of the top-k selections)
and keeps exponential moving averages of the expert counts and the token count (decay 0.9); the
Hy4 deep-dive's MoERouter adds N(0, 0.01^2) noise to the scores before the softmax. These pins
hold the oracle to closed forms (uniform and one-hot routers, the two-expert sigmoid case, the
EMA recurrence), invariants and numpy's bincount.
"""
import math

import numpy as np
import pytest


@pytest.mark.parametrize("E,K", [(32, 2), (24, 3), (256, 8)])
def test_uniform_router_closed_form(orc, E, K):
    T = 40
    lg = np.zeros((T, E), np.float32)
    idx, _ = orc.route_from_logits(lg, K, 1.0)
    assert np.all(idx == np.arange(K))  # equal scores: the lowest indices win
    r = orc.router_train_stats(lg, idx)
    np.testing.assert_allclose(r["prob_mean"], 1.0 / E, rtol=1e-14)
    want_f = np.where(np.arange(E) < K, 1.0 / K, 0.0)
    np.testing.assert_allclose(r["load_frac"], want_f, rtol=1e-15)
    assert abs(r["aux_loss"] - 1.0) < 1e-13  # E * K * (1/E) * (1/K)


def test_one_hot_router_closed_form(orc):
    T, E = 30, 16
    lg = np.zeros((T, E), np.float32)
    lg[:, 5] = 60.0
    idx, _ = orc.route_from_logits(lg, 1, 1.0)
    r = orc.router_train_stats(lg, idx)
    p5 = 1.0 / (1.0 + (E - 1) * math.exp(-60.0))
    assert abs(r["prob_mean"][5] - p5) < 1e-15
    assert r["load_frac"][5] == 1.0 and r["load_frac"].sum() == 1.0
    assert abs(r["aux_loss"] - E * p5) < 1e-12  # collapsed routing: the loss approaches E


def test_two_experts_sigmoid_closed_form(orc):
    rng = np.random.default_rng(3)
    T = 50
    d = rng.standard_normal(T).astype(np.float32) * 3
    d[:3] = 0.0  # exact ties go to expert 0
    lg = np.stack([d, np.zeros(T, np.float32)], axis=1)
    idx, _ = orc.route_from_logits(lg, 1, 1.0)
    r = orc.router_train_stats(lg, idx)
    p0 = np.mean([1.0 / (1.0 + math.exp(-float(v))) for v in d])
    f0 = np.mean(d >= 0)
    assert abs(r["prob_mean"][0] - p0) < 1e-14 and abs(r["prob_mean"][1] - (1 - p0)) < 1e-14
    assert r["load_frac"][0] == f0
    assert abs(r["aux_loss"] - 2 * (p0 * f0 + (1 - p0) * (1 - f0))) < 1e-13


def test_invariants_and_bincount(orc):
    rng = np.random.default_rng(4)
    T, E, K = 77, 64, 6
    lg = (rng.standard_normal((T, E)) * 2).astype(np.float32)
    idx, _ = orc.route_from_logits(lg, K, 2.827)
    r = orc.router_train_stats(lg, idx)
    assert abs(r["prob_mean"].sum() - 1.0) < 1e-13
    assert abs(r["load_frac"].sum() - 1.0) < 1e-13
    np.testing.assert_array_equal(r["load_frac"] * T * K, np.bincount(idx.ravel(), minlength=E))
    # the loss is 1 for a perfectly even router and grows with concentration; it is bounded by E
    assert 0.0 < r["aux_loss"] <= E
    # scores shifted by a per-token constant leave every statistic unchanged
    r2 = orc.router_train_stats(lg + 3.0, idx)
    np.testing.assert_allclose(r2["prob_mean"], r["prob_mean"], rtol=1e-6)


def test_ema_recurrence_closed_form(orc):
    rng = np.random.default_rng(5)
    T, E, K = 20, 8, 2
    lg = rng.standard_normal((T, E)).astype(np.float32)
    idx, _ = orc.route_from_logits(lg, K, 1.0)
    c = np.bincount(idx.ravel(), minlength=E).astype(np.float64)
    ema0 = rng.uniform(0, 10, E)
    ec, et = ema0.copy(), 3.0
    for _ in range(5):
        r = orc.router_train_stats(lg, idx, decay=0.9, ema_counts=ec, ema_tokens=et)
        ec, et = r["ema_counts"], r["ema_tokens"]
    np.testing.assert_allclose(ec, c + 0.9 ** 5 * (ema0 - c), rtol=1e-13)
    assert abs(et - (T + 0.9 ** 5 * (3.0 - T))) < 1e-12
    # without initial values nothing is tracked
    r = orc.router_train_stats(lg, idx)
    assert r["ema_counts"] is None and r["ema_tokens"] is None


def test_noise_enters_before_the_softmax(orc):
    rng = np.random.default_rng(6)
    T, H, E = 9, 64, 8
    b16 = lambda a: (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    x = b16(rng.standard_normal((T, H)))
    wr = b16(rng.standard_normal((E, H)) * 0.02)
    lg = orc.router_logits(x, wr)
    np.testing.assert_array_equal(orc.router_logits_noisy(x, wr, None, np.zeros((T, E))), lg)
    noise = np.zeros((T, E), np.float32)
    noise[:, 7] = 50.0  # a large score shift moves every token's top-1 to expert 7
    ln = orc.router_logits_noisy(x, wr, None, noise)
    np.testing.assert_allclose(ln - lg, noise, atol=1e-5)
    idx, _ = orc.route_from_logits(ln, 1, 1.0)
    assert np.all(idx == 7)
