"""Pins of the oracle's FP8 expert-weight path (CPU only).

FP8 weights are OCP E4M3 codes with one fp32 scale per weight row (weight = scale * e4m3(code));
activations and intermediates stay bf16 exactly as in the bf16 layer. The decode is pinned to
hand-derived codes and to PyTorch's float8_e4m3fn over all 256 codes; the FP8 layer is pinned to
a float64 PyTorch SwiGLU FFN over the dequantised weights, to the (separately pinned) bf16 layer
where every dequantised weight is exactly a bf16 value, and to its own dense brute force.
"""
import math
import os

import numpy as np
import pytest
import torch

from tests.test_oracle_pins import _bf16_torch, _f64, _rand_bf16, _ulp_close

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3_golden_cases(orc):
    n = 0
    with open(os.path.join(GOLDEN, "fp8_e4m3.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            code, expr = line.split(None, 1)
            got = orc.double_from_e4m3(int(code, 16))
            if expr.strip() == "nan":
                assert math.isnan(got), code
            else:
                want = float(eval(expr, {"__builtins__": {}}))
                assert got == want and math.copysign(1, got) == math.copysign(1, want), (code, got)
            n += 1
    assert n >= 15


def test_e4m3_decode_matches_torch_for_every_code(orc):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([orc.double_from_e4m3(c) for c in range(256)])
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(nan, np.isnan(got))
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _rand_fp8(rng, shape, std, pow2_scales=False):
    """Random E4M3 codes (finite only) and per-row scales."""
    w = torch.from_numpy(rng.standard_normal(shape) * std)
    scale = w.abs().amax(dim=-1) / 448.0
    if pow2_scales:  # the next power of two up, times a random extra 2^0..2^2 per row
        scale = 2.0 ** (torch.ceil(torch.log2(scale)) +
                        torch.from_numpy(rng.integers(0, 3, size=shape[:-1]).astype(np.float64)))
    q = (w / scale.unsqueeze(-1)).to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)
    return q.numpy(), scale.to(torch.float32).numpy()


def _dequant64(q, scale):
    """float64 weights from codes and row scales, via PyTorch's E4M3 decode."""
    v = torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(torch.float64)
    return v * torch.from_numpy(scale.astype(np.float64)).unsqueeze(-1)


@pytest.mark.parametrize("limit", [10.0, 0.0])
def test_fp8_single_expert_equals_dense_swiglu_ffn(orc, limit):
    """E=1, k=1, no shared expert: a dense SwiGLU FFN over the dequantised weights (float64)."""
    rng = np.random.default_rng(31)
    T, H, I = 24, 64, 96
    x = _rand_bf16(rng, (T, H), 1.0)
    wr = _rand_bf16(rng, (1, H), 0.02)
    wg, wu, wd = (orc.Fp8(*_rand_fp8(rng, s, sd)) for s, sd in
                  (((1, I, H), 1.0), ((1, I, H), 1.0), ((1, H, I), 0.05)))
    # row scales differ: a scale applied per column or to the wrong operand fails below
    assert len(set(wg.scale[0].tolist())) > I // 2
    r = orc.layer_forward_fp8(x, wr, wg, wu, wd, 1, scale=1.0, limit=limit)
    X = _f64(x)
    G, U, D = _dequant64(wg.q[0], wg.scale[0]), _dequant64(wu.q[0], wu.scale[0]), \
        _dequant64(wd.q[0], wd.scale[0])
    g, u = X @ G.T, X @ U.T
    if limit > 0:
        assert (g.abs() > limit).any(), "test inputs must exercise the clamp"
        g, u = g.clamp(-limit, limit), u.clamp(-limit, limit)
    h_ref = _bf16_torch(torch.nn.functional.silu(g) * u)
    assert _ulp_close(r["h_routed"], h_ref).all()
    assert (r["h_routed"] == h_ref).mean() > 0.99
    y_ref = _bf16_torch(_f64(r["h_routed"]) @ D.T)
    assert _ulp_close(r["y_routed"], y_ref).all()
    assert (r["y_routed"] == y_ref).mean() > 0.99
    assert np.all(r["topk_idx"] == 0) and np.all(r["topk_w"] == 1.0)
    np.testing.assert_array_equal(r["out"], r["y_routed"])


def _fp8_layer_inputs(T=64, H=128, E=16, K=4, I=64, seed=0, pow2=False, shared=True):
    rng = np.random.default_rng(seed)
    x = _rand_bf16(rng, (T, H), 1.0)
    wr = _rand_bf16(rng, (E, H), 0.05)
    w = [orc_fp8(*_rand_fp8(rng, s, 0.05, pow2)) for s in ((E, I, H), (E, I, H), (E, H, I))]
    sw = [orc_fp8(*_rand_fp8(rng, s, 0.05, pow2)) for s in ((I, H), (I, H), (H, I))] \
        if shared else [None] * 3
    return x, wr, w, sw


def orc_fp8(q, scale):
    import oracle
    return oracle.Fp8(q, scale)


def _as_bf16_weights(w):
    """Exact bf16 bit patterns of scale * e4m3(code) (asserting exactness)."""
    v = _dequant64(w.q, w.scale)
    b = _bf16_torch(v)
    assert torch.equal(_f64(b).reshape(v.shape), v), "dequantised weight not exact in bf16"
    return b.reshape(w.q.shape)


def test_fp8_layer_equals_bf16_layer_on_exact_weights(orc):
    """With power-of-two row scales every dequantised weight is exactly a bf16 value (3 mantissa
    bits, exponents in range), so the FP8 layer must reproduce the bf16 layer bit for bit."""
    x, wr, w, sw = _fp8_layer_inputs(T=48, seed=5, pow2=True)
    bias = (1.2 * np.log(1.0 / (np.arange(16) + 1.0))).astype(np.float32)
    r8 = orc.layer_forward_fp8(x, wr, *w, 4, bias=bias, sg=sw[0], su=sw[1], sd=sw[2],
                               scale=2.827, limit=10.0)
    wb = [_as_bf16_weights(t) for t in w]
    sb = [_as_bf16_weights(t) for t in sw]
    rb = orc.layer_forward(x, wr, *wb, 4, bias=bias, sg=sb[0], su=sb[1], sd=sb[2], scale=2.827,
                           limit=10.0)
    for key in ("topk_idx", "topk_w", "row_to_slot", "h_routed", "y_routed", "h_shared",
                "y_shared", "out"):
        np.testing.assert_array_equal(r8[key], rb[key], err_msg=key)
    assert (r8["out"] != 0).mean() > 0.9


@pytest.mark.parametrize("capacity", [0, 9])
def test_fp8_sparse_equals_dense_bruteforce(orc, capacity):
    x, wr, w, sw = _fp8_layer_inputs(seed=6)
    r = orc.layer_forward_fp8(x, wr, *w, 4, sg=sw[0], su=sw[1], sd=sw[2], scale=2.827,
                              limit=10.0, capacity=capacity)
    if capacity:
        assert (r["slot_to_row"] < 0).any(), "capacity case must drop something"
    dense = orc.layer_dense_fp8(x, *w, r["topk_idx"], r["topk_w"], r["slot_to_row"],
                                sg=sw[0], su=sw[1], sd=sw[2], limit=10.0)
    np.testing.assert_array_equal(r["out"], dense)


def test_fp8_down_scale_is_linear(orc):
    """Doubling every down-projection row scale doubles y exactly (bf16 rounding commutes with
    multiplication by 2 away from overflow and underflow)."""
    rng = np.random.default_rng(7)
    n, H, I = 10, 48, 80
    h = _rand_bf16(rng, (n, I), 1.0)
    wd = orc.Fp8(*_rand_fp8(rng, (H, I), 0.05))
    y1 = orc.down_rows_fp8(h, wd)
    y2 = orc.down_rows_fp8(h, orc.Fp8(wd.q, wd.scale * 2))
    np.testing.assert_array_equal(_f64(y2).numpy(), 2 * _f64(y1).numpy())
    # scaling one row touches one output column only
    s = wd.scale.copy()
    s[5] *= 4
    y3 = orc.down_rows_fp8(h, orc.Fp8(wd.q, s))
    keep = np.arange(H) != 5
    np.testing.assert_array_equal(y3[:, keep], y1[:, keep])
    np.testing.assert_array_equal(_f64(y3[:, 5]).numpy(), 4 * _f64(y1[:, 5]).numpy())
