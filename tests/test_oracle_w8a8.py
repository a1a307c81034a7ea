"""Pins of the oracle's W8A8 path (CPU only): FP8 E4M3 expert weights with per-row scales, and the
activations entering each expert projection quantised per row to E4M3 with one fp32 scale.

- The E4M3 encoder is pinned to PyTorch's float8_e4m3fn conversion: on every representable
  value, every midpoint between neighbours (ties go to the even code), subnormals, values past
  448 (saturated before the library call, which would give NaN) and random values.
- The per-row quantiser is pinned by properties the definition fixes: the row maximum maps to
  +-448, the dequantisation error stays within half an E4M3 step, exactly representable rows
  come back exactly with a power-of-two scale, zero rows and sign symmetry.
- The W8A8 projections are pinned to the separately pinned W8A16 oracle. On activation rows
  that quantise exactly, the two compute the same sums and must agree bit for bit.
- The W8A8 layer is pinned to a brute-force composition of those projections.
"""
import numpy as np
import pytest
import torch

from tests.test_oracle_fp8 import _rand_fp8
from tests.test_oracle_pins import _f64, _rand_bf16


def _torch_e4m3(q):
    """PyTorch's E4M3 codes of float32 values clipped to +-448 (the library returns NaN past
    the largest finite value, where the encoder here saturates)."""
    q = np.clip(np.asarray(q, dtype=np.float32), -448.0, 448.0)
    return torch.from_numpy(np.ascontiguousarray(q)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _e4m3_values():
    """All finite E4M3 values, ascending, non-negative (codes 0x00..0x7E)."""
    v = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.all(np.diff(v) > 0)
    return v


def test_encoder_round_trips_every_finite_code(orc):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = orc.e4m3_from_float(vals)
    np.testing.assert_array_equal(got, codes)


def test_encoder_ties_go_to_even(orc):
    v = _e4m3_values()
    mid = ((v[:-1] + v[1:]) / 2).astype(np.float32)  # exact in float32: one more mantissa bit
    assert np.array_equal(mid.astype(np.float64), (v[:-1] + v[1:]) / 2)
    for sign in (1.0, -1.0):
        q = sign * mid
        got = orc.e4m3_from_float(q)
        np.testing.assert_array_equal(got, _torch_e4m3(q))
        # the even code of each pair wins: both neighbours are codes c and c + 1
        lo = np.arange(len(mid))
        even = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)
        np.testing.assert_array_equal(got & 0x7F, even)


def test_encoder_matches_torch_on_random_and_edge_values(orc):
    rng = np.random.default_rng(123)
    mag = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(600.0), size=200000))
    q = (mag * rng.choice([-1.0, 1.0], size=mag.size)).astype(np.float32)
    edges = np.array([0.0, -0.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -6, 2.0 ** -6 * 0.96,
                      448.0, 447.0, 463.9, 464.0, 500.0, 1e30, -1e30, 1e-30, -1e-30], dtype=np.float32)
    q = np.concatenate([q, edges, -edges])
    got = orc.e4m3_from_float(q)
    np.testing.assert_array_equal(got, _torch_e4m3(q))
    # saturation: everything at or beyond 448 in magnitude is the largest finite code
    big = np.abs(q) >= 448
    assert np.all((got[big] & 0x7F) == 0x7E)


def _deq(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _e4m3_step(m):
    """Distance between neighbouring E4M3 values around magnitude m (float64 array)."""
    m = np.maximum(np.asarray(m, dtype=np.float64), 2.0 ** -6)
    return 2.0 ** (np.floor(np.log2(m)) - 3)


def test_quant_rows_properties(orc):
    rng = np.random.default_rng(7)
    rows, cols = 40, 256
    v = _rand_bf16(rng, (rows, cols), 1.0)
    v[3] = 0                                   # an all-zero row
    v[5, :] = _rand_bf16(rng, (1, cols), 1e-3)  # small values
    v[6, :] = _rand_bf16(rng, (1, cols), 300.0)  # large values
    codes, scales = orc.quant_rows_e4m3(v)
    x = _f64(v).numpy()
    amax = np.abs(x).max(axis=1)
    nz = amax > 0
    # the row maximum maps to the largest finite code; the scale is amax / 448 in float32
    arg = np.abs(x).argmax(axis=1)
    assert np.all((codes[nz, arg[nz]] & 0x7F) == 0x7E)
    np.testing.assert_array_equal(scales[nz], (amax[nz].astype(np.float32) / np.float32(448.0)))
    # zero row: scale 1, codes all zero
    assert scales[3] == 1.0 and not codes[3].any()
    # dequantisation error within half a step of the scaled value (plus float32 rounding of the
    # scaled product, at most one part in 2^23)
    deq = _deq(codes) * scales[:, None].astype(np.float64)
    q = np.abs(x) / scales[:, None]
    bound = (0.5 * _e4m3_step(q) + q * 2.0 ** -22) * scales[:, None] + 1e-30
    assert np.all(np.abs(deq - x) <= bound)
    # sign symmetry
    c2, s2 = orc.quant_rows_e4m3(v ^ np.uint16(0x8000))
    np.testing.assert_array_equal(s2, scales)
    np.testing.assert_array_equal(c2, codes ^ np.uint8(0x80))


def test_quant_rows_tiny_rows_are_unscaled(orc):
    """A row whose 448 / amax overflows fp32 is quantised with scale 1 and E4M3_RNE(v): at those
    magnitudes (below 448 / FLT_MAX, about 1.3e-36, far under the smallest E4M3 subnormal 2^-9)
    every code is a signed zero, and nothing is NaN or saturated. Rows just above the threshold
    keep the scaled form, so the row maximum still maps to code 0x7E."""
    cols = 16
    tiny = np.array([1e-38, -3e-37, 2.0 ** -133, -(2.0 ** -126), 0.0, -0.0, 1.2e-36, 5e-37] * 2)
    just_above = np.linspace(-1.0, 1.0, cols) * 2e-36       # amax 2e-36: 448 / amax is finite
    v = torch.from_numpy(np.stack([tiny, just_above])).to(torch.bfloat16)
    v16 = v.view(torch.int16).numpy().view(np.uint16)
    codes, scales = orc.quant_rows_e4m3(v16)
    x = v.to(torch.float64).numpy()
    assert scales[0] == 1.0
    np.testing.assert_array_equal(codes[0], np.where(np.signbit(x[0]), 0x80, 0x00).astype(np.uint8))
    amax = np.float32(np.abs(x[1]).max())
    assert np.isfinite(np.float32(448.0) / amax)
    assert scales[1] == amax / np.float32(448.0)
    assert (codes[1][np.abs(x[1]).argmax()] & 0x7F) == 0x7E


def _exact_rows(rng, rows, cols, exps):
    """bf16 rows whose values are E4M3 values times 2^k (k per row) with the row maximum exactly
    448 * 2^k, so that quantisation is exact: codes back, scale 2^k. Returns (bf16 rows, codes,
    2^k)."""
    codes = rng.integers(0, 0x7F, size=(rows, cols)).astype(np.uint8)
    codes |= (rng.integers(0, 2, size=(rows, cols)) << 7).astype(np.uint8)
    codes[np.arange(rows), rng.integers(0, cols, size=rows)] = 0x7E  # +448 somewhere in each row
    codes[(codes & 0x7F) == 0x7F] = 0x7E
    k = np.asarray(exps, dtype=np.float64)
    v = _deq(codes) * 2.0 ** k[:, None]
    b = torch.from_numpy(v).to(torch.bfloat16)
    assert torch.equal(b.to(torch.float64), torch.from_numpy(v)), "row not exact in bf16"
    return b.view(torch.int16).numpy().view(np.uint16), codes, (2.0 ** k).astype(np.float32)


def test_quant_rows_exact_on_representable_rows(orc):
    rng = np.random.default_rng(8)
    v, codes, s = _exact_rows(rng, 12, 192, rng.integers(-12, 6, size=12))
    got_c, got_s = orc.quant_rows_e4m3(v)
    np.testing.assert_array_equal(got_s, s)
    # codes agree up to the sign of zero (a -0 input and a +0 input both decode to 0)
    np.testing.assert_array_equal(_deq(got_c), _deq(codes))


def _exact_fp8_weights(orc, rng, shape, std):
    return orc.Fp8(*_rand_fp8(rng, shape, std))


def test_w8a8_projections_equal_w8a16_on_exact_rows(orc):
    """Activation rows that quantise exactly: (sum codes_x * codes_w) * w_scale * x_scale equals
    the W8A16 sum of x * (w_scale * e4m3(code)) up to float64 rounding, so h and y agree with
    the (separately pinned) W8A16 oracle bit for bit."""
    rng = np.random.default_rng(9)
    n, H, I = 16, 128, 96
    x, _, _ = _exact_rows(rng, n, H, rng.integers(-8, -2, size=n))
    wg = _exact_fp8_weights(orc, rng, (I, H), 0.05)
    wu = _exact_fp8_weights(orc, rng, (I, H), 0.05)
    wd = _exact_fp8_weights(orc, rng, (H, I), 0.05)
    xq, sx = orc.quant_rows_e4m3(x)
    for limit in (10.0, 0.0):
        h8 = orc.gateup_rows_w8a8(xq, sx, wg, wu, limit)
        h16 = orc.gateup_rows_fp8(x, wg, wu, limit)
        np.testing.assert_array_equal(h8, h16)
    assert (h8 != 0).mean() > 0.9
    # down, on h rows that quantise exactly as well
    hb, _, _ = _exact_rows(rng, n, I, rng.integers(-6, 0, size=n))
    hq, sh = orc.quant_rows_e4m3(hb)
    y8 = orc.down_rows_w8a8(hq, sh, wd)
    y16 = orc.down_rows_fp8(hb, wd)
    np.testing.assert_array_equal(y8, y16)
    assert (y8 != 0).mean() > 0.9


def test_w8a8_projection_scales_are_per_row_and_per_column(orc):
    """Doubling one activation row doubles only that row's scale (same codes) and that output
    row; doubling one weight row's scale doubles only that output column (bf16 doubling is
    exact)."""
    rng = np.random.default_rng(10)
    n, H, N = 6, 64, 32
    x = _rand_bf16(rng, (n, H), 1.0)
    w = _exact_fp8_weights(orc, rng, (N, H), 0.05)
    xq, sx = orc.quant_rows_e4m3(x)
    row2 = np.where(np.arange(n) == 2, 2.0, 1.0)
    x2 = (torch.from_numpy(_f64(x).numpy() * row2[:, None])
          .to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    xq2, sx2 = orc.quant_rows_e4m3(x2)
    np.testing.assert_array_equal(xq2, xq)
    np.testing.assert_array_equal(sx2, sx * row2.astype(np.float32))
    y1 = _f64(orc.down_rows_w8a8(xq, sx, w)).numpy()
    y2 = _f64(orc.down_rows_w8a8(xq2, sx2, w)).numpy()
    np.testing.assert_array_equal(y2, y1 * row2[:, None])
    col5 = np.where(np.arange(N) == 5, 2.0, 1.0)
    w5 = orc.Fp8(w.q, w.scale * col5.astype(np.float32))
    y3 = _f64(orc.down_rows_w8a8(xq, sx, w5)).numpy()
    np.testing.assert_array_equal(y3, y1 * col5[None, :])
    assert (y1 != 0).mean() > 0.9


def _layer_inputs(orc, T=48, H=128, E=12, K=3, I=64, seed=0, shared=True):
    rng = np.random.default_rng(seed)
    x = _rand_bf16(rng, (T, H), 1.0)
    wr = _rand_bf16(rng, (E, H), 0.05)
    w = [orc.Fp8(*_rand_fp8(rng, s, 0.05)) for s in ((E, I, H), (E, I, H), (E, H, I))]
    sw = [orc.Fp8(*_rand_fp8(rng, s, 0.05)) for s in ((I, H), (I, H), (H, I))] if shared else [None] * 3
    return x, wr, w, sw


@pytest.mark.parametrize("capacity,shared", [(0, True), (7, True), (0, False)])
def test_w8a8_layer_equals_bruteforce_composition(orc, capacity, shared):
    x, wr, w, sw = _layer_inputs(orc, seed=11 + capacity, shared=shared)
    E, K = 12, 3
    r = orc.layer_forward_w8a8(x, wr, *w, K, sg=sw[0], su=sw[1], sd=sw[2], scale=2.827,
                               limit=10.0, capacity=capacity)
    if capacity:
        assert (r["slot_to_row"] < 0).any(), "capacity case must drop something"
    xq, sx = orc.quant_rows_e4m3(x)
    np.testing.assert_array_equal(r["xq"], xq)
    np.testing.assert_array_equal(r["x_scale"], sx)
    T, H = x.shape
    # every kept (token, slot) evaluated on its own through the row functions
    y_rows = np.zeros((T * K, H), dtype=np.uint16)
    for t in range(T):
        for j in range(K):
            row = r["slot_to_row"][t * K + j]
            if row < 0:
                continue
            e = r["topk_idx"][t, j]
            sub = lambda m: orc.Fp8(m.q[e], m.scale[e])
            h = orc.gateup_rows_w8a8(xq[t:t + 1], sx[t:t + 1], sub(w[0]), sub(w[1]), 10.0)
            hq, sh = orc.quant_rows_e4m3(h)
            y_rows[row] = orc.down_rows_w8a8(hq, sh, sub(w[2]))[0]
            np.testing.assert_array_equal(r["h_routed"][row], h[0])
    np.testing.assert_array_equal(r["y_routed"], y_rows)
    ys = None
    if shared:
        hs = orc.gateup_rows_w8a8(xq, sx, sw[0], sw[1], 10.0)
        hq, sh = orc.quant_rows_e4m3(hs)
        ys = orc.down_rows_w8a8(hq, sh, sw[2])
        np.testing.assert_array_equal(r["y_shared"], ys)
    out = orc.combine(r["topk_w"], r["slot_to_row"], y_rows, ys)
    np.testing.assert_array_equal(r["out"], out)
    assert (r["out"] != 0).mean() > 0.9
