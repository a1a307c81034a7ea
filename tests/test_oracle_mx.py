"""Pins of the oracle's MX block-scaled FP8 (MXFP8) form, against things other than its own
formulas:
  * hand-derived block conversions (tests/golden/mx_blocks.txt): the shared-exponent rule and its
    clamping, nearest-even ties, saturation, subnormal elements, signed zero;
  * a brute-force search of the shared exponent (amax / 2^shared in [256, 512)) and of the nearest
    E4M3 code (all 256 codes, ties to the even code) on random blocks;
  * torch's float8_e4m3fn decoding of every code, scaled by 2^(s - 127), for the dequantisation;
  * float64 matrix products of the dequantised operands (numpy) for the block-scaled projections,
    and the per-expert functions composed by hand for the layer.
The format is OCP Microscaling (MX) v1.0, MXFP8 with E4M3 elements; the pages name an FP8
checkpoint without its scale format ("Tencent Hunyuan Hy4 Preview deep technical analysis",
deployment commands).
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mx_blocks.txt")


def _bf16_bits(vals):
    t = torch.tensor(vals, dtype=torch.float64).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _e4m3_table():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _golden():
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        body = line.split("#")[0]
        s, els, cs = [t.strip() for t in body.split("|")]
        els = [float(eval(e, {"__builtins__": {}})) for e in els.split(",")]
        cs = [int(c, 16) for c in cs.split(",")]
        yield int(s), els, cs


def test_golden_blocks():
    n = 0
    for s, els, cs in _golden():
        row = els + [0.0] * (32 - len(els))
        v = _bf16_bits(row)
        assert [float(x) for x in torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).double()[: len(els)]] == els
        codes, scales = oracle.mx_quant_rows(v[None, :])
        assert int(scales[0, 0]) == s, (els, int(scales[0, 0]), s)
        assert [int(c) for c in codes[0, : len(els)]] == cs, (els, codes[0, : len(els)], cs)
        assert all(int(c) == 0 for c in codes[0, len(els):])
        n += 1
    assert n >= 12


def _nearest_e4m3(q, table):
    """Brute force: the code whose value is nearest to clamp(q, +-448), ties to the even code."""
    a = min(abs(q), 448.0)
    best_d, best_c = None, None
    for c in range(128):
        if c == 0x7F:
            continue
        d = abs(table[c] - a)
        if best_d is None or d < best_d or (d == best_d and c % 2 == 0 and best_c % 2 == 1):
            best_d, best_c = d, c
    return best_c | (0x80 if math.copysign(1.0, q) < 0 else 0)


def test_random_blocks_brute_force():
    rng = np.random.default_rng(5)
    table = _e4m3_table()
    rows = []
    for mag in (1.0, 1e-3, 37.0, 2.0 ** -120, 2.0 ** 100):
        for dist in ("normal", "heavy"):
            x = rng.standard_normal(64) * mag
            if dist == "heavy":
                x = x * np.exp(rng.standard_normal(64) * 3)
            rows.append(x)
    v = _bf16_bits(np.array(rows))
    vals = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).double().numpy()
    codes, scales = oracle.mx_quant_rows(v)
    for r in range(v.shape[0]):
        for b in range(2):
            blk = vals[r, 32 * b: 32 * b + 32]
            amax = np.abs(blk).max()
            sh = next(k for k in range(-400, 400) if 256 <= amax / 2.0 ** k < 512) if amax > 0 else -127
            sh = max(-127, min(127, sh))
            assert int(scales[r, b]) == sh + 127
            for c in range(32):
                want = _nearest_e4m3(blk[c] / 2.0 ** sh, table)
                assert int(codes[r, 32 * b + c]) == want, (r, b, c, blk[c], sh)


def test_dequant_is_e4m3_times_power_of_two():
    table = _e4m3_table()
    rng = np.random.default_rng(6)
    codes = rng.integers(0, 256, size=(5, 64)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x7E  # no NaN codes
    scales = rng.integers(100, 160, size=(5, 2)).astype(np.uint8)
    got = oracle.mx_dequant(codes, scales)
    want = table[codes] * np.ldexp(1.0, np.repeat(scales.astype(np.int64) - 127, 32, axis=1))
    assert np.array_equal(got, want)


def test_quantisation_error_bound():
    """|dequant - v| is at most half an E4M3 step of v / 2^shared, times 2^shared, except for the
    saturated elements (v / 2^shared in (448, 512)), whose error is below 64 * 2^shared."""
    rng = np.random.default_rng(8)
    v = _bf16_bits(rng.standard_normal((16, 128)) * np.exp(rng.standard_normal((16, 1)) * 4))
    vals = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).double().numpy()
    codes, scales = oracle.mx_quant_rows(v)
    deq = oracle.mx_dequant(codes, scales)
    X = np.ldexp(1.0, np.repeat(scales.astype(np.int64) - 127, 32, axis=1))
    q = np.abs(vals) / X
    assert q.max() < 512
    e = np.floor(np.log2(np.maximum(q, 2.0 ** -6)))
    half_step = np.ldexp(1.0, (e - 4).astype(np.int64))  # 3 mantissa bits: step 2^(e-3)
    ok = np.where(q > 448, np.abs(deq - vals) < 64 * X, np.abs(deq - vals) <= half_step * X)
    assert ok.all()


def _mx_random(rng, rows, cols, lo=118, hi=130):
    codes = rng.integers(0, 256, size=(rows, cols)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x7E
    scales = rng.integers(lo, hi, size=(rows, cols // 32)).astype(np.uint8)
    return oracle.Mx(codes, scales)


def _swiglu(g, u, limit):
    g = np.clip(g, -limit, limit)
    u = np.clip(u, -limit, limit)
    return g / (1.0 + np.exp(-g)) * u


def test_projections_against_float64_matmul():
    rng = np.random.default_rng(9)
    n, H, I, limit = 6, 128, 64, 10.0
    x = _bf16_bits(rng.standard_normal((n, H)))
    xq, xs = oracle.mx_quant_rows(x)
    wg, wu = _mx_random(rng, I, H, 112, 118), _mx_random(rng, I, H, 112, 118)
    A = oracle.mx_dequant(xq, xs)
    g = (A @ oracle.mx_dequant(wg.q, wg.s).T).astype(np.float32).astype(np.float64)
    u = (A @ oracle.mx_dequant(wu.q, wu.s).T).astype(np.float32).astype(np.float64)
    want = _bf16_bits(_swiglu(g, u, limit))
    got = oracle.gateup_rows_mx(xq, xs, wg, wu, limit)
    # the fp64 sums differ only in summation order; fp32 rounding hides that except at a
    # rounding boundary, where the results differ by one bf16 step at most
    diff = np.abs(got.astype(np.int32) - want.astype(np.int32))
    assert diff.max() <= 1 and (diff != 0).mean() < 0.01
    # transposed weights (a plausible indexing mistake) give a different result
    wgt = oracle.Mx(wg.q.reshape(H, I).T.copy().reshape(I, H), wg.s)
    assert not np.array_equal(oracle.gateup_rows_mx(xq, xs, wgt, wu, limit), got)
    # down projection
    wd = _mx_random(rng, H, I, 112, 118)
    hq, hs = oracle.mx_quant_rows(got)
    y = oracle.down_rows_mx(hq, hs, wd)
    yw = _bf16_bits((oracle.mx_dequant(hq, hs) @ oracle.mx_dequant(wd.q, wd.s).T).astype(np.float32))
    d = np.abs(y.astype(np.int32) - yw.astype(np.int32))
    assert d.max() <= 1 and (d != 0).mean() < 0.01


def test_layer_composes_the_expert_functions():
    rng = np.random.default_rng(10)
    T, H, E, K, I, limit = 24, 64, 6, 2, 32, 7.0
    x = _bf16_bits(rng.standard_normal((T, H)))
    wr = _bf16_bits(rng.standard_normal((E, H)) * 0.1)
    wg, wu = _mx_random(rng, E * I, H), _mx_random(rng, E * I, H)
    wd = _mx_random(rng, E * H, I)
    stk = lambda m, e, r: oracle.Mx(m.q.reshape(e, r, -1), m.s.reshape(e, r, -1))
    sg, su, sd = _mx_random(rng, I, H), _mx_random(rng, I, H), _mx_random(rng, H, I)
    r = oracle.layer_forward_mx(x, wr, stk(wg, E, I), stk(wu, E, I), stk(wd, E, H), K, sg=sg, su=su,
                                sd=sd, scale=2.5, limit=limit)
    base = oracle.layer_forward(x, wr, np.zeros((E, I, H), np.uint16), np.zeros((E, I, H), np.uint16),
                                np.zeros((E, H, I), np.uint16), K, scale=2.5, limit=limit)
    for k in ("logits", "topk_idx", "topk_w", "counts", "offsets", "row_to_slot", "slot_to_row"):
        assert np.array_equal(r[k], base[k]), k
    xq, xs = oracle.mx_quant_rows(x)
    assert np.array_equal(r["xq"], xq) and np.array_equal(r["x_scale"], xs)
    ys = None
    for e in range(E):
        o0, o1 = int(r["offsets"][e]), int(r["offsets"][e + 1])
        if o1 == o0:
            continue
        toks = r["row_to_slot"][o0:o1] // K
        h = oracle.gateup_rows_mx(xq[toks], xs[toks], oracle.Mx(wg.q[e * I:(e + 1) * I], wg.s[e * I:(e + 1) * I]),
                                  oracle.Mx(wu.q[e * I:(e + 1) * I], wu.s[e * I:(e + 1) * I]), limit)
        assert np.array_equal(r["h_routed"][o0:o1], h)
        hq, hs = oracle.mx_quant_rows(h)
        y = oracle.down_rows_mx(hq, hs, oracle.Mx(wd.q[e * H:(e + 1) * H], wd.s[e * H:(e + 1) * H]))
        assert np.array_equal(r["y_routed"][o0:o1], y)
    hsh = oracle.gateup_rows_mx(xq, xs, sg, su, limit)
    assert np.array_equal(r["h_shared"], hsh)
    hq, hs = oracle.mx_quant_rows(hsh)
    ys = oracle.down_rows_mx(hq, hs, sd)
    assert np.array_equal(r["y_shared"], ys)
    out = oracle.combine(r["topk_w"], r["slot_to_row"], r["y_routed"], ys)
    assert np.array_equal(r["out"], out)
