"""CPU pins of the parity helpers in tests/parity.py: the vectorised bf16 rounding against the
oracle's own, and the fp32 chain bound against fp32 arithmetic carried out on the CPU."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from tests import parity as P


def test_bf16_rne_matches_oracle():
    rng = np.random.default_rng(5)
    v = rng.standard_normal(3000) * 10.0 ** rng.integers(-40, 38, 3000)
    # exact midpoints between neighbouring bf16 values (ties to even), zeros, subnormals, overflow
    b = rng.integers(0, 0x7F7F, 400).astype(np.uint16)
    lo = P.f64(b)
    hi = P.f64(b + 1)
    v = np.concatenate([v, (lo + hi) / 2, -(lo + hi) / 2, [0.0, -0.0, 2.0 ** -140, -(2.0 ** -133),
                                                           3.3e38, 3.4e38, -3.39e38, 2.0 ** -127]])
    np.testing.assert_array_equal(P.bf16_rne(v), oracle.bf16_round_array(v))


def _cut(v, granule):
    return np.copysign(np.floor(np.abs(v) / granule) * granule, v)


def _align_sum(vals, guard):
    """Sum over the last axis after aligning each term to the largest one's exponent with
    `guard` bits below the fp32 significand (the hardware model pinned on the GPU)."""
    big = np.abs(vals).max(axis=-1, keepdims=True)
    e = np.floor(np.log2(np.where(big > 0, big, 1.0)))
    granule = np.ldexp(1.0, (e - 23 - guard).astype(int))
    return _cut(vals, granule).sum(axis=-1)


def _chain_fp32(A, W, order, guard=1):
    """The fp32 chain the bound models, on the CPU: instructions in `order` (lists of K indices,
    each a multiple of 8 long); each sums its groups of 8 products aligned, then the accumulator
    and the group sums aligned, and rounds once to fp32."""
    out = np.zeros((A.shape[0], W.shape[0]))
    for ks in order:
        prods = A[:, None, ks] * W[None, :, ks]                     # [n, m, len]
        groups = _align_sum(prods.reshape(*prods.shape[:2], -1, 8), guard)
        terms = np.concatenate([out[..., None], groups], axis=-1)
        out = _align_sum(terms, guard).astype(np.float32).astype(np.float64)
    return out


def test_chain_bound_covers_fp32_chains():
    # products of bf16 values summed in fp32 instruction by instruction (contiguous 16-element
    # steps, and a permuted order inside 32-element blocks), against the bound; large offsets
    # make the running sums much larger than the result, the bound's worst case
    rng = np.random.default_rng(6)
    for K, blk, per in ((256, 16, 1), (512, 32, 2)):
        A = P.f64(P.bf16_rne(rng.standard_normal((20, K))))
        W = P.f64(P.bf16_rne(rng.standard_normal((24, K)) * 0.05))
        A[:5, :K // 2] += 300.0
        A[:5, K // 2:] -= 300.0
        A = P.f64(P.bf16_rne(A))
        if per == 1:
            order = [list(range(k, k + blk)) for k in range(0, K, blk)]
        else:  # two instructions per block: even and odd 8-element chunks
            order = []
            for k in range(0, K, blk):
                order.append([k + i for i in range(blk) if (i // 8) % 2 == 0])
                order.append([k + i for i in range(blk) if (i // 8) % 2 == 1])
        chain = P.Chain(blk, per, blk // per)
        S, d, _ = P.chain_sums(A, W, chain)
        for guard in (1, 2):
            got = _chain_fp32(A, W, order, guard)
            err = np.abs(got - S)
            assert np.all(err <= d), (K, blk, per, guard, float((err / d).max()))
        assert (err / d).max() > 0.01  # the bound is not vacuous


def test_check_interval_accepts_and_rejects():
    v = np.array([1.0, 1.0 + 2.0 ** -8, 3.0])    # 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7
    ref = P.bf16_rne(v)
    d = np.array([0.0, 1e-6, 0.0])
    got = ref.copy()
    got[1] = P.bf16_rne(1.0 + 2.0 ** -7)         # the other neighbour of the midpoint: allowed
    flips = P.check_interval(got, v, d, "ok", ref)
    assert flips.tolist() == [False, True, False]
    bad = ref.copy()
    bad[0] = P.bf16_rne(1.0 + 2.0 ** -7)         # one ulp off where no midpoint is near: rejected
    try:
        P.check_interval(bad, v, d, "bad", ref)
    except AssertionError:
        pass
    else:
        raise AssertionError("an off-interval value must be rejected")


def test_f64_and_e4m3_decodes_match_the_oracle():
    """The parity helpers' own bf16 and E4M3 decodes (through torch) against the oracle's, on
    every bit pattern (NaN patterns compared as NaN)."""
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns
        mine, ref = P.f64(b), oracle.bf16_to_f64(b)
    np.testing.assert_array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(mine[ok], ref[ok])
    np.testing.assert_array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))
    c = np.arange(256, dtype=np.uint8)
    mine8 = P.e4m3_f64(c)
    ref8 = np.array([oracle.double_from_e4m3(int(v)) for v in c])
    np.testing.assert_array_equal(np.isnan(mine8), np.isnan(ref8))
    ok = ~np.isnan(ref8)
    np.testing.assert_array_equal(mine8[ok], ref8[ok])
    np.testing.assert_array_equal(np.signbit(mine8[ok]), np.signbit(ref8[ok]))


def test_run_pipelined_keeps_order_and_raises():
    """Results come back in item order whatever order the pool finishes them in, and a failing
    check surfaces as its exception."""
    import time

    prepared = []

    def prepare(i):
        prepared.append(i)
        return i

    def check(i):
        time.sleep(0.002 * ((7 * i) % 5))
        return i * i

    assert P.run_pipelined(prepare, check, range(40), workers=4, window=6) == [i * i for i in range(40)]
    assert prepared == list(range(40))

    def bad(i):
        if i == 13:
            raise AssertionError("item 13")
        return i

    try:
        P.run_pipelined(lambda i: i, bad, range(30), workers=3, window=4)
    except AssertionError as e:
        assert "item 13" in str(e)
    else:
        raise AssertionError("the failing check did not raise")
