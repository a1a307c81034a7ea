"""Pins of the CPU oracle against facts fixed by the pages and by mathematics (CPU only).

Each test pins one part of the oracle to something other than itself: hand-derived fixtures
(tests/golden/), brute force over the bf16 value table, closed forms of softmax and the clamp,
a library stable sort, a dense brute-force evaluation, and a float64 PyTorch SwiGLU FFN.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- bf16 rounding
def _bf16_table():
    """All finite non-negative bf16 values (exact as Python floats), ascending, with bits."""
    bits = np.arange(0, 0x7F80, dtype=np.uint32)
    vals = (bits << 16).view(np.float32).astype(np.float64)
    return vals, bits


_TABLE = None


def brute_bf16(v: float) -> int:
    """Nearest bf16 by exhaustive table lookup with exact rational comparison; ties to even."""
    global _TABLE
    if _TABLE is None:
        _TABLE = _bf16_table()
    vals, bits = _TABLE
    if math.isnan(v):
        return 0x7FC0
    sign = 0x8000 if math.copysign(1.0, v) < 0 else 0
    a = abs(v)
    if math.isinf(a):
        return sign | 0x7F80
    i = int(np.searchsorted(vals, a, side="left"))
    if i < len(vals) and vals[i] == a:
        return sign | int(bits[i])
    if i == len(vals):  # beyond the largest finite: compare with the halfway point to 2^128
        lo = Fraction(vals[-1])
        hi = Fraction(2) ** 128
        da, db = Fraction(a) - lo, hi - Fraction(a)
        if da < db:
            return sign | int(bits[-1])
        return sign | 0x7F80  # tie or above: the largest finite has an odd mantissa
    lo, hi = Fraction(vals[i - 1]), Fraction(vals[i])
    da, db = Fraction(a) - lo, hi - Fraction(a)
    if da < db:
        return sign | int(bits[i - 1])
    if db < da:
        return sign | int(bits[i])
    return sign | int(bits[i - 1] if bits[i - 1] % 2 == 0 else bits[i])


def test_bf16_golden_cases(orc):
    n = 0
    with open(os.path.join(GOLDEN, "bf16_rne.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            expr, want = line.rsplit(None, 1)
            v = float(eval(expr, {"__builtins__": {}}))
            assert orc.bf16_from_double(v) == int(want, 16), (expr, hex(orc.bf16_from_double(v)))
            assert brute_bf16(v) == int(want, 16), expr
            n += 1
    assert n >= 15


def test_bf16_matches_brute_force_random_doubles(orc):
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        rng.standard_normal(3000) * 10.0 ** rng.integers(-45, 39, 3000),
        rng.standard_normal(500),
        # doubles sitting exactly on or next to bf16 halfway points
        [(1 + (2 * m + 1) * 2.0 ** -8) * 2.0 ** e for m in range(0, 128, 9) for e in (-130, -3, 0, 7, 126)],
        [np.nextafter((1 + 2.0 ** -8), 2.0), np.nextafter((1 + 2.0 ** -8), 0.0)],
    ])
    for v in vals:
        assert orc.bf16_from_double(float(v)) == brute_bf16(float(v)), repr(v)


def test_bf16_matches_torch_for_float32_inputs(orc):
    # torch's float32 -> bfloat16 conversion is round-to-nearest-even (a library routine)
    rng = np.random.default_rng(3)
    f = (rng.standard_normal(4000) * 10.0 ** rng.integers(-30, 30, 4000)).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.bf16_from_double(float(v)) for v in f], dtype=np.uint16)
    np.testing.assert_array_equal(got, ref)


def test_bf16_widening_is_exact(orc):
    for b in (0x0001, 0x0080, 0x3F80, 0x42C8, 0x7F7F, 0xBF80, 0x8000):
        assert orc.double_from_bf16(b) == float(
            np.array([b << 16], dtype=np.uint32).view(np.float32)[0])


# ----------------------------------------------------------------------------- routing
def _read_route_cases():
    cases = []
    with open(os.path.join(GOLDEN, "route_ties.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            head, lg, idx, w = [p.strip() for p in line.split("|")]
            E, K, s = head.split()
            cases.append((int(E), int(K), float(s), [float(v) for v in lg.split()],
                          [int(v) for v in idx.split()],
                          [float(eval(v, {"__builtins__": {}})) for v in w.split()]))
    return cases


def test_route_golden_ties(orc):
    cases = _read_route_cases()
    assert len(cases) >= 6
    for E, K, s, lg, idx, w in cases:
        got_i, got_w = orc.route_from_logits(np.array([lg], dtype=np.float32), K, scale=s)
        assert list(got_i[0]) == idx, (lg, got_i)
        np.testing.assert_allclose(got_w[0], w, rtol=1e-6)


def test_route_topk_matches_library_sort_with_ties(orc):
    rng = np.random.default_rng(11)
    T, E, K = 300, 64, 8
    lg = np.round(rng.standard_normal((T, E)), 1).astype(np.float32)  # many exact ties
    lg[::7, 3] = -0.0
    lg[::7, 5] = 0.0
    idx, _ = orc.route_from_logits(lg, K, scale=2.827)
    for t in range(T):
        ref = sorted(range(E), key=lambda e: (-float(lg[t, e]), e))[:K]
        assert list(idx[t]) == ref


def test_softmax_closed_forms(orc):
    # uniform logits -> p = 1/E
    E = 32
    _, _, p = orc.route_from_logits(np.full((2, E), 0.75, np.float32), 4, want_probs=True)
    np.testing.assert_allclose(p, 1.0 / E, rtol=1e-14)
    # E = 2 -> p0 = sigmoid(l0 - l1); with K = E and renorm, w = s * p
    lg = np.array([[0.3, -1.2], [4.0, 4.5], [-20.0, 3.0]], np.float32)
    idx, w, p = orc.route_from_logits(lg, 2, scale=2.827, want_probs=True)
    for t in range(3):
        d = float(lg[t, 0]) - float(lg[t, 1])
        p0 = 1.0 / (1.0 + math.exp(-d))
        np.testing.assert_allclose(p[t], [p0, 1.0 - p0], rtol=1e-12)
        np.testing.assert_allclose(w[t], 2.827 * p[t, idx[t]], rtol=1e-6)
    # without renormalisation the weights are the plain probabilities times the scale
    idx, w, p = orc.route_from_logits(lg, 1, scale=1.0, norm_topk=False, want_probs=True)
    for t in range(3):
        assert w[t, 0] == np.float32(p[t].max())


def test_renorm_scale_invariants(orc):
    rng = np.random.default_rng(5)
    T, E, K, s = 200, 256, 8, 2.827
    lg = (rng.standard_normal((T, E)) * 0.47).astype(np.float32)
    idx, w = orc.route_from_logits(lg, K, scale=s)
    np.testing.assert_allclose(w.astype(np.float64).sum(1), s, rtol=1e-6)
    # closed form of renormalised softmax over the selected set: s * e^{l_j} / sum_top e^{l_i}
    for t in range(0, T, 17):
        sel = lg[t, idx[t]].astype(np.float64)
        ref = s * np.exp(sel - sel.max()) / np.exp(sel - sel.max()).sum()
        np.testing.assert_allclose(w[t], ref, rtol=2e-7)
    # weights are decreasing with slot order
    assert np.all(np.diff(w, axis=1) <= 0)
    # perturbing an unselected logit (kept below the k-th) changes no weight beyond rounding
    lg2 = lg.copy()
    for t in range(T):
        others = np.setdiff1d(np.arange(E), idx[t])
        kth = lg[t, idx[t, -1]]
        lg2[t, others[0]] = min(lg2[t, others[0]] - 3.0, kth - 1.0)
    idx2, w2 = orc.route_from_logits(lg2, K, scale=s)
    np.testing.assert_array_equal(idx2, idx)
    np.testing.assert_allclose(w2, w, rtol=3e-7)


# ----------------------------------------------------------------------------- dispatch
def test_dispatch_matches_stable_sort(orc):
    rng = np.random.default_rng(9)
    T, K, E = 777, 8, 256
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    counts, offsets, r2s, s2r = orc.dispatch(idx, E)
    flat = idx.ravel()
    ref = np.argsort(flat, kind="stable")  # library stable sort of slot ids by expert
    np.testing.assert_array_equal(r2s, ref)
    np.testing.assert_array_equal(counts, np.bincount(flat, minlength=E))
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    assert offsets[-1] == T * K
    # bijection: slot_to_row o row_to_slot = id
    np.testing.assert_array_equal(s2r[r2s], np.arange(T * K))
    # slot ids strictly increase inside each expert segment
    for e in range(E):
        seg = r2s[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(flat[seg] == e)


def test_dispatch_capacity_golden(orc):
    d = {}
    with open(os.path.join(GOLDEN, "capacity_drop.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                key, *vals = line.split()
                d[key] = [int(v) for v in vals]
    T, K, E, C = d["T"][0], d["K"][0], d["E"][0], d["C"][0]
    counts, offsets, r2s, s2r = orc.dispatch(np.array(d["topk_idx"], np.int32).reshape(T, K), E, C)
    assert list(counts) == d["counts"]
    assert list(offsets) == d["offsets"]
    assert list(r2s) == d["row_to_slot"]
    assert list(s2r) == d["slot_to_row"]


def test_dispatch_capacity_invariants(orc):
    rng = np.random.default_rng(13)
    T, K, E = 500, 2, 16
    pop = np.exp(-0.4 * np.arange(E))
    idx = np.stack([rng.choice(E, K, replace=False, p=pop / pop.sum()) for _ in range(T)]).astype(np.int32)
    C = 40
    counts, offsets, r2s, s2r = orc.dispatch(idx, E, C)
    flat = idx.ravel()
    full = np.bincount(flat, minlength=E)
    np.testing.assert_array_equal(counts, np.minimum(full, C))
    assert (s2r < 0).sum() == T * K - counts.sum()
    for e in range(E):
        slots = np.nonzero(flat == e)[0]
        kept = r2s[offsets[e]:offsets[e + 1]]
        np.testing.assert_array_equal(kept, slots[:C])  # first C in (token, slot) order
        assert np.all(s2r[slots[C:]] == -1)
    assert np.all(r2s[offsets[-1]:] == -1)


# ----------------------------------------------------------------------------- expert FFN
def _f64(u16):
    return torch.from_numpy((np.asarray(u16, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64))


def _bf16_torch(t64):
    return t64.to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _rand_bf16(rng, shape, std):
    return torch.from_numpy((rng.standard_normal(shape) * std).astype(np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _ulp_close(a_u16, b_u16, max_ulps=1):
    a = np.asarray(a_u16, np.uint16).astype(np.int32)
    b = np.asarray(b_u16, np.uint16).astype(np.int32)
    # map sign-magnitude bit patterns to a monotone integer line
    a = np.where(a & 0x8000, -(a & 0x7FFF), a)
    b = np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(a - b) <= max_ulps


@pytest.mark.parametrize("limit", [10.0, 0.0])
def test_single_expert_equals_dense_swiglu_ffn(orc, limit):
    """E=1, k=1, no shared expert: the layer is a dense SwiGLU FFN (PyTorch float64 pin)."""
    rng = np.random.default_rng(21)
    T, H, I = 24, 64, 96
    x = _rand_bf16(rng, (T, H), 1.0)
    wr = _rand_bf16(rng, (1, H), 0.02)
    wg = _rand_bf16(rng, (1, I, H), 1.0)   # g ~ N(0, 8^2): the clamp fires often
    wu = _rand_bf16(rng, (1, I, H), 1.0)
    wd = _rand_bf16(rng, (1, H, I), 0.05)
    r = orc.layer_forward(x, wr, wg, wu, wd, 1, scale=1.0, limit=limit)
    X, G, U, D = _f64(x), _f64(wg[0]), _f64(wu[0]), _f64(wd[0])
    # the projections are fp32 values: float64 matmuls rounded to float32 (the order of a float64
    # sum moves it by ~1e-16 relative, far from any fp32 or bf16 rounding boundary here)
    g, u = (X @ G.T).float().double(), (X @ U.T).float().double()
    if limit > 0:
        assert (g.abs() > limit).any(), "test inputs must exercise the clamp"
        g, u = g.clamp(-limit, limit), u.clamp(-limit, limit)
    h_ref = torch.nn.functional.silu(g) * u
    h_ref_b = _bf16_torch(h_ref)
    np.testing.assert_array_equal(r["h_routed"], h_ref_b)
    y_ref = (_f64(r["h_routed"]) @ D.T).float()  # same bf16 h on both sides
    y_ref_b = y_ref.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(r["y_routed"], y_ref_b)
    # the fp32 rounding of g, u and y is a step of its own: a reference that skips it differs
    h_direct = _bf16_torch(torch.nn.functional.silu((X @ G.T).clamp(-limit, limit) if limit > 0 else X @ G.T)
                           * ((X @ U.T).clamp(-limit, limit) if limit > 0 else X @ U.T))
    assert _ulp_close(r["h_routed"], h_direct).all()
    # with one expert, k = 1 and s = 1 the renormalised weight is exactly 1 and out == y
    assert np.all(r["topk_idx"] == 0) and np.all(r["topk_w"] == 1.0)
    np.testing.assert_array_equal(r["out"], r["y_routed"])


def test_single_expert_with_shared_expert(orc):
    rng = np.random.default_rng(22)
    T, H, I = 16, 64, 64
    x = _rand_bf16(rng, (T, H), 1.0)
    wr = _rand_bf16(rng, (1, H), 0.02)
    w = [_rand_bf16(rng, s, 0.1) for s in ((1, I, H), (1, I, H), (1, H, I))]
    sw = [_rand_bf16(rng, s, 0.1) for s in ((I, H), (I, H), (H, I))]
    r = orc.layer_forward(x, wr, *w, 1, sg=sw[0], su=sw[1], sd=sw[2], scale=2.827, limit=10.0)
    X = _f64(x)

    def ffn(G, U, D):
        h = _bf16_torch(torch.nn.functional.silu((X @ _f64(G).T).clamp(-10, 10)) * (X @ _f64(U).T).clamp(-10, 10))
        return _bf16_torch(_f64(h) @ _f64(D).T)

    y1, ys = ffn(w[0][0], w[1][0], w[2][0]), ffn(*sw)
    out_ref = 2.827 * _f64(y1) + _f64(ys)
    ref = out_ref.numpy()
    got = _f64(r["out"]).numpy()
    tol = 1e-2 * np.abs(ref) + 1e-3 * np.sqrt((ref ** 2).mean())
    assert np.all(np.abs(got - ref) <= tol)


def test_clamp_closed_form(orc):
    # x = [1, 1]; gate/up rows chosen so that g, u = +-32 (far beyond the limit 10) or small
    x = np.array([[0x3F80, 0x3F80]], np.uint16)
    b16 = lambda v: orc.bf16_from_double(v)
    wg = np.array([[b16(16), b16(16)], [b16(-16), b16(-16)], [b16(1), b16(2)], [b16(16), b16(16)]], np.uint16)
    wu = np.array([[b16(16), b16(16)], [b16(16), b16(16)], [b16(1), b16(1)], [b16(-0.5), b16(0)]], np.uint16)
    h = orc.gateup_rows(x, wg, wu, 10.0)[0]
    silu = lambda v: v / (1.0 + math.exp(-v))
    expect = [10 * silu(10), 10 * silu(-10), 2 * silu(3), -0.5 * silu(10)]
    assert list(h) == [brute_bf16(v) for v in expect]
    assert h[0] == 0x42C8  # 10*silu(10) = 99.9954... rounds to 100.0
    h_off = orc.gateup_rows(x, wg, wu, 0.0)[0]  # limit disabled
    expect_off = [32 * silu(32), 32 * silu(-32), 2 * silu(3), -0.5 * silu(32)]
    assert list(h_off) == [brute_bf16(v) for v in expect_off]


def test_zero_input_routes_to_first_experts(orc):
    T, H, E, K, I = 5, 32, 8, 3, 16
    rng = np.random.default_rng(1)
    x = np.zeros((T, H), np.uint16)
    ws = [_rand_bf16(rng, s, 0.1) for s in ((E, H), (E, I, H), (E, I, H), (E, H, I))]
    sw = [_rand_bf16(rng, s, 0.1) for s in ((I, H), (I, H), (H, I))]
    r = orc.layer_forward(x, *ws, K, sg=sw[0], su=sw[1], sd=sw[2], scale=2.827)
    assert np.all(r["topk_idx"] == np.arange(K))
    np.testing.assert_allclose(r["topk_w"], 2.827 / K, rtol=1e-7)
    assert np.all((r["out"] & 0x7FFF) == 0)  # FFN(0) = 0, no biases


# ----------------------------------------------------------------------------- whole layer
def _tiny_inputs(T=64, H=128, E=16, K=4, I=64, seed=0, with_shared=True):
    rng = np.random.default_rng(seed)
    x = _rand_bf16(rng, (T, H), 1.0)
    wr = _rand_bf16(rng, (E, H), 0.05)
    wg, wu = _rand_bf16(rng, (E, I, H), 0.05), _rand_bf16(rng, (E, I, H), 0.05)
    wd = _rand_bf16(rng, (E, H, I), 0.05)
    sw = [_rand_bf16(rng, s, 0.05) for s in ((I, H), (I, H), (H, I))] if with_shared else [None] * 3
    return x, wr, wg, wu, wd, sw


@pytest.mark.parametrize("capacity", [0, 9])
def test_sparse_equals_dense_bruteforce(orc, capacity):
    x, wr, wg, wu, wd, sw = _tiny_inputs()
    K = 4
    r = orc.layer_forward(x, wr, wg, wu, wd, K, sg=sw[0], su=sw[1], sd=sw[2], scale=2.827,
                          limit=10.0, capacity=capacity)
    if capacity:
        assert (r["slot_to_row"] < 0).any(), "capacity case must drop something"
    dense = orc.layer_dense(x, wg, wu, wd, r["topk_idx"], r["topk_w"], r["slot_to_row"],
                            sg=sw[0], su=sw[1], sd=sw[2], limit=10.0)
    np.testing.assert_array_equal(r["out"], dense)


def test_layer_invariants_and_same_logits_mode(orc):
    x, wr, wg, wu, wd, sw = _tiny_inputs(T=50, E=16, K=4, seed=3)
    r = orc.layer_forward(x, wr, wg, wu, wd, 4, sg=sw[0], su=sw[1], sd=sw[2], scale=2.827)
    np.testing.assert_allclose(r["topk_w"].astype(np.float64).sum(1), 2.827, rtol=1e-6)
    assert r["counts"].sum() == 50 * 4
    np.testing.assert_array_equal(np.sort(r["row_to_slot"]), np.arange(200))
    r2 = orc.layer_forward(x, wr, wg, wu, wd, 4, sg=sw[0], su=sw[1], sd=sw[2], scale=2.827,
                           logits=r["logits"])
    for key in ("topk_idx", "topk_w", "counts", "row_to_slot", "y_routed", "out"):
        np.testing.assert_array_equal(r[key], r2[key])


def test_router_logits_against_float64_matmul(orc):
    rng = np.random.default_rng(4)
    T, H, E = 40, 256, 24
    x, wr = _rand_bf16(rng, (T, H), 1.0), _rand_bf16(rng, (E, H), 0.02)
    bias = (1.2 * np.log(1.0 / (np.arange(E) + 1.0))).astype(np.float32)
    lg = orc.router_logits(x, wr, bias)
    # fp32 logit (float64 matmul rounded to float32), then the bias as a float32 add
    ref = (_f64(x) @ _f64(wr).T).numpy().astype(np.float32) + bias
    np.testing.assert_array_equal(lg, ref)
    # the token subset mode writes only the listed rows
    lg2 = orc.router_logits(x, wr, bias, tokens=[3, 17])
    np.testing.assert_array_equal(lg2[[3, 17]], lg[[3, 17]])
    assert np.all(lg2[0] == 0)


def test_oracle_is_deterministic_across_thread_counts(orc):
    # every output element is one sequential sum, so the thread count cannot change a bit
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r); import numpy as np, oracle;"
            "from tests.test_oracle_pins import _tiny_inputs;"
            "x, wr, wg, wu, wd, sw = _tiny_inputs(T=33, seed=8);"
            "r = oracle.layer_forward(x, wr, wg, wu, wd, 4, sg=sw[0], su=sw[1], sd=sw[2], scale=2.827);"
            "sys.stdout.write(r['out'].tobytes().hex()[:4000] + str(int(r['out'].astype(np.int64).sum())))"
            % os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    outs = []
    for nt in ("1", "5"):
        env = dict(os.environ, OMP_NUM_THREADS=nt)
        outs.append(subprocess.run([sys.executable, "-c", code], env=env, capture_output=True,
                                   text=True, check=True).stdout)
    assert outs[0] == outs[1]
