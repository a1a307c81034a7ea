"""Helpers shared by the GPU parity tests: a-priori rounding-interval checks and GPU/oracle runners.

How a bf16 tensor of the GPU is compared with the oracle
---------------------------------------------------------
Every stored bf16 tensor (h, y, y_shared, out) is the round-to-nearest-even of a value that both
sides compute from the same bf16/fp32 inputs: the oracle exactly (sequential double sums, fp32
rounding of each projection), the GPU in fp32. For every element the test computes

  v   the oracle's value before the bf16 rounding (rebuilt here from the oracle's inputs with
      float64 matmuls and checked to round to the oracle's own bf16 output), and
  d   an a-priori bound on |GPU pre-rounding value - v|, from the arithmetic alone:
        * a projection's fp32 chain (see Chain and chain_sums): a bf16 matrix-core instruction
          sums groups of 8 products aligned to their largest, then the accumulator and the
          group sums aligned to the largest of them, and rounds once to fp32 nearest even
          (pinned on the GPU by tests/test_gpu_mfma_accumulation.py); every aligned term that
          is not the largest loses less than u times the largest, u = 2^-24, and the rounding
          u |result|; the running sums come from float64 partial sums at the kernel's
          instruction boundaries;
        * one u * |value| per fp32 multiply by a row scale, and for the oracle's own fp32
          rounding of the projection;
        * the SwiGLU's sensitivity to g and u over that interval, plus (|g| + 8) u |h| for the
          GPU's fp32 evaluation of exp, the division and the product;
        * the combine's fp32 sum: u times the running sums and products in slot order;
        * in the end-to-end comparison (the oracle's own chain), the upstream differences that
          were themselves checked first: each bf16 element where the GPU's h (or y) differs from
          the oracle's, by the amount it differs (|dh| |Wd| for y; |w| |dy|, |dw| |y| and the
          shared row for out), and nothing else.
and requires the GPU's bf16 value to lie in [RNE(v - d), RNE(v + d)]. Where that interval holds
one value (almost everywhere) the GPU must equal the oracle bit for bit; only elements whose v
lies within d of a rounding midpoint (the flip set) may differ, and by no more than the interval
allows. The benchmark spec bound |gpu - oracle| <= 1e-2 |oracle| + 1e-3 rms(oracle) is asserted on
every element outside the flip set (it follows from bit equality) and reported inside it.

Chained comparisons (each stage from the GPU's own inputs of that stage) use the same intervals
with no upstream term. fp32 router logits: |gpu - oracle| <= 1e-4 rms(oracle) + 1e-5 |oracle|;
fp32 routing weights: |gpu - oracle| <= 1e-5 routed_scaling; integers: bit-exact.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

import oracle
import sparse_moe_layer_softmax_amd as moe
from sparse_moe_layer_softmax_amd.workloads import as_u16

U = 2.0 ** -24  # fp32 unit roundoff


def f64(u16) -> np.ndarray:
    """bf16 bit patterns -> float64 values (exact; through torch, whose conversion runs on every
    core: the weights of a full-size layer pass through here once per checked group)."""
    a = np.ascontiguousarray(u16, np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


# ----------------------------------------------------------------------------- group checks
def run_pipelined(prepare, check, items, workers: int = 6, window: int = 12):
    """check(prepare(item)) for every item, results in item order. prepare runs here (it may
    copy device tensors to the host); check runs on a thread pool (numpy, torch and the oracle's
    C calls release the interpreter lock in their heavy parts). At most `window` prepared items
    are held at once, which bounds the host memory of full-size layers."""
    import collections
    from concurrent.futures import ThreadPoolExecutor

    out, pending = [], collections.deque()
    with ThreadPoolExecutor(workers) as ex:
        for it in items:
            pending.append(ex.submit(check, prepare(it)))
            while len(pending) >= window:
                out.append(pending.popleft().result())
        while pending:
            out.append(pending.popleft().result())
    return out


# ----------------------------------------------------------------------------- bf16 rounding
def bf16_rne(v) -> np.ndarray:
    """float64 -> bf16 bit patterns, round to nearest, ties to even (vectorised; finite inputs).
    Pinned against the oracle's scalar rounding by tests/test_parity_helpers.py."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    m, e = np.frexp(a)                       # a = m 2^e, m in [0.5, 1)
    q = np.where(a >= 2.0 ** -126, e - 8, -133)  # exponent of the last kept bit
    r = np.ldexp(np.rint(np.ldexp(a, -q)), q)  # rint: ties to even
    with np.errstate(over="ignore"):
        r32 = r.astype(np.float32)             # exact: r is a bf16 value (or overflows to inf)
    bits = (r32.view(np.uint32) >> 16).astype(np.uint16)
    return np.where(np.signbit(v), bits | np.uint16(0x8000), bits).astype(np.uint16)


def ulp_bf16(u16: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at each element (2^(e-7), fixed below the smallest normal)."""
    e = (np.asarray(u16, np.uint16).astype(np.int64) >> 7) & 0xFF
    return np.ldexp(1.0, np.maximum(e, 1) - 127 - 7)


def bare_ok(got_u16, ref_u16):
    """The benchmark spec bound |gpu - oracle| <= 1e-2 |oracle| + 1e-3 rms(oracle), element-wise."""
    g, r = f64(got_u16), f64(ref_u16)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    return np.abs(g - r) <= 1e-2 * np.abs(r) + 1e-3 * rms


class Stats:
    """Per-stage counts: elements, flip candidates (interval of two or more values) and flips
    (GPU differs from the oracle)."""

    def __init__(self):
        self.rows = {}

    def add(self, stage, n, cand, flips, bare_bad=0):
        c = self.rows.setdefault(stage, [0, 0, 0, 0])
        c[0] += n
        c[1] += cand
        c[2] += flips
        c[3] += bare_bad

    def merge(self, other: "Stats") -> None:
        for k, v in other.rows.items():
            self.add(k, *v)

    def line(self) -> str:
        return "; ".join("%s: %d elements, %d candidates, %d flips%s"
                         % (k, v[0], v[1], v[2], (", %d outside the bare bound" % v[3]) if v[3] else "")
                         for k, v in self.rows.items())


def check_interval(got_u16, v, d, what, ref_u16=None, stats=None, stage=None, bare=False):
    """Assert RNE(v - d) <= got <= RNE(v + d) element-wise (bf16 values). With ref_u16 (the
    oracle's bf16 result, RNE of v) count the flips; with bare, also assert the benchmark spec bound
    on every element outside the flip set. Returns the mask of elements where got != ref."""
    got_u16 = np.asarray(got_u16, np.uint16)
    v = np.asarray(v, np.float64)
    d = np.broadcast_to(np.asarray(d, np.float64), v.shape)
    assert got_u16.shape == v.shape, (what, got_u16.shape, v.shape)
    assert np.all(d >= 0) and np.all(np.isfinite(d)), what
    lo, hi = f64(bf16_rne(v - d)), f64(bf16_rne(v + d))
    g = f64(got_u16)
    ok = (g >= lo) & (g <= hi)
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(
            "%s: %d/%d elements outside their a-priori interval; first at %s: gpu=%r oracle "
            "value=%r bound=%r interval=[%r, %r]" % (what, len(bad), ok.size, i, g[i], v[i], d[i],
                                                      lo[i], hi[i]))
    cand = lo != hi
    flips = np.zeros(v.shape, bool)
    if ref_u16 is not None:
        ref_u16 = np.asarray(ref_u16, np.uint16)
        flips = (got_u16 != ref_u16) & ~((got_u16 | ref_u16) & 0x7FFF == 0)  # +0 == -0
        assert not (flips & ~cand).any(), what  # implied by the interval; kept explicit
        bb = 0
        if bare:
            okb = bare_ok(got_u16, ref_u16)
            assert okb[~cand].all(), "%s: bare north_star bound outside the flip set" % what
            bb = int((~okb).sum())
        if stats is not None:
            stats.add(stage or what, v.size, int(cand.sum()), int(flips.sum()), bb)
    return flips


def check_reconstruction(v, ref_u16, what, tol):
    """The float64 value rebuilt here must round to the oracle's own bf16 output, up to `tol`
    (absolute, per element): the rebuilt sums run in another order than the oracle's
    sequential double sums (and may then round to the other fp32 neighbour)."""
    ref_u16 = np.asarray(ref_u16, np.uint16)
    lo, hi = f64(bf16_rne(v - tol)), f64(bf16_rne(v + tol))
    r = f64(ref_u16)
    ok = (r >= lo) & (r <= hi)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError("%s: rebuilt value %r (tol %r) does not round to the oracle's %r"
                             % (what, v[i], np.broadcast_to(tol, v.shape)[i], r[i]))


def sum_tol(S, Aabs):
    """Tolerance of a rebuilt float64 projection against the oracle's fp32 value of it: the
    order of a double sum (2^-40 of the absolute terms) and, where that straddles an fp32
    rounding midpoint, one fp32 step."""
    t = 2.0 ** -40 * Aabs + 1e-300
    amb = fl32(S - t) != fl32(S + t)
    return t + np.where(amb, U * np.abs(S) * 2.0, 0.0)


# ----------------------------------------------------------------------------- fp32 chains
@dataclass(frozen=True)
class Chain:
    """How a projection kernel accumulates in fp32. K is consumed in aligned blocks of `block`
    elements in ascending order; each block takes `per_block` instructions of `span` products
    (per_block 1: the instruction is the block, so the running sums at instruction ends are the
    block-end sums; more: the kernel's K order inside a block is a permutation, and every running
    sum inside the block is bounded by the block's start sum plus the block's absolute products).
    An instruction aligns its products in groups of `group` consecutive K elements, then the
    accumulator and the group sums, each alignment keeping `guard` bits below the fp32
    significand (bf16 MFMAs: groups of 8, one guard bit or more, pinned; the FP8 MFMA is not
    pinned to a model and is charged from measurement, see CHAINS). `scale_mults` fp32
    multiplies by per-row scales follow the chain."""
    block: int
    per_block: int = 1
    span: int = 16
    group: int = 8
    guard: int = 1
    scale_mults: int = 0


CHAINS = {
    # LDS-tiled kernel: MFMA 32x32x16 bf16, one instruction per contiguous 16-element K step
    "tiled": Chain(16, 1, 16),
    # weight-streaming kernel: MFMA 16x16x32 bf16, one instruction per contiguous 32 elements
    "skinny": Chain(32, 1, 32),
    # FP8 weights decoded to bf16, then the same MFMAs: the tiled kernel's two instructions per
    # 32-element slice and the weight-streaming kernel's four per 128-element block take
    # permuted 8-element chunks; one fp32 multiply by the weight-row scale
    "tiled_w8": Chain(32, 2, 16, scale_mults=1),
    "skinny_w8": Chain(128, 4, 32, scale_mults=1),
    # W8A8: the tiled kernel's FP8 MFMA 32x32x64 (one instruction per 64 codes). No alignment
    # model reproduces it bit for bit; measured on small W8A8 layers, its error reaches 2^-14.6
    # of the sum over instructions of max|a| max|w|. Charged as one alignment group of 64 with
    # granule 2^-18 (63 granules: 2^-12 of the instruction's largest product bound, six times
    # the largest error seen). The weight-streaming kernel decodes both operands to bf16 (W8
    # order). Both then multiply by the weight and row scales.
    "tiled_a8": Chain(64, 1, 64, group=64, guard=-5, scale_mults=2),
    "skinny_a8": Chain(128, 4, 32, scale_mults=2),
    # MX: the tiled kernel's scaled FP8 MFMA applies the block scales inside the instruction, so
    # the chain runs on the dequantised values with no scale multiply after it; its precision is
    # charged as the W8A8 MFMA's (measured). The weight-streaming kernel decodes code * scale to
    # bf16 exactly and runs the bf16 MFMA (W8 order).
    "tiled_mx": Chain(64, 1, 64, group=64, guard=-5, scale_mults=0),
    "skinny_mx": Chain(128, 4, 32, scale_mults=0),
}


def kernel_of(rows_max: int, n_groups: int, train: bool = False) -> str:
    """Which grouped-GEMM kernel a launch takes (the library's rule: the tiled kernel from 64 rows
    per group on average, and always for the training forward)."""
    return "tiled" if train or rows_max >= 64 * n_groups else "skinny"


def chain_for(kern: str, fp8: bool, act_fp8: bool, mx: bool = False) -> Chain:
    return CHAINS[kern + ("_mx" if mx else "_a8" if act_fp8 else "_w8" if fp8 else "")]


def chain_sums(A, W, chain: Chain):
    """Exact sums S = A W^T (float64) and the a-priori bound on |fp32 chain - S| per element, for
    A [n, K], W [m, K] float64 values (dequantised for FP8 operands). With u = 2^-24 and the
    alignment granule gamma = 2^(1 - guard) u (relative to the largest aligned term):
      one instruction j: gamma ((group - 1) sum over its groups of the largest |product|
                         + (span / group) max(|S_{j-1}|, A_j)) + u |S_j|
    (the largest term of each alignment is exact, every other one loses less than a granule; the
    last term is the rounding), summed over the chain. The largest |product| of a group is
    bounded by max|a| max|w| over the group; S_j, A_j are the running sum and the instruction's
    absolute products."""
    A = torch.from_numpy(np.ascontiguousarray(A, np.float64))
    W = torch.from_numpy(np.ascontiguousarray(W, np.float64))
    n, K = A.shape
    m = W.shape[0]
    absW = W.abs()
    S = A @ W.T
    Aabs = A.abs() @ absW.T
    blk, per_block = chain.block, chain.per_block
    assert K % blk == 0 and blk % chain.group == 0, (K, blk, chain.group)
    # long reductions: running sums taken every c instructions only (each instruction's running
    # sum then bounded by its block's start sum plus the block's absolute products), which
    # loosens the bound by about the reduction's absolute products and cuts the work c times
    c = 1
    while K // (blk * c) > 96 and K % (blk * c * 2) == 0:
        c *= 2
    blk, per_block = blk * c, per_block * c
    nb = K // blk
    gamma = 2.0 ** (1 - chain.guard) * U
    # sum over groups of the largest |product| bound max|a| max|w|
    g = chain.group
    XW = A.abs().view(n, -1, g).amax(2) @ absW.view(m, -1, g).amax(2).T
    mg = chain.span // chain.group
    # running sums at block ends, one block product at a time
    run = torch.zeros((n, m), dtype=torch.float64)
    after = torch.zeros((n, m), dtype=torch.float64)  # sum over blocks of |running sum at its end|
    for b in range(nb):
        run += A[:, b * blk:(b + 1) * blk] @ W[:, b * blk:(b + 1) * blk].T
        after += run.abs()
    before = (after - run.abs()).numpy()  # sum over blocks of |running sum at the block's start|
    S, Aabs, XW, after = S.numpy(), Aabs.numpy(), XW.numpy(), after.numpy()
    if per_block == 1:
        acc = gamma * ((chain.group - 1) * XW + mg * (before + Aabs)) + U * after
    else:  # every running sum inside block b is at most |S_{b-1}| + A_b
        acc = gamma * (chain.group - 1) * XW + (gamma * mg + U) * per_block * (before + Aabs)
    d = 1.05 * (acc + U * chain.scale_mults * np.abs(S))
    return S, d, Aabs


# ----------------------------------------------------------------------------- the SwiGLU stage
def fl32(v):
    return np.asarray(v, np.float64).astype(np.float32).astype(np.float64)


def swiglu64(g, u, limit):
    if limit > 0:
        g, u = np.clip(g, -limit, limit), np.clip(u, -limit, limit)
    return g / (1.0 + np.exp(-g)) * u


def swiglu_bound(g, u, dg, du, limit):
    """Bound on |silu(clamp g') clamp u' - silu(clamp g) clamp u| for |g' - g| <= dg,
    |u' - u| <= du (|silu'| <= 1.1 everywhere), plus the GPU's fp32 evaluation error."""
    gc = np.clip(g, -limit, limit) if limit > 0 else g
    uc = np.clip(u, -limit, limit) if limit > 0 else u
    silu = gc / (1.0 + np.exp(-gc))
    h = silu * uc
    return (1.1 * (np.abs(uc) + du) * dg + (np.abs(silu) + 1.1 * dg) * du
            + (np.abs(gc) + 8.0) * U * np.abs(h) + 1e-300)


# ----------------------------------------------------------------------------- weights
def e4m3_f64(codes) -> np.ndarray:
    """float64 values of E4M3 codes (torch's float8_e4m3fn, to which the oracle's own decoding is
    pinned code by code; multithreaded, unlike a table gather)."""
    q = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return q.to(torch.float64).numpy()


def weight_f64(w) -> np.ndarray:
    """Float64 values of a weight matrix: bf16 bit patterns, or an oracle.Fp8 (scale * e4m3;
    the codes decode through torch's float8_e4m3fn, to which the oracle's own decoding is pinned
    code by code)."""
    if isinstance(w, oracle.Fp8):
        q = torch.from_numpy(np.ascontiguousarray(w.q, np.uint8)).view(torch.float8_e4m3fn)
        return (q.to(torch.float64) * torch.from_numpy(w.scale.astype(np.float64))[..., None]).numpy()
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


# ----------------------------------------------------------------------------- stage checks
def h_reference(Sg, Ag, Su, Au, limit):
    """The oracle's h before its bf16 rounding, rebuilt from the float64 gate and up sums (each
    rounded to fp32 as the oracle does), and the tolerance of that rebuild."""
    tg, tu = sum_tol(Sg, Ag), sum_tol(Su, Au)
    g32, u32 = fl32(Sg), fl32(Su)
    vh = swiglu64(g32, u32, limit)
    gc = np.clip(g32, -limit, limit) if limit > 0 else g32
    uc = np.clip(u32, -limit, limit) if limit > 0 else u32
    silu = gc / (1.0 + np.exp(-gc))
    tol = 1.1 * (np.abs(uc) + tu) * tg + (np.abs(silu) + 1.1 * tg) * tu + 1e-15 * np.abs(vh) + 1e-300
    return vh, tol


def _mmT(a, w, absolute=False):
    """a @ w.T in float64 (|a| @ |w|.T with absolute), through torch's multithreaded CPU
    product."""
    ta = torch.from_numpy(np.ascontiguousarray(a, np.float64))
    tw = torch.from_numpy(np.ascontiguousarray(w, np.float64))
    if absolute:
        ta, tw = ta.abs(), tw.abs()
    return (ta @ tw.T).numpy()


def check_ffn_rows(what, x_rows, w3, limit, chain, h_gpu, y_gpu, h_orc=None, y_orc=None,
                   stats=None):
    """One group's rows of the expert FFN (bf16 or FP8 weights, bf16 activations).
    x_rows [n, H] bf16 (the GPU's inputs), w3 = (gate, up, down) in the oracle's form, h_gpu,
    y_gpu the GPU's rows; h_orc, y_orc the oracle's own rows (default: computed here).
    Checks h against the oracle from x (its own chain is the same one: x is an input), y chained
    (from the GPU's h) and end to end (the oracle's y, with the GPU's checked h flips)."""
    x = f64(x_rows)
    wg, wu, wd = (weight_f64(w) for w in w3)
    if h_orc is None or y_orc is None:
        h_orc, y_orc = ffn_rows(x_rows, w3, limit)
    # h: the same bf16 x on both sides
    Sg, dg, Ag = chain_sums(x, wg, chain)
    Su, du, Au = chain_sums(x, wu, chain)
    vh, th = h_reference(Sg, Ag, Su, Au, limit)
    check_reconstruction(vh, h_orc, what + " h", th)
    dh = swiglu_bound(fl32(Sg), fl32(Su), dg + U * np.abs(Sg), du + U * np.abs(Su), limit)
    fh = check_interval(h_gpu, vh, dh, what + " h", h_orc, stats, "h", bare=True)
    # y chained: from the GPU's own h
    hg = f64(h_gpu)
    Syc, dyc, _ = chain_sums(hg, wd, chain)
    check_interval(y_gpu, Syc, dyc, what + " y (chained)", stats=None)
    # y end to end: the oracle's y, widened only by the checked h flips
    ho = f64(h_orc)
    Syo = _mmT(ho, wd)
    vy = fl32(Syo)
    check_reconstruction(vy, y_orc, what + " y", sum_tol(Syo, _mmT(ho, wd, absolute=True)))
    prop = _mmT(np.abs(hg - ho) * fh, wd, absolute=True) if fh.any() else 0.0
    fy = check_interval(y_gpu, vy, dyc + U * np.abs(Syo) + prop, what + " y (end to end)", y_orc,
                        stats, "y", bare=True)
    return fh, fy


def _code_sums(codes, row_scale, w):
    """The oracle's scaled W8A8 projection in float64, in its own order of operations: the exact
    sum of E4M3 code products (small dyadic numbers: exact in any order), times the weight-row
    scale, times the activation-row scale; and the absolute terms."""
    A, Wc = e4m3_f64(codes), e4m3_f64(w.q)
    ws = w.scale.astype(np.float64)[None, :]
    rs = np.asarray(row_scale, np.float64)[:, None]
    return _mmT(A, Wc) * ws * rs, _mmT(A, Wc, absolute=True) * ws * np.abs(rs)


def check_w8a8_rows(what, xq, sx, w3, limit, chain, h_gpu, hq_gpu, sh_gpu, y_gpu, h_orc, hq_orc,
                    sh_orc, y_orc, stats=None):
    """One group's rows of the W8A8 expert FFN. xq, sx: the rows' x codes and scales (the same on
    both sides: checked bit for bit first); hq_gpu, sh_gpu: the GPU's h codes and scales (checked
    bit for bit against the oracle's quantisation of the GPU's h); *_orc: the oracle's own chain.
    h against the oracle from the x codes; y chained from the GPU's h codes and end to end, the
    end-to-end interval widened by the difference of the dequantised h rows, which comes only
    from checked h flips (one flip can move the codes of its element, or the whole row's scale
    when it is the row maximum)."""
    wg, wu, wd = (weight_f64(w) for w in w3)
    A = e4m3_f64(xq) * np.asarray(sx, np.float64)[:, None]
    _, dg, _ = chain_sums(A, wg, chain)
    _, du, _ = chain_sums(A, wu, chain)
    Sg, Ag = _code_sums(xq, sx, w3[0])
    Su, Au = _code_sums(xq, sx, w3[1])
    vh, th = h_reference(Sg, Ag, Su, Au, limit)
    check_reconstruction(vh, h_orc, what + " h", th)
    dh = swiglu_bound(fl32(Sg), fl32(Su), dg + U * np.abs(Sg), du + U * np.abs(Su), limit)
    check_interval(h_gpu, vh, dh, what + " h", h_orc, stats, "h", bare=True)
    Ag8 = e4m3_f64(hq_gpu) * np.asarray(sh_gpu, np.float64)[:, None]
    _, dyc, _ = chain_sums(Ag8, wd, chain)
    Syc, _ = _code_sums(hq_gpu, sh_gpu, w3[2])
    check_interval(y_gpu, Syc, dyc, what + " y (chained)")
    Syo, Ayo = _code_sums(hq_orc, sh_orc, w3[2])
    vy = fl32(Syo)
    check_reconstruction(vy, y_orc, what + " y", sum_tol(Syo, Ayo))
    Ao8 = e4m3_f64(hq_orc) * np.asarray(sh_orc, np.float64)[:, None]
    diff = np.abs(Ag8 - Ao8)
    prop = _mmT(diff, wd, absolute=True) if diff.any() else 0.0
    check_interval(y_gpu, vy, dyc + U * np.abs(Syo) + prop, what + " y (end to end)", y_orc, stats,
                   "y", bare=True)


def check_mx_rows(what, xq, xs, w3, limit, chain, h_gpu, hq_gpu, hs_gpu, y_gpu, h_orc, hq_orc,
                  hs_orc, y_orc, stats=None):
    """check_w8a8_rows for the MX form: xq, xs the rows' x codes and block-scale bytes [n, H/32]
    (the same on both sides, checked bit for bit first); w3 three oracle.Mx weights; hq/hs the h
    codes and scale bytes of each side. The projections run on the dequantised values (every
    product exact), so the sums and their absolute terms are plain float64 matrix products."""
    deq = oracle.mx_dequant
    wg, wu, wd = (deq(w.q, w.s) for w in w3)
    A = deq(xq, xs)
    Sg, dg, Ag = chain_sums(A, wg, chain)
    Su, du, Au = chain_sums(A, wu, chain)
    vh, th = h_reference(Sg, Ag, Su, Au, limit)
    check_reconstruction(vh, h_orc, what + " h", th)
    dh = swiglu_bound(fl32(Sg), fl32(Su), dg + U * np.abs(Sg), du + U * np.abs(Su), limit)
    check_interval(h_gpu, vh, dh, what + " h", h_orc, stats, "h", bare=True)
    Ag8 = deq(hq_gpu, hs_gpu)
    Syc, dyc, _ = chain_sums(Ag8, wd, chain)
    check_interval(y_gpu, Syc, dyc, what + " y (chained)")
    Ao8 = deq(hq_orc, hs_orc)
    Syo, _, Ayo = chain_sums(Ao8, wd, chain)
    vy = fl32(Syo)
    check_reconstruction(vy, y_orc, what + " y", sum_tol(Syo, Ayo))
    diff = np.abs(Ag8 - Ao8)
    prop = _mmT(diff, wd, absolute=True) if diff.any() else 0.0
    check_interval(y_gpu, vy, dyc + U * np.abs(Syo) + prop, what + " y (end to end)", y_orc, stats,
                   "y", bare=True)


def combine_value(w, rows_of_slots, y_rows_f64, ys_f64):
    """sum_j w_j y_j + y_shared in float64 (slot order, kept slots only), the fp32 running-sum
    bound of the GPU's combine, and the sum of the absolute terms. w [T, K] fp32 weights,
    rows_of_slots [T, K] (row or -1), y_rows_f64 indexable by row, ys_f64 [T, H] or None."""
    T, K = w.shape
    H = y_rows_f64.shape[1]
    P = np.zeros((T, H))
    run = np.zeros((T, H))
    absum = np.zeros((T, H))
    for j in range(K):
        rows = rows_of_slots[:, j]
        kept = rows >= 0
        t = w[kept, j:j + 1].astype(np.float64) * y_rows_f64[rows[kept]]
        P[kept] += t
        run[kept] += np.abs(P[kept]) + np.abs(t)
        absum[kept] += np.abs(t)
    if ys_f64 is not None:
        P = P + ys_f64
        run += np.abs(P)
        absum += np.abs(ys_f64)
    return P, U * run * 1.05 + 1e-300, absum


def check_out(what, w_gpu, w_orc, s2r, y_gpu_rows, y_orc_rows, ys_gpu, ys_orc, out_gpu, out_orc,
              stats=None):
    """The combined output of T tokens: chained (the GPU's weights and rows) and end to end (the
    oracle's weights and rows, widened by the checked differences of the weights, of the y rows
    and of the shared rows). s2r [T, K]: row of each slot in y_*_rows (or -1)."""
    yg, yo = f64(y_gpu_rows), f64(y_orc_rows)
    ysg = None if ys_gpu is None else f64(ys_gpu)
    yso = None if ys_orc is None else f64(ys_orc)
    vc, dc, _ = combine_value(w_gpu, s2r, yg, ysg)
    check_interval(out_gpu, vc, dc, what + " out (chained)")
    vo, _, ao = combine_value(w_orc, s2r, yo, yso)
    check_reconstruction(vo, out_orc, what + " out", 2.0 ** -45 * ao + 1e-300)
    T, K = w_gpu.shape
    prop = np.zeros(vo.shape)
    dw = np.abs(w_gpu.astype(np.float64) - w_orc.astype(np.float64))
    dyr = np.abs(yg - yo)
    for j in range(K):
        rows = s2r[:, j]
        kept = rows >= 0
        prop[kept] += dw[kept, j:j + 1] * np.abs(yo[rows[kept]]) + \
            np.abs(w_gpu[kept, j:j + 1].astype(np.float64)) * dyr[rows[kept]]
    if ysg is not None:
        prop += np.abs(ysg - yso)
    return check_interval(out_gpu, vo, dc + prop, what + " out (end to end)", out_orc, stats,
                          "out", bare=True)


# ----------------------------------------------------------------------------- older helpers
def bf16_close(got_u16, ref_u16, extra=None):
    g, r = f64(got_u16), f64(ref_u16)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    tol = 1e-2 * np.abs(r) + 1e-3 * rms
    if extra is not None:
        tol = tol + extra
    ok = np.abs(g - r) <= tol
    return ok, g, r, tol


def assert_bf16_close(got_u16, ref_u16, what, extra=None):
    """The benchmark spec bound alone (used for the training tensors, whose tolerances their own
    files derive)."""
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


def mx_planes_to_rows(planes, rows):
    """MX scale planes [K/128][plane_rows][4] -> per-row scale bytes [rows][K/32]."""
    return np.ascontiguousarray(planes[:, :rows, :].transpose(1, 0, 2).reshape(rows, -1))


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
    if layer.mx:  # the block-quantised activations: codes, and scale planes by GEMM row
        sr = layer.layout["scale_rows"]
        g["xq"] = layer.intermediate("xq", torch.uint8, (T, H)).cpu().numpy()
        g["hq"] = layer.intermediate("hq", torch.uint8, (rows, I)).cpu().numpy()
        g["x_scale"] = mx_planes_to_rows(
            layer.intermediate("x_scale", torch.uint8, (H // 128, sr, 4)).cpu().numpy(), rows)
        g["h_scale"] = mx_planes_to_rows(
            layer.intermediate("h_scale", torch.uint8, (I // 128, sr, 4)).cpu().numpy(), rows)
    elif layer.act_fp8:  # the quantised activations (W8A8)
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


def compare_layer(wl, hw: dict, g: dict, r: dict, check_routing_bits: bool = True, train=False,
                  stats=None):
    """Element-wise comparison of a GPU layer run with the oracle run from the same logits: the
    routing integers bit for bit, the weights within 1e-5 s, and every bf16 tensor within its
    a-priori rounding interval (see the module docstring). Returns the Stats."""
    stats = stats or Stats()
    if check_routing_bits:
        for k in ("topk_idx", "counts", "offsets", "row_to_slot", "slot_to_row"):
            np.testing.assert_array_equal(g[k], r[k], err_msg=k)
    np.testing.assert_allclose(g["topk_w"], r["topk_w"], rtol=0, atol=1e-5 * max(wl.scale, 1e-30))
    T, K, E = wl.T, wl.K, wl.E
    R = int(r["offsets"][-1])
    off = r["offsets"]
    n_groups = E + (1 if wl.n_shared else 0)
    chain = chain_for(kernel_of(T * K + (T if wl.n_shared else 0), n_groups, train), is_fp8(hw),
                      False)
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if a == b:
            continue
        x_rows = hw["x"][r["row_to_slot"][a:b] // K]
        check_ffn_rows("expert %d" % e, x_rows, routed_weights(hw, e), wl.limit, chain,
                       g["h_routed"][a:b], g["y_routed"][a:b], r["h_routed"][a:b],
                       r["y_routed"][a:b], stats)
    if wl.n_shared:
        check_ffn_rows("shared", hw["x"], shared_weights(hw), wl.limit, chain, g["h_shared"],
                       g["y_shared"], r["h_shared"], r["y_shared"], stats)
    s2r = g["slot_to_row"].reshape(T, K)
    check_out("layer", g["topk_w"], r["topk_w"], s2r, g["y_routed"][:max(R, 1)],
              r["y_routed"][:max(R, 1)], g["y_shared"], r.get("y_shared"), g["out"], r["out"], stats)
    print("[parity] %s: %s" % (wl.name, stats.line()), flush=True)
    return stats
