"""CPU oracle for the sparse MoE FFN layer forward (ctypes wrapper of ``libmoe_oracle.so``).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It never imports the HIP library and the HIP library
never imports it. The arithmetic is in ``moe_oracle.cpp``; this file only marshals numpy
arrays (bf16 tensors are ``uint16`` bit patterns, row-major).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "moe_oracle.cpp"), os.path.join(_HERE, "moe_oracle_bwd.cpp"),
         os.path.join(_HERE, "moe_oracle_w8a8.cpp"), os.path.join(_HERE, "moe_oracle_mx.cpp")]
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with g++ (OpenMP, no fast-math, no FMA contraction)."""
    deps = _SRCS + [os.path.join(_HERE, "moe_oracle.h")]
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < max(
        os.path.getmtime(f) for f in deps
    ):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["g++", "-O2", "-std=c++17", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
               *_SRCS, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        build()
        _lib = ctypes.CDLL(_LIB_PATH)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I = ctypes.c_int
_D = ctypes.c_double


def _declare(L):
    L.oracle_bf16_from_double.argtypes = [_D]
    L.oracle_bf16_from_double.restype = ctypes.c_uint16
    L.oracle_double_from_bf16.argtypes = [ctypes.c_uint16]
    L.oracle_double_from_bf16.restype = _D
    L.oracle_router_logits.argtypes = [_I, _I, _I, _P, _P, _P, _P, _I, _P]
    L.oracle_route_from_logits.argtypes = [_I, _I, _I, _I, _D, _P, _P, _P, _P]
    L.oracle_dispatch.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _P]
    L.oracle_gateup_rows.argtypes = [_I, _I, _I, _D, _P, _P, _P, _P]
    L.oracle_down_rows.argtypes = [_I, _I, _I, _P, _P, _P]
    L.oracle_combine.argtypes = [_I, _I, _I, _P, _P, _P, _P, _P]
    L.oracle_layer_forward.argtypes = [_I, _I, _I, _I, _I, _I, _D, _D, _I] + [_P] * 9 + [_I] + [_P] * 12
    L.oracle_layer_dense.argtypes = [_I, _I, _I, _I, _I, _D] + [_P] * 11
    L.oracle_double_from_e4m3.argtypes = [ctypes.c_uint8]
    L.oracle_double_from_e4m3.restype = _D
    L.oracle_gateup_rows_fp8.argtypes = [_I, _I, _I, _D] + [_P] * 6
    L.oracle_down_rows_fp8.argtypes = [_I, _I, _I] + [_P] * 4
    L.oracle_layer_forward_fp8.argtypes = [_I, _I, _I, _I, _I, _I, _D, _D, _I] + [_P] * 15 + [_I] + [_P] * 12
    L.oracle_layer_dense_fp8.argtypes = [_I, _I, _I, _I, _I, _D] + [_P] * 17
    L.oracle_router_train_stats.argtypes = [_I, _I, _I, _P, _P, _D, _P, _P, _P, _P, _P]
    L.oracle_combine_bwd.argtypes = [_I, _I, _I, _I] + [_P] * 6
    L.oracle_down_bwd_rows.argtypes = [_I, _I, _I, _I, _P, _P, _P]
    L.oracle_swiglu_bwd_rows.argtypes = [_I, _I, _I, _D, _I] + [_P] * 6
    L.oracle_gateup_dgrad_rows.argtypes = [_I, _I, _I, _I] + [_P] * 5
    L.oracle_wgrad.argtypes = [_I, _I, _I, _P, _P, _P]
    L.oracle_router_bwd.argtypes = [_I, _I, _I, _I, _D, _P, _P, _P, _D, _P]
    L.oracle_layer_backward.argtypes = [_I] * 6 + [_D, _D, _I] + [_P] * 16 + [_D] + [_P] * 15
    L.oracle_num_threads.restype = _I
    L.oracle_set_num_threads.argtypes = [_I]
    L.oracle_set_num_threads.restype = None
    L.oracle_e4m3_from_float_array.argtypes = [ctypes.c_long, _P, _P]
    L.oracle_quant_rows_e4m3.argtypes = [_I, _I, _P, _P, _P]
    L.oracle_gateup_rows_w8a8.argtypes = [_I, _I, _I, _D] + [_P] * 7
    L.oracle_down_rows_w8a8.argtypes = [_I, _I, _I] + [_P] * 5
    L.oracle_layer_forward_w8a8.argtypes = ([_I, _I, _I, _I, _I, _I, _D, _D, _I] + [_P] * 15 + [_I]
                                            + [_P] * 14)
    L.oracle_mx_scale_of_amax.argtypes = [_D]
    L.oracle_mx_scale_of_amax.restype = ctypes.c_uint8
    L.oracle_mx_quant_rows.argtypes = [_I, _I, _P, _P, _P]
    L.oracle_mx_dequant.argtypes = [_I, _I, _P, _P, _P]
    L.oracle_gateup_rows_mx.argtypes = [_I, _I, _I, _D] + [_P] * 7
    L.oracle_down_rows_mx.argtypes = [_I, _I, _I] + [_P] * 5
    L.oracle_layer_forward_mx.argtypes = ([_I, _I, _I, _I, _I, _I, _D, _D, _I] + [_P] * 15 + [_I]
                                          + [_P] * 14)


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a):
    return np.ascontiguousarray(a, dtype=np.uint16)


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    """Threads of the following oracle calls (its results do not depend on the count)."""
    lib().oracle_set_num_threads(int(n))


def bf16_from_double(v: float) -> int:
    return int(lib().oracle_bf16_from_double(float(v)))


def double_from_bf16(b: int) -> float:
    return float(lib().oracle_double_from_bf16(int(b)))


def bf16_round_array(a: np.ndarray) -> np.ndarray:
    """Element-wise oracle bf16 rounding of a float64 array (slow; for small arrays)."""
    f = lib().oracle_bf16_from_double
    flat = np.asarray(a, dtype=np.float64).ravel()
    return np.array([f(float(v)) for v in flat], dtype=np.uint16).reshape(np.shape(a))


def router_logits(x, wr, bias=None, tokens=None):
    x, wr = _u16(x), _u16(wr)
    T, H = x.shape
    E = wr.shape[0]
    logits = np.zeros((T, E), dtype=np.float32)
    tok = None if tokens is None else _i32(tokens)
    lib().oracle_router_logits(T, H, E, _ptr(x), _ptr(wr), _ptr(_f32(bias)), _ptr(tok),
                               0 if tok is None else len(tok), _ptr(logits))
    return logits


def route_from_logits(logits, K, scale=1.0, norm_topk=True, want_probs=False):
    logits = _f32(logits)
    T, E = logits.shape
    idx = np.zeros((T, K), dtype=np.int32)
    w = np.zeros((T, K), dtype=np.float32)
    probs = np.zeros((T, E), dtype=np.float64) if want_probs else None
    lib().oracle_route_from_logits(T, E, K, int(bool(norm_topk)), float(scale), _ptr(logits),
                                   _ptr(idx), _ptr(w), _ptr(probs))
    return (idx, w, probs) if want_probs else (idx, w)


def dispatch(topk_idx, E, capacity=0):
    topk_idx = _i32(topk_idx)
    T, K = topk_idx.shape
    counts = np.zeros(E, dtype=np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    r2s = np.zeros(T * K, dtype=np.int32)
    s2r = np.zeros(T * K, dtype=np.int32)
    lib().oracle_dispatch(T, K, E, int(capacity), _ptr(topk_idx), _ptr(counts), _ptr(offsets),
                          _ptr(r2s), _ptr(s2r))
    return counts, offsets, r2s, s2r


def gateup_rows(x_rows, wg, wu, limit):
    x_rows, wg, wu = _u16(x_rows), _u16(wg), _u16(wu)
    n, H = x_rows.shape
    I = wg.shape[0]
    h = np.zeros((n, I), dtype=np.uint16)
    if n:
        lib().oracle_gateup_rows(n, H, I, float(limit), _ptr(x_rows), _ptr(wg), _ptr(wu), _ptr(h))
    return h


def down_rows(h, wd):
    h, wd = _u16(h), _u16(wd)
    n, I = h.shape
    H = wd.shape[0]
    y = np.zeros((n, H), dtype=np.uint16)
    if n:
        lib().oracle_down_rows(n, H, I, _ptr(h), _ptr(wd), _ptr(y))
    return y


def expert_ffn_rows(x_rows, wg, wu, wd, limit):
    h = gateup_rows(x_rows, wg, wu, limit)
    return h, down_rows(h, wd)


def combine(topk_w, slot_to_row, y_routed, y_shared=None):
    topk_w, slot_to_row, y_routed = _f32(topk_w), _i32(slot_to_row), _u16(y_routed)
    T, K = topk_w.shape
    H = y_routed.shape[1]
    out = np.zeros((T, H), dtype=np.uint16)
    ys = None if y_shared is None else _u16(y_shared)
    lib().oracle_combine(T, K, H, _ptr(topk_w), _ptr(slot_to_row), _ptr(y_routed), _ptr(ys),
                         _ptr(out))
    return out


def layer_forward(x, wr, wg, wu, wd, K, *, bias=None, sg=None, su=None, sd=None, scale=1.0,
                  limit=10.0, capacity=0, norm_topk=True, logits=None):
    """Sparse evaluation of the whole layer; returns a dict of every intermediate.

    When ``logits`` is given the router projection is skipped and those fp32 logits are used
    (the "same logits" mode)."""
    x, wr, wg, wu, wd = _u16(x), _u16(wr), _u16(wg), _u16(wu), _u16(wd)
    T, H = x.shape
    E, I = wg.shape[0], wg.shape[1]
    use_logits = logits is not None
    lg = _f32(logits).copy() if use_logits else np.zeros((T, E), dtype=np.float32)
    r = dict(
        logits=lg,
        topk_idx=np.zeros((T, K), dtype=np.int32),
        topk_w=np.zeros((T, K), dtype=np.float32),
        counts=np.zeros(E, dtype=np.int32),
        offsets=np.zeros(E + 1, dtype=np.int32),
        row_to_slot=np.zeros(T * K, dtype=np.int32),
        slot_to_row=np.zeros(T * K, dtype=np.int32),
        h_routed=np.zeros((T * K, I), dtype=np.uint16),
        y_routed=np.zeros((T * K, H), dtype=np.uint16),
        out=np.zeros((T, H), dtype=np.uint16),
    )
    has_shared = sg is not None
    if has_shared:
        sg, su, sd = _u16(sg), _u16(su), _u16(sd)
        r["h_shared"] = np.zeros((T, I), dtype=np.uint16)
        r["y_shared"] = np.zeros((T, H), dtype=np.uint16)
    lib().oracle_layer_forward(
        T, H, E, K, I, int(bool(norm_topk)), float(scale), float(limit), int(capacity),
        _ptr(x), _ptr(wr), _ptr(_f32(bias)), _ptr(wg), _ptr(wu), _ptr(wd),
        _ptr(sg), _ptr(su), _ptr(sd), int(use_logits), _ptr(lg),
        _ptr(r["topk_idx"]), _ptr(r["topk_w"]), _ptr(r["counts"]), _ptr(r["offsets"]),
        _ptr(r["row_to_slot"]), _ptr(r["slot_to_row"]), _ptr(r["h_routed"]), _ptr(r["y_routed"]),
        _ptr(r.get("h_shared")), _ptr(r.get("y_shared")), _ptr(r["out"]))
    return r


def layer_dense(x, wg, wu, wd, topk_idx, topk_w, slot_to_row, *, sg=None, su=None, sd=None,
                limit=10.0):
    x, wg, wu, wd = _u16(x), _u16(wg), _u16(wu), _u16(wd)
    topk_idx, topk_w, slot_to_row = _i32(topk_idx), _f32(topk_w), _i32(slot_to_row)
    T, H = x.shape
    E, I = wg.shape[0], wg.shape[1]
    K = topk_idx.shape[1]
    out = np.zeros((T, H), dtype=np.uint16)
    if sg is not None:
        sg, su, sd = _u16(sg), _u16(su), _u16(sd)
    lib().oracle_layer_dense(T, H, E, K, I, float(limit), _ptr(x), _ptr(wg), _ptr(wu), _ptr(wd),
                             _ptr(sg), _ptr(su), _ptr(sd), _ptr(topk_idx), _ptr(topk_w),
                             _ptr(slot_to_row), _ptr(out))
    return out


# ---------------------------------------------------------------------------- FP8 expert weights
class Fp8:
    """An FP8 weight matrix (or stack of matrices): E4M3 codes ``q`` (uint8, [..., rows, cols]) and
    one fp32 scale per row ``scale`` ([..., rows]); weight value = scale * e4m3(code)."""

    def __init__(self, q, scale):
        self.q = np.ascontiguousarray(np.asarray(q, dtype=np.uint8))
        self.scale = np.ascontiguousarray(np.asarray(scale, dtype=np.float32))
        assert self.scale.shape == self.q.shape[:-1]

    @property
    def shape(self):
        return self.q.shape


def double_from_e4m3(code: int) -> float:
    return lib().oracle_double_from_e4m3(int(code))


def gateup_rows_fp8(x_rows, wg: Fp8, wu: Fp8, limit):
    x_rows = _u16(x_rows)
    n, H = x_rows.shape
    I = wg.q.shape[0]
    h = np.zeros((n, I), dtype=np.uint16)
    if n:
        lib().oracle_gateup_rows_fp8(n, H, I, float(limit), _ptr(x_rows), _ptr(wg.q), _ptr(wg.scale),
                                     _ptr(wu.q), _ptr(wu.scale), _ptr(h))
    return h


def down_rows_fp8(h, wd: Fp8):
    h = _u16(h)
    n, I = h.shape
    H = wd.q.shape[0]
    y = np.zeros((n, H), dtype=np.uint16)
    if n:
        lib().oracle_down_rows_fp8(n, H, I, _ptr(h), _ptr(wd.q), _ptr(wd.scale), _ptr(y))
    return y


def expert_ffn_rows_fp8(x_rows, wg: Fp8, wu: Fp8, wd: Fp8, limit):
    h = gateup_rows_fp8(x_rows, wg, wu, limit)
    return h, down_rows_fp8(h, wd)


def _fp8_ptrs(*ws):
    out = []
    for w in ws:
        out += [None, None] if w is None else [_ptr(w.q), _ptr(w.scale)]
    return out


def layer_forward_fp8(x, wr, wg: Fp8, wu: Fp8, wd: Fp8, K, *, bias=None, sg=None, su=None,
                      sd=None, scale=1.0, limit=10.0, capacity=0, norm_topk=True, logits=None):
    """layer_forward with FP8 expert weights (routed and shared); returns the same dict."""
    x, wr = _u16(x), _u16(wr)
    T, H = x.shape
    E, I = wg.q.shape[0], wg.q.shape[1]
    use_logits = logits is not None
    lg = _f32(logits).copy() if use_logits else np.zeros((T, E), dtype=np.float32)
    r = dict(
        logits=lg,
        topk_idx=np.zeros((T, K), dtype=np.int32),
        topk_w=np.zeros((T, K), dtype=np.float32),
        counts=np.zeros(E, dtype=np.int32),
        offsets=np.zeros(E + 1, dtype=np.int32),
        row_to_slot=np.zeros(T * K, dtype=np.int32),
        slot_to_row=np.zeros(T * K, dtype=np.int32),
        h_routed=np.zeros((T * K, I), dtype=np.uint16),
        y_routed=np.zeros((T * K, H), dtype=np.uint16),
        out=np.zeros((T, H), dtype=np.uint16),
    )
    if sg is not None:
        r["h_shared"] = np.zeros((T, I), dtype=np.uint16)
        r["y_shared"] = np.zeros((T, H), dtype=np.uint16)
    lib().oracle_layer_forward_fp8(
        T, H, E, K, I, int(bool(norm_topk)), float(scale), float(limit), int(capacity),
        _ptr(x), _ptr(wr), _ptr(_f32(bias)), *_fp8_ptrs(wg, wu, wd, sg, su, sd), int(use_logits),
        _ptr(lg), _ptr(r["topk_idx"]), _ptr(r["topk_w"]), _ptr(r["counts"]), _ptr(r["offsets"]),
        _ptr(r["row_to_slot"]), _ptr(r["slot_to_row"]), _ptr(r["h_routed"]), _ptr(r["y_routed"]),
        _ptr(r.get("h_shared")), _ptr(r.get("y_shared")), _ptr(r["out"]))
    return r


def layer_dense_fp8(x, wg: Fp8, wu: Fp8, wd: Fp8, topk_idx, topk_w, slot_to_row, *, sg=None,
                    su=None, sd=None, limit=10.0):
    x = _u16(x)
    topk_idx, topk_w, slot_to_row = _i32(topk_idx), _f32(topk_w), _i32(slot_to_row)
    T, H = x.shape
    E, I = wg.q.shape[0], wg.q.shape[1]
    K = topk_idx.shape[1]
    out = np.zeros((T, H), dtype=np.uint16)
    lib().oracle_layer_dense_fp8(T, H, E, K, I, float(limit), _ptr(x), *_fp8_ptrs(wg, wu, wd, sg, su, sd),
                                 _ptr(topk_idx), _ptr(topk_w), _ptr(slot_to_row), _ptr(out))
    return out


# ------------------------------------------------------- FP8 weights and FP8 activations (W8A8)
def e4m3_from_float(q):
    """Nearest-even OCP E4M3 codes (uint8) of float32 values, saturating at +-448."""
    q = np.ascontiguousarray(np.asarray(q, dtype=np.float32))
    out = np.zeros(q.shape, dtype=np.uint8)
    if q.size:
        lib().oracle_e4m3_from_float_array(q.size, _ptr(q), _ptr(out))
    return out


def quant_rows_e4m3(v):
    """Per-row dynamic E4M3 quantisation of bf16 rows [rows, cols] -> (codes uint8 [rows, cols],
    scales float32 [rows]); value ~= scale * e4m3(code)."""
    v = _u16(v)
    rows, cols = v.shape
    codes = np.zeros((rows, cols), dtype=np.uint8)
    scales = np.zeros(rows, dtype=np.float32)
    if rows:
        lib().oracle_quant_rows_e4m3(rows, cols, _ptr(v), _ptr(codes), _ptr(scales))
    return codes, scales


def gateup_rows_w8a8(xq, sx, wg: Fp8, wu: Fp8, limit):
    xq = np.ascontiguousarray(np.asarray(xq, dtype=np.uint8))
    sx = _f32(sx)
    n, H = xq.shape
    I = wg.q.shape[0]
    h = np.zeros((n, I), dtype=np.uint16)
    if n:
        lib().oracle_gateup_rows_w8a8(n, H, I, float(limit), _ptr(xq), _ptr(sx), _ptr(wg.q),
                                      _ptr(wg.scale), _ptr(wu.q), _ptr(wu.scale), _ptr(h))
    return h


def down_rows_w8a8(hq, sh, wd: Fp8):
    hq = np.ascontiguousarray(np.asarray(hq, dtype=np.uint8))
    sh = _f32(sh)
    n, I = hq.shape
    H = wd.q.shape[0]
    y = np.zeros((n, H), dtype=np.uint16)
    if n:
        lib().oracle_down_rows_w8a8(n, H, I, _ptr(hq), _ptr(sh), _ptr(wd.q), _ptr(wd.scale), _ptr(y))
    return y


def layer_forward_w8a8(x, wr, wg: Fp8, wu: Fp8, wd: Fp8, K, *, bias=None, sg=None, su=None,
                       sd=None, scale=1.0, limit=10.0, capacity=0, norm_topk=True, logits=None):
    """layer_forward_fp8 with the activations of each expert projection quantised per row to
    E4M3; returns the same dict plus the quantised input (xq, x_scale)."""
    x, wr = _u16(x), _u16(wr)
    T, H = x.shape
    E, I = wg.q.shape[0], wg.q.shape[1]
    use_logits = logits is not None
    lg = _f32(logits).copy() if use_logits else np.zeros((T, E), dtype=np.float32)
    r = dict(
        logits=lg,
        topk_idx=np.zeros((T, K), dtype=np.int32),
        topk_w=np.zeros((T, K), dtype=np.float32),
        counts=np.zeros(E, dtype=np.int32),
        offsets=np.zeros(E + 1, dtype=np.int32),
        row_to_slot=np.zeros(T * K, dtype=np.int32),
        slot_to_row=np.zeros(T * K, dtype=np.int32),
        xq=np.zeros((T, H), dtype=np.uint8),
        x_scale=np.zeros(T, dtype=np.float32),
        h_routed=np.zeros((T * K, I), dtype=np.uint16),
        y_routed=np.zeros((T * K, H), dtype=np.uint16),
        out=np.zeros((T, H), dtype=np.uint16),
    )
    if sg is not None:
        r["h_shared"] = np.zeros((T, I), dtype=np.uint16)
        r["y_shared"] = np.zeros((T, H), dtype=np.uint16)
    lib().oracle_layer_forward_w8a8(
        T, H, E, K, I, int(bool(norm_topk)), float(scale), float(limit), int(capacity),
        _ptr(x), _ptr(wr), _ptr(_f32(bias)), *_fp8_ptrs(wg, wu, wd, sg, su, sd), int(use_logits),
        _ptr(lg), _ptr(r["topk_idx"]), _ptr(r["topk_w"]), _ptr(r["counts"]), _ptr(r["offsets"]),
        _ptr(r["row_to_slot"]), _ptr(r["slot_to_row"]), _ptr(r["xq"]), _ptr(r["x_scale"]),
        _ptr(r["h_routed"]), _ptr(r["y_routed"]), _ptr(r.get("h_shared")), _ptr(r.get("y_shared")),
        _ptr(r["out"]))
    return r


# ------------------------------------------------------ MX block-scaled FP8 (MXFP8) operands
MX_BLOCK = 32


class Mx:
    """An MX matrix (or stack of matrices): E4M3 codes ``q`` (uint8, [..., rows, cols]) and E8M0
    scale bytes ``s`` (uint8, [..., rows, cols / 32]); value = e4m3(q) * 2^(s - 127), one scale per
    32 consecutive elements of a row."""

    def __init__(self, q, s):
        self.q = np.ascontiguousarray(np.asarray(q, dtype=np.uint8))
        self.s = np.ascontiguousarray(np.asarray(s, dtype=np.uint8))
        assert self.q.shape[-1] % MX_BLOCK == 0
        assert self.s.shape == self.q.shape[:-1] + (self.q.shape[-1] // MX_BLOCK,)

    @property
    def shape(self):
        return self.q.shape


def mx_scale_of_amax(amax: float) -> int:
    """E8M0 scale byte of a block whose largest magnitude is amax."""
    return int(lib().oracle_mx_scale_of_amax(float(amax)))


def mx_quant_rows(v):
    """MX quantisation of bf16 rows [rows, cols] -> (codes uint8 [rows, cols], scale bytes uint8
    [rows, cols / 32])."""
    v = _u16(v)
    rows, cols = v.shape
    codes = np.zeros((rows, cols), dtype=np.uint8)
    scales = np.zeros((rows, cols // MX_BLOCK), dtype=np.uint8)
    if rows:
        lib().oracle_mx_quant_rows(rows, cols, _ptr(v), _ptr(codes), _ptr(scales))
    return codes, scales


def mx_dequant(codes, scales):
    """Values (float64 [rows, cols]) of MX data."""
    codes = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    scales = np.ascontiguousarray(np.asarray(scales, dtype=np.uint8))
    rows, cols = codes.shape
    out = np.zeros((rows, cols), dtype=np.float64)
    if rows:
        lib().oracle_mx_dequant(rows, cols, _ptr(codes), _ptr(scales), _ptr(out))
    return out


def gateup_rows_mx(xq, xs, wg: Mx, wu: Mx, limit):
    xq = np.ascontiguousarray(np.asarray(xq, dtype=np.uint8))
    xs = np.ascontiguousarray(np.asarray(xs, dtype=np.uint8))
    n, H = xq.shape
    I = wg.q.shape[0]
    h = np.zeros((n, I), dtype=np.uint16)
    if n:
        lib().oracle_gateup_rows_mx(n, H, I, float(limit), _ptr(xq), _ptr(xs), _ptr(wg.q), _ptr(wg.s),
                                    _ptr(wu.q), _ptr(wu.s), _ptr(h))
    return h


def down_rows_mx(hq, hs, wd: Mx):
    hq = np.ascontiguousarray(np.asarray(hq, dtype=np.uint8))
    hs = np.ascontiguousarray(np.asarray(hs, dtype=np.uint8))
    n, I = hq.shape
    H = wd.q.shape[0]
    y = np.zeros((n, H), dtype=np.uint16)
    if n:
        lib().oracle_down_rows_mx(n, H, I, _ptr(hq), _ptr(hs), _ptr(wd.q), _ptr(wd.s), _ptr(y))
    return y


def _mx_ptrs(*ws):
    out = []
    for w in ws:
        out += [None, None] if w is None else [_ptr(w.q), _ptr(w.s)]
    return out


def layer_forward_mx(x, wr, wg: Mx, wu: Mx, wd: Mx, K, *, bias=None, sg=None, su=None, sd=None,
                     scale=1.0, limit=10.0, capacity=0, norm_topk=True, logits=None):
    """The layer with MX expert weights and MX activations; returns the dict of layer_forward_w8a8
    with x_scale the block scale bytes [T, H / 32]."""
    x, wr = _u16(x), _u16(wr)
    T, H = x.shape
    E, I = wg.q.shape[0], wg.q.shape[1]
    use_logits = logits is not None
    lg = _f32(logits).copy() if use_logits else np.zeros((T, E), dtype=np.float32)
    r = dict(
        logits=lg,
        topk_idx=np.zeros((T, K), dtype=np.int32),
        topk_w=np.zeros((T, K), dtype=np.float32),
        counts=np.zeros(E, dtype=np.int32),
        offsets=np.zeros(E + 1, dtype=np.int32),
        row_to_slot=np.zeros(T * K, dtype=np.int32),
        slot_to_row=np.zeros(T * K, dtype=np.int32),
        xq=np.zeros((T, H), dtype=np.uint8),
        x_scale=np.zeros((T, H // MX_BLOCK), dtype=np.uint8),
        h_routed=np.zeros((T * K, I), dtype=np.uint16),
        y_routed=np.zeros((T * K, H), dtype=np.uint16),
        out=np.zeros((T, H), dtype=np.uint16),
    )
    if sg is not None:
        r["h_shared"] = np.zeros((T, I), dtype=np.uint16)
        r["y_shared"] = np.zeros((T, H), dtype=np.uint16)
    lib().oracle_layer_forward_mx(
        T, H, E, K, I, int(bool(norm_topk)), float(scale), float(limit), int(capacity),
        _ptr(x), _ptr(wr), _ptr(_f32(bias)), *_mx_ptrs(wg, wu, wd, sg, su, sd), int(use_logits),
        _ptr(lg), _ptr(r["topk_idx"]), _ptr(r["topk_w"]), _ptr(r["counts"]), _ptr(r["offsets"]),
        _ptr(r["row_to_slot"]), _ptr(r["slot_to_row"]), _ptr(r["xq"]), _ptr(r["x_scale"]),
        _ptr(r["h_routed"]), _ptr(r["y_routed"]), _ptr(r.get("h_shared")), _ptr(r.get("y_shared")),
        _ptr(r["out"]))
    return r


# ---------------------------------------------------------------------------- training side
def router_logits_noisy(x, wr, bias=None, noise=None):
    """Router logits with the training noise added to the scores before the softmax (Hy4
    deep-dive MoERouter, training branch). The noise is drawn by the caller (the page draws
    N(0, 0.01^2) per score) and passed in; logits and noise are added in float64 and rounded to
    float32."""
    lg = router_logits(x, wr, bias)
    if noise is None:
        return lg
    return (lg.astype(np.float64) + _f32(noise).astype(np.float64)).astype(np.float32)


def router_train_stats(logits, topk_idx, decay=0.9, ema_counts=None, ema_tokens=None):
    """Training-side router statistics (Hy3 deep-dive SparseMoERouter training branch): returns
    dict(prob_mean [E], load_frac [E], aux_loss, ema_counts [E] or None, ema_tokens or None),
    all float64; ema_* are the updated averages when initial values are given."""
    logits, topk_idx = _f32(logits), _i32(topk_idx)
    T, E = logits.shape
    K = topk_idx.shape[1]
    pm = np.zeros(E)
    lf = np.zeros(E)
    aux = np.zeros(1)
    ec = None if ema_counts is None else np.ascontiguousarray(np.asarray(ema_counts, np.float64)).copy()
    et = None if ema_tokens is None else np.array([float(ema_tokens)])
    lib().oracle_router_train_stats(T, E, K, _ptr(logits), _ptr(topk_idx), float(decay), _ptr(pm),
                                    _ptr(lf), _ptr(aux), _ptr(ec), _ptr(et))
    return dict(prob_mean=pm, load_frac=lf, aux_loss=float(aux[0]), ema_counts=ec,
                ema_tokens=None if et is None else float(et[0]))


# ---------------------------------------------------------------------------- backward pass
def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def combine_bwd(topk_w, slot_to_row, y_rows, dout, round_bf16=True):
    """(dy_rows [R,H], d_topk_w [T,K]) of the combine; y_rows [R,H] as float64 values."""
    topk_w, slot_to_row, dout = _f32(topk_w), _i32(slot_to_row), _u16(dout)
    T, K = topk_w.shape
    H = dout.shape[1]
    y_rows = _f64(y_rows)
    dy = np.zeros_like(y_rows)
    dw = np.zeros((T, K))
    lib().oracle_combine_bwd(T, K, H, int(round_bf16), _ptr(topk_w), _ptr(slot_to_row),
                             _ptr(y_rows), _ptr(dout), _ptr(dy), _ptr(dw))
    return dy, dw


def down_bwd_rows(dy, wd, round_bf16=True):
    dy, wd = _f64(dy), _u16(wd)
    n, H = dy.shape
    I = wd.shape[1]
    dh = np.zeros((n, I))
    if n:
        lib().oracle_down_bwd_rows(n, H, I, int(round_bf16), _ptr(dy), _ptr(wd), _ptr(dh))
    return dh


def swiglu_bwd_rows(x_rows, wg, wu, dh, limit, round_bf16=True):
    x_rows, wg, wu, dh = _u16(x_rows), _u16(wg), _u16(wu), _f64(dh)
    n, H = x_rows.shape
    I = wg.shape[0]
    dg, du = np.zeros((n, I)), np.zeros((n, I))
    if n:
        lib().oracle_swiglu_bwd_rows(n, H, I, float(limit), int(round_bf16), _ptr(x_rows), _ptr(wg),
                                     _ptr(wu), _ptr(dh), _ptr(dg), _ptr(du))
    return dg, du


def gateup_dgrad_rows(dg, du, wg, wu, round_bf16=True):
    dg, du, wg, wu = _f64(dg), _f64(du), _u16(wg), _u16(wu)
    n, I = dg.shape
    H = wg.shape[1]
    dx = np.zeros((n, H))
    if n:
        lib().oracle_gateup_dgrad_rows(n, H, I, int(round_bf16), _ptr(dg), _ptr(du), _ptr(wg),
                                       _ptr(wu), _ptr(dx))
    return dx


def wgrad(A, B):
    """A^T B over rows, float64 (weight gradients)."""
    A, B = _f64(A), _f64(B)
    n, M = A.shape
    N = B.shape[1]
    out = np.zeros((M, N))
    lib().oracle_wgrad(n, M, N, _ptr(A), _ptr(B), _ptr(out))
    return out


def router_bwd(logits, topk_idx, d_topk_w, scale=1.0, norm_topk=True, d_aux=0.0):
    logits, topk_idx, d_topk_w = _f32(logits), _i32(topk_idx), _f64(d_topk_w)
    T, E = logits.shape
    K = topk_idx.shape[1]
    dl = np.zeros((T, E))
    lib().oracle_router_bwd(T, E, K, int(bool(norm_topk)), float(scale), _ptr(logits),
                            _ptr(topk_idx), _ptr(d_topk_w), float(d_aux), _ptr(dl))
    return dl


def layer_backward(x, wr, wg, wu, wd, fwd, dout, *, sg=None, su=None, sd=None, scale=1.0,
                   limit=10.0, norm_topk=True, d_aux=0.0, round_bf16=True):
    """Backward of layer_forward. ``fwd`` holds the forward's logits, topk_idx, topk_w, counts,
    offsets, row_to_slot, slot_to_row (a layer_forward result). Returns a dict of float64
    arrays: d_topk_w, d_logits, dx, d_wr, d_wg, d_wu, d_wd, (d_sg, d_su, d_sd), dh_rows,
    dg_rows, du_rows, dx_rows, dx_router."""
    x, wr, wg, wu, wd, dout = _u16(x), _u16(wr), _u16(wg), _u16(wu), _u16(wd), _u16(dout)
    T, H = x.shape
    E, I = wg.shape[0], wg.shape[1]
    K = fwd["topk_idx"].shape[1]
    off = _i32(fwd["offsets"])
    R = int(off[-1])
    r = dict(d_topk_w=np.zeros((T, K)), d_logits=np.zeros((T, E)), dx=np.zeros((T, H)),
             d_wr=np.zeros((E, H)), d_wg=np.zeros((E, I, H)), d_wu=np.zeros((E, I, H)),
             d_wd=np.zeros((E, H, I)), dh_rows=np.zeros((R, I)), dg_rows=np.zeros((R, I)),
             du_rows=np.zeros((R, I)), dx_rows=np.zeros((R, H)), dx_router=np.zeros((T, H)))
    if sg is not None:
        sg, su, sd = _u16(sg), _u16(su), _u16(sd)
        r.update(d_sg=np.zeros((I, H)), d_su=np.zeros((I, H)), d_sd=np.zeros((H, I)))
    keep = [_f32(fwd["logits"]), _i32(fwd["topk_idx"]), _f32(fwd["topk_w"]), _i32(fwd["counts"]),
            off, _i32(fwd["row_to_slot"]), _i32(fwd["slot_to_row"])]
    lib().oracle_layer_backward(
        T, H, E, K, I, int(bool(norm_topk)), float(scale), float(limit), int(round_bf16),
        _ptr(x), _ptr(wr), _ptr(wg), _ptr(wu), _ptr(wd), _ptr(sg), _ptr(su), _ptr(sd),
        *[_ptr(a) for a in keep], _ptr(dout), float(d_aux),
        _ptr(r["d_topk_w"]), _ptr(r["d_logits"]), _ptr(r["dx"]), _ptr(r["d_wr"]), _ptr(r["d_wg"]),
        _ptr(r["d_wu"]), _ptr(r["d_wd"]), _ptr(r.get("d_sg")), _ptr(r.get("d_su")),
        _ptr(r.get("d_sd")), _ptr(r["dh_rows"]), _ptr(r["dg_rows"]), _ptr(r["du_rows"]),
        _ptr(r["dx_rows"]), _ptr(r["dx_router"]))
    return r


def bf16_to_f64(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (numpy bit shift; used by tests for comparisons)."""
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
