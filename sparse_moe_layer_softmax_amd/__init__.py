"""MI355X (gfx950) sparse Mixture-of-Experts FFN layer forward.

Thin ctypes binding of ``libmoe.so`` (C ABI in ``include/moe.h``). Functions carry the same
names as the C entry points and only marshal arguments: torch tensors supply device memory and
the current HIP stream; every step of the layer runs in the library's kernels. There is no
fallback: if ``libmoe.so`` is missing or cannot be loaded, the first call raises ImportError.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4
MOE_ERR_SCRATCH = -5

EXPORTED = (
    "moe_strerror", "moe_route_workspace_size", "moe_route", "moe_permute_workspace_size",
    "moe_permute", "moe_expert_ffn_workspace_size", "moe_expert_ffn", "moe_combine",
    "moe_layer_workspace_size", "moe_layer_workspace_layout", "moe_layer_forward",
    "moe_layer_forward_profiled", "moe_layer_forward_train", "moe_expert_ffn_fp8", "moe_layer_forward_fp8",
    "moe_route_train_workspace_size", "moe_route_train", "moe_layer_backward_workspace_size",
    "moe_layer_backward_workspace_layout", "moe_layer_backward", "moe_quantize_rows_e4m3",
    "moe_layer_w8a8_workspace_size", "moe_layer_w8a8_workspace_layout", "moe_layer_forward_w8a8",
    "moe_layer_noalloc_scratch_bytes", "moe_layer_forward_noalloc", "moe_quantize_rows_mx",
    "moe_layer_mx_workspace_size", "moe_layer_mx_workspace_layout", "moe_layer_forward_mx",
)
MOE_LAYER_PHASE_EVENTS = 7


class MoeError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__("%s failed: %s (%d)" % (where, strerror(code), code))
        self.code = code


class moe_shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("K", ctypes.c_int32), ("I", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("norm_topk_prob", ctypes.c_int32), ("routed_scaling", ctypes.c_float),
                ("swiglu_limit", ctypes.c_float), ("capacity", ctypes.c_int32)]


class moe_layer_ws_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("logits", "topk_w", "topk_idx", "counts", "offsets",
                                               "row_to_slot", "slot_to_row", "h", "y", "total")]


class moe_layer_a8_ws_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("xq", "x_scale", "hq", "h_scale", "total")]


class moe_layer_mx_ws_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("xq", "x_scale", "hq", "h_scale", "scale_rows", "total")]


class moe_bwd_ws_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("dy", "dh", "dgu", "dx_rows", "dx_router",
                                               "d_topk_w", "d_logits", "total")]


@dataclass(frozen=True)
class Shape:
    T: int
    H: int
    E: int
    K: int
    I: int
    n_shared: int = 1
    norm_topk_prob: bool = True
    routed_scaling: float = 1.0
    swiglu_limit: float = 10.0
    capacity: int = 0

    @staticmethod
    def of(wl) -> "Shape":
        """From a workloads.Workload."""
        return Shape(wl.T, wl.H, wl.E, wl.K, wl.I, wl.n_shared, wl.norm_topk, wl.scale, wl.limit,
                     wl.capacity)

    def c(self) -> moe_shape:
        return moe_shape(self.T, self.H, self.E, self.K, self.I, self.n_shared,
                         int(bool(self.norm_topk_prob)), self.routed_scaling, self.swiglu_limit,
                         self.capacity)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libmoe.so is not built (run `python -m sparse_moe_layer_softmax_amd.build`)")
    L = ctypes.CDLL(LIB_PATH)
    P, S, I32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    sp = ctypes.POINTER(moe_shape)
    sig = {
        "moe_strerror": ([ctypes.c_int], ctypes.c_char_p),
        "moe_route_workspace_size": ([sp], S),
        "moe_route": ([sp, P, P, P, P, P, P, P, S, P], ctypes.c_int),
        "moe_permute_workspace_size": ([sp], S),
        "moe_permute": ([sp, P, P, P, P, P, P, S, P], ctypes.c_int),
        "moe_expert_ffn_workspace_size": ([sp, I32, I32], S),
        "moe_expert_ffn": ([sp, I32, I32, P, P, P, P, P, P, P, P, P, S, P], ctypes.c_int),
        "moe_combine": ([sp, P, P, P, P, P, P], ctypes.c_int),
        "moe_layer_workspace_size": ([sp], S),
        "moe_layer_workspace_layout": ([sp, ctypes.POINTER(moe_layer_ws_layout)], ctypes.c_int),
        "moe_layer_forward": ([sp, P, P, P, P, P, P, P, P, P, P, P, S, P], ctypes.c_int),
        "moe_layer_forward_profiled": ([sp, P, P, P, P, P, P, P, P, P, P, P, S, P, P], ctypes.c_int),
        "moe_layer_forward_train": ([sp] + [P] * 12 + [S, P], ctypes.c_int),
        "moe_expert_ffn_fp8": ([sp, I32, I32] + [P] * 12 + [S, P], ctypes.c_int),
        "moe_route_train_workspace_size": ([sp], S),
        "moe_route_train": ([sp] + [P] * 12 + [ctypes.c_float, P, S, P], ctypes.c_int),
        "moe_layer_backward_workspace_size": ([sp], S),
        "moe_layer_backward_workspace_layout": ([sp, ctypes.POINTER(moe_bwd_ws_layout)], ctypes.c_int),
        "moe_layer_backward": ([sp] + [P] * 9 + [S, P, P, ctypes.c_float] + [P] * 10 + [P, S, P],
                               ctypes.c_int),
        "moe_layer_forward_fp8": ([sp] + [P] * 17 + [S, P, P], ctypes.c_int),
        "moe_quantize_rows_e4m3": ([P, I32, I32, P, P, P], ctypes.c_int),
        "moe_layer_w8a8_workspace_size": ([sp], S),
        "moe_layer_w8a8_workspace_layout": ([sp, ctypes.POINTER(moe_layer_a8_ws_layout)], ctypes.c_int),
        "moe_layer_forward_w8a8": ([sp] + [P] * 17 + [S, P, P], ctypes.c_int),
        "moe_layer_noalloc_scratch_bytes": ([], S),
        "moe_layer_forward_noalloc": ([sp] + [P] * 11, ctypes.c_int),
        "moe_quantize_rows_mx": ([P, I32, I32, P, P, P], ctypes.c_int),
        "moe_layer_mx_workspace_size": ([sp], S),
        "moe_layer_mx_workspace_layout": ([sp, ctypes.POINTER(moe_layer_mx_ws_layout)], ctypes.c_int),
        "moe_layer_forward_mx": ([sp] + [P] * 17 + [S, P, P], ctypes.c_int),
    }
    for name, (argtypes, restype) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = argtypes
        fn.restype = restype
    return L


_lib = None


def library():
    """The loaded libmoe.so (loaded on first use; raises ImportError if it is not built)."""
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


def strerror(code: int) -> str:
    return library().moe_strerror(code).decode()


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, where: str):
    if rc != MOE_OK:
        raise MoeError(rc, where)


def _ws(nbytes: int, device):
    # 256-byte alignment: torch's caching allocator returns 512-byte aligned blocks
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------------- workspace sizes
def moe_route_workspace_size(shape: Shape) -> int:
    return library().moe_route_workspace_size(ctypes.byref(shape.c()))


def moe_permute_workspace_size(shape: Shape) -> int:
    return library().moe_permute_workspace_size(ctypes.byref(shape.c()))


def moe_expert_ffn_workspace_size(shape: Shape, n_groups: int, rows_max: int) -> int:
    return library().moe_expert_ffn_workspace_size(ctypes.byref(shape.c()), n_groups, rows_max)


def moe_layer_workspace_size(shape: Shape) -> int:
    return library().moe_layer_workspace_size(ctypes.byref(shape.c()))


def moe_layer_workspace_layout(shape: Shape) -> dict:
    lay = moe_layer_ws_layout()
    _check(library().moe_layer_workspace_layout(ctypes.byref(shape.c()), ctypes.byref(lay)),
           "moe_layer_workspace_layout")
    return {n: getattr(lay, n) for n, _ in moe_layer_ws_layout._fields_}


# ----------------------------------------------------------------------------- entry points
def moe_route(shape: Shape, x, w_router, bias, logits, topk_w, topk_idx, ws, stream=None):
    _check(library().moe_route(ctypes.byref(shape.c()), _p(x), _p(w_router), _p(bias), _p(logits),
                         _p(topk_w), _p(topk_idx), _p(ws), ws.numel() if ws is not None else 0,
                         _stream(stream)), "moe_route")


def moe_route_train_workspace_size(shape: Shape) -> int:
    return library().moe_route_train_workspace_size(ctypes.byref(shape.c()))


def moe_route_train(shape: Shape, x, w_router, bias, noise, logits, topk_w, topk_idx, prob_mean,
                    load_frac, aux_loss, ema_counts, ema_tokens, ws, ema_decay=0.9, stream=None):
    """moe_route in training mode (score noise) plus P, f, the load-balancing loss and the EMAs."""
    _check(library().moe_route_train(
        ctypes.byref(shape.c()), _p(x), _p(w_router), _p(bias), _p(noise), _p(logits), _p(topk_w),
        _p(topk_idx), _p(prob_mean), _p(load_frac), _p(aux_loss), _p(ema_counts), _p(ema_tokens),
        float(ema_decay), _p(ws), ws.numel() if ws is not None else 0, _stream(stream)),
        "moe_route_train")


def moe_layer_backward_workspace_size(shape: Shape) -> int:
    return library().moe_layer_backward_workspace_size(ctypes.byref(shape.c()))


def moe_layer_backward_workspace_layout(shape: Shape) -> dict:
    lay = moe_bwd_ws_layout()
    _check(library().moe_layer_backward_workspace_layout(ctypes.byref(shape.c()), ctypes.byref(lay)),
           "moe_layer_backward_workspace_layout")
    return {n: getattr(lay, n) for n, _ in moe_bwd_ws_layout._fields_}


def moe_layer_backward(shape: Shape, x, w_router, w_gate, w_up, w_down, s_gate, s_up, s_down,
                       fwd_ws, d_out, d_aux, d_x, d_w_router, d_w_gate, d_w_up, d_w_down,
                       d_s_gate, d_s_up, d_s_down, d_topk_w, d_logits, ws, stream=None, gu=None):
    """Backward of moe_layer_forward (or moe_layer_forward_train, whose stored gate/up sums gu
    it then reads) from its workspace fwd_ws (see include/moe.h)."""
    _check(library().moe_layer_backward(
        ctypes.byref(shape.c()), _p(x), _p(w_router), _p(w_gate), _p(w_up), _p(w_down),
        _p(s_gate), _p(s_up), _p(s_down), _p(fwd_ws), fwd_ws.numel(), _p(gu), _p(d_out),
        float(d_aux),
        _p(d_x), _p(d_w_router), _p(d_w_gate), _p(d_w_up), _p(d_w_down), _p(d_s_gate),
        _p(d_s_up), _p(d_s_down), _p(d_topk_w), _p(d_logits), _p(ws),
        ws.numel() if ws is not None else 0, _stream(stream)), "moe_layer_backward")


def moe_permute(shape: Shape, topk_idx, counts, offsets, row_to_slot, slot_to_row, ws,
                stream=None):
    _check(library().moe_permute(ctypes.byref(shape.c()), _p(topk_idx), _p(counts), _p(offsets),
                           _p(row_to_slot), _p(slot_to_row), _p(ws),
                           ws.numel() if ws is not None else 0, _stream(stream)), "moe_permute")


def moe_expert_ffn(shape: Shape, n_groups: int, rows_max: int, x, row_to_slot, group_offsets,
                   w_gate, w_up, w_down, h, y, ws, stream=None):
    _check(library().moe_expert_ffn(ctypes.byref(shape.c()), n_groups, rows_max, _p(x), _p(row_to_slot),
                              _p(group_offsets), _p(w_gate), _p(w_up), _p(w_down), _p(h), _p(y),
                              _p(ws), ws.numel() if ws is not None else 0, _stream(stream)),
           "moe_expert_ffn")


def moe_combine(shape: Shape, y_routed, topk_w, slot_to_row, y_shared, out, stream=None):
    _check(library().moe_combine(ctypes.byref(shape.c()), _p(y_routed), _p(topk_w), _p(slot_to_row),
                           _p(y_shared), _p(out), _stream(stream)), "moe_combine")


def moe_layer_noalloc_scratch_bytes() -> int:
    return library().moe_layer_noalloc_scratch_bytes()


def moe_layer_forward_noalloc(shape: Shape, x, w_router, bias, w_gate, w_up, w_down, s_gate, s_up,
                              s_down, out, stream=None):
    """moe_layer_forward on the library's static per-device scratch (no workspace argument)."""
    _check(library().moe_layer_forward_noalloc(
        ctypes.byref(shape.c()), _p(x), _p(w_router), _p(bias), _p(w_gate), _p(w_up), _p(w_down),
        _p(s_gate), _p(s_up), _p(s_down), _p(out), _stream(stream)), "moe_layer_forward_noalloc")


def moe_layer_forward_train(shape: Shape, x, w_router, bias, w_gate, w_up, w_down, s_gate, s_up,
                            s_down, out, gu, ws, stream=None):
    """moe_layer_forward that also stores the fp32 gate/up sums gu [T + T*K, 2I] for the backward."""
    _check(library().moe_layer_forward_train(ctypes.byref(shape.c()), _p(x), _p(w_router), _p(bias),
                                       _p(w_gate), _p(w_up), _p(w_down), _p(s_gate), _p(s_up),
                                       _p(s_down), _p(out), _p(gu), _p(ws),
                                       ws.numel() if ws is not None else 0, _stream(stream)),
           "moe_layer_forward_train")


def moe_layer_forward(shape: Shape, x, w_router, bias, w_gate, w_up, w_down, s_gate, s_up,
                      s_down, out, ws, stream=None):
    _check(library().moe_layer_forward(ctypes.byref(shape.c()), _p(x), _p(w_router), _p(bias),
                                 _p(w_gate), _p(w_up), _p(w_down), _p(s_gate), _p(s_up),
                                 _p(s_down), _p(out), _p(ws), ws.numel() if ws is not None else 0,
                                 _stream(stream)), "moe_layer_forward")


def moe_layer_forward_profiled(shape: Shape, x, w_router, bias, w_gate, w_up, w_down, s_gate,
                               s_up, s_down, out, ws, phase_events, stream=None):
    """phase_events: ctypes array of MOE_LAYER_PHASE_EVENTS hipEvent_t handles (entries may be 0)."""
    _check(library().moe_layer_forward_profiled(
        ctypes.byref(shape.c()), _p(x), _p(w_router), _p(bias), _p(w_gate), _p(w_up), _p(w_down),
        _p(s_gate), _p(s_up), _p(s_down), _p(out), _p(ws), ws.numel() if ws is not None else 0,
        _stream(stream), phase_events), "moe_layer_forward_profiled")


def moe_expert_ffn_fp8(shape: Shape, n_groups: int, rows_max: int, x, row_to_slot, group_offsets,
                       w_gate, w_gate_scale, w_up, w_up_scale, w_down, w_down_scale, h, y, ws,
                       stream=None):
    """moe_expert_ffn with FP8 E4M3 weight codes (uint8) and per-row fp32 scales."""
    _check(library().moe_expert_ffn_fp8(
        ctypes.byref(shape.c()), n_groups, rows_max, _p(x), _p(row_to_slot), _p(group_offsets),
        _p(w_gate), _p(w_gate_scale), _p(w_up), _p(w_up_scale), _p(w_down), _p(w_down_scale),
        _p(h), _p(y), _p(ws), ws.numel() if ws is not None else 0, _stream(stream)),
        "moe_expert_ffn_fp8")


def moe_layer_forward_fp8(shape: Shape, x, w_router, bias, w_gate, w_gate_scale, w_up, w_up_scale,
                          w_down, w_down_scale, s_gate, s_gate_scale, s_up, s_up_scale, s_down,
                          s_down_scale, out, ws, phase_events=None, stream=None):
    """moe_layer_forward with FP8 expert weights; phase_events as for moe_layer_forward_profiled."""
    _check(library().moe_layer_forward_fp8(
        ctypes.byref(shape.c()), _p(x), _p(w_router), _p(bias), _p(w_gate), _p(w_gate_scale),
        _p(w_up), _p(w_up_scale), _p(w_down), _p(w_down_scale), _p(s_gate), _p(s_gate_scale),
        _p(s_up), _p(s_up_scale), _p(s_down), _p(s_down_scale), _p(out), _p(ws),
        ws.numel() if ws is not None else 0, _stream(stream), phase_events),
        "moe_layer_forward_fp8")


def moe_quantize_rows_e4m3(x, codes, scales, stream=None):
    """Per-row dynamic E4M3 quantisation: x [rows, cols] bf16 -> codes uint8, scales fp32 [rows]."""
    rows, cols = x.shape
    _check(library().moe_quantize_rows_e4m3(_p(x), rows, cols, _p(codes), _p(scales),
                                            _stream(stream)), "moe_quantize_rows_e4m3")


def moe_layer_w8a8_workspace_size(shape: Shape) -> int:
    return library().moe_layer_w8a8_workspace_size(ctypes.byref(shape.c()))


def moe_layer_w8a8_workspace_layout(shape: Shape) -> dict:
    lay = moe_layer_a8_ws_layout()
    _check(library().moe_layer_w8a8_workspace_layout(ctypes.byref(shape.c()), ctypes.byref(lay)),
           "moe_layer_w8a8_workspace_layout")
    return {n: getattr(lay, n) for n, _ in moe_layer_a8_ws_layout._fields_}


def moe_layer_forward_w8a8(shape: Shape, x, w_router, bias, w_gate, w_gate_scale, w_up, w_up_scale,
                           w_down, w_down_scale, s_gate, s_gate_scale, s_up, s_up_scale, s_down,
                           s_down_scale, out, ws, phase_events=None, stream=None):
    """moe_layer_forward_fp8 with the expert activations quantised per row to E4M3 (W8A8)."""
    _check(library().moe_layer_forward_w8a8(
        ctypes.byref(shape.c()), _p(x), _p(w_router), _p(bias), _p(w_gate), _p(w_gate_scale),
        _p(w_up), _p(w_up_scale), _p(w_down), _p(w_down_scale), _p(s_gate), _p(s_gate_scale),
        _p(s_up), _p(s_up_scale), _p(s_down), _p(s_down_scale), _p(out), _p(ws),
        ws.numel() if ws is not None else 0, _stream(stream), phase_events),
        "moe_layer_forward_w8a8")


def moe_quantize_rows_mx(x, codes, scales, stream=None):
    """MX block quantisation: x [rows, cols] bf16 -> codes uint8 [rows, cols], scale bytes
    [cols/128][rows][4] (K-tile-major)."""
    rows, cols = x.shape
    _check(library().moe_quantize_rows_mx(_p(x), rows, cols, _p(codes), _p(scales), _stream(stream)),
           "moe_quantize_rows_mx")


def moe_layer_mx_workspace_size(shape: Shape) -> int:
    return library().moe_layer_mx_workspace_size(ctypes.byref(shape.c()))


def moe_layer_mx_workspace_layout(shape: Shape) -> dict:
    lay = moe_layer_mx_ws_layout()
    _check(library().moe_layer_mx_workspace_layout(ctypes.byref(shape.c()), ctypes.byref(lay)),
           "moe_layer_mx_workspace_layout")
    return {n: getattr(lay, n) for n, _ in moe_layer_mx_ws_layout._fields_}


def moe_layer_forward_mx(shape: Shape, x, w_router, bias, w_gate, w_gate_scale, w_up, w_up_scale,
                         w_down, w_down_scale, s_gate, s_gate_scale, s_up, s_up_scale, s_down,
                         s_down_scale, out, ws, phase_events=None, stream=None):
    """The layer with MX block-scaled FP8 weights and activations (scale bytes K-tile-major)."""
    _check(library().moe_layer_forward_mx(
        ctypes.byref(shape.c()), _p(x), _p(w_router), _p(bias), _p(w_gate), _p(w_gate_scale),
        _p(w_up), _p(w_up_scale), _p(w_down), _p(w_down_scale), _p(s_gate), _p(s_gate_scale),
        _p(s_up), _p(s_up_scale), _p(s_down), _p(s_down_scale), _p(out), _p(ws),
        ws.numel() if ws is not None else 0, _stream(stream), phase_events),
        "moe_layer_forward_mx")


# ----------------------------------------------------------------------------- conveniences
_WEIGHTS = ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down")


class MoELayer:
    """Holds device weights and a workspace; ``forward(x)`` runs moe_layer_forward (bf16 expert
    weights) or moe_layer_forward_fp8 (uint8 E4M3 expert weights; ``scales`` then maps each weight
    name of _WEIGHTS to its fp32 per-row scale tensor); with ``act_fp8`` (FP8 weights only)
    moe_layer_forward_w8a8, which quantises the expert activations per row as well; with
    ``mx_scales`` (E8M0 block-scale bytes [..., rows, cols / 32] per weight name) instead of
    ``scales``, moe_layer_forward_mx, which takes them K-tile-major ([..., cols / 128, rows, 4],
    a layout change made here once)."""

    def __init__(self, shape: Shape, w_router, w_gate, w_up, w_down, s_gate=None, s_up=None,
                 s_down=None, router_bias=None, scales=None, act_fp8=False, mx_scales=None):
        self.shape = shape
        self.w = (w_router, router_bias, w_gate, w_up, w_down, s_gate, s_up, s_down)
        self.fp8 = w_gate.dtype == torch.uint8
        self.mx = mx_scales is not None
        self.scales = scales or {}
        if self.mx:
            self.scales = {}
            for n, t in zip(_WEIGHTS, (w_gate, w_up, w_down, s_gate, s_up, s_down)):
                m = mx_scales.get(n)
                if t is not None and m is None:
                    raise ValueError("MX weight %s needs its block scales" % n)
                if m is not None:  # [..., rows, cols/32] -> [..., cols/128, rows, 4]
                    r, nb = m.shape[-2], m.shape[-1]
                    self.scales[n] = m.reshape(*m.shape[:-2], r, nb // 4, 4).transpose(-3, -2).contiguous()
            act_fp8 = True
        elif self.fp8:
            for n, t in zip(_WEIGHTS, (w_gate, w_up, w_down, s_gate, s_up, s_down)):
                if t is not None and self.scales.get(n) is None:
                    raise ValueError("FP8 weight %s needs a scale tensor" % n)
        if act_fp8 and not self.fp8:
            raise ValueError("FP8 activations come with FP8 expert weights")
        self.act_fp8 = act_fp8
        self.device = w_router.device
        self.layout = moe_layer_workspace_layout(shape)
        if self.mx:
            self.layout.update({k: v for k, v in moe_layer_mx_workspace_layout(shape).items()
                                if k != "total"})
            self.ws = _ws(moe_layer_mx_workspace_size(shape), self.device)
        elif act_fp8:
            self.layout.update({k: v for k, v in moe_layer_w8a8_workspace_layout(shape).items()
                                if k != "total"})
            self.ws = _ws(moe_layer_w8a8_workspace_size(shape), self.device)
        else:
            self.ws = _ws(moe_layer_workspace_size(shape), self.device)

    @classmethod
    def from_inputs(cls, shape: Shape, d: dict):
        """Build from a ``workloads.generate`` dict (bf16 or FP8 expert weights)."""
        scales = {n: d.get(n + "_scale") for n in _WEIGHTS}
        mx = {n: d.get(n + "_mx") for n in _WEIGHTS} if d.get("mx") else None
        return cls(shape, d["w_router"], d["w_gate"], d["w_up"], d["w_down"], d["s_gate"], d["s_up"],
                   d["s_down"], d["router_bias"], scales=scales, act_fp8=bool(d.get("act_fp8")),
                   mx_scales=mx)

    def forward(self, x, out=None, stream=None, phase_events=None, train=False):
        """The layer's output. train=True: moe_layer_forward_train, keeping the fp32 gate/up sums
        (self.gu) that backward() then reads instead of recomputing them."""
        if out is None:
            out = torch.empty((self.shape.T, self.shape.H), dtype=torch.bfloat16, device=self.device)
        wr, b, wg, wu, wd, sg, su, sd = self.w
        self._x = x
        self._gu = None
        if train:
            if self.fp8:
                raise ValueError("the training forward takes bf16 expert weights")
            s = self.shape
            rows = s.T * s.K + (s.T if s.n_shared else 0)
            if getattr(self, "gu", None) is None or tuple(self.gu.shape) != (rows, 2 * s.I):
                self.gu = torch.empty((rows, 2 * s.I), dtype=torch.float32, device=self.device)
            moe_layer_forward_train(s, x, wr, b, wg, wu, wd, sg, su, sd, out, self.gu, self.ws, stream)
            self._gu = self.gu
        elif self.fp8:
            sc = self.scales
            fwd = (moe_layer_forward_mx if self.mx else
                   moe_layer_forward_w8a8 if self.act_fp8 else moe_layer_forward_fp8)
            fwd(self.shape, x, wr, b, wg, sc["w_gate"], wu, sc["w_up"], wd, sc["w_down"], sg,
                sc.get("s_gate"), su, sc.get("s_up"), sd, sc.get("s_down"), out, self.ws,
                phase_events, stream)
        elif phase_events is not None:
            moe_layer_forward_profiled(self.shape, x, wr, b, wg, wu, wd, sg, su, sd, out, self.ws,
                                       phase_events, stream)
        else:
            moe_layer_forward(self.shape, x, wr, b, wg, wu, wd, sg, su, sd, out, self.ws, stream)
        return out

    def backward(self, d_out, d_aux=0.0, stream=None):
        """moe_layer_backward after forward(): returns a dict of gradients (d_x bf16; d_w_router,
        d_w_gate, d_w_up, d_w_down and the shared expert's d_s_* fp32; d_topk_w, d_logits fp32).
        The backward workspace stays in self.bws (layout in self.blayout)."""
        if self.fp8:
            raise ValueError("the backward pass takes bf16 expert weights")
        s, dev = self.shape, self.device
        wr, _, wg, wu, wd, sg, su, sd = self.w
        f32 = dict(dtype=torch.float32, device=dev)
        g = dict(d_x=torch.empty((s.T, s.H), dtype=torch.bfloat16, device=dev),
                 d_w_router=torch.empty((s.E, s.H), **f32),
                 d_w_gate=torch.empty((s.E, s.I, s.H), **f32),
                 d_w_up=torch.empty((s.E, s.I, s.H), **f32),
                 d_w_down=torch.empty((s.E, s.H, s.I), **f32),
                 d_topk_w=torch.empty((s.T, s.K), **f32),
                 d_logits=torch.empty((s.T, s.E), **f32))
        if sg is not None:
            g.update(d_s_gate=torch.empty((s.I, s.H), **f32), d_s_up=torch.empty((s.I, s.H), **f32),
                     d_s_down=torch.empty((s.H, s.I), **f32))
        if getattr(self, "bws", None) is None:
            self.bws = _ws(moe_layer_backward_workspace_size(s), dev)
            self.blayout = moe_layer_backward_workspace_layout(s)
        moe_layer_backward(s, self._x, wr, wg, wu, wd, sg, su, sd, self.ws, d_out, d_aux,
                           g["d_x"], g["d_w_router"], g["d_w_gate"], g["d_w_up"], g["d_w_down"],
                           g.get("d_s_gate"), g.get("d_s_up"), g.get("d_s_down"), g["d_topk_w"],
                           g["d_logits"], self.bws, stream, gu=getattr(self, "_gu", None))
        return g

    def bwd_intermediate(self, name: str, dtype, shape):
        """A view of a backward intermediate (dy, dh, dgu, dx_rows, dx_router)."""
        off = self.blayout[name]
        n = 1
        for d in shape:
            n *= d
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        return self.bws[off:off + nbytes].view(dtype).view(*shape)

    def intermediate(self, name: str, dtype, shape):
        """A view of an intermediate inside the workspace (valid after the stream completes)."""
        off = self.layout[name]
        n = 1
        for d in shape:
            n *= d
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        return self.ws[off:off + nbytes].view(dtype).view(*shape)
