"""Seeded synthetic workloads for the MoE layer forward.

Input generation only: this module holds none of the layer's arithmetic. It is the one piece
of code that both the HIP path (tests, benchmark) and the CPU oracle's callers share, so that
both sides see the same bits.

Shapes and distributions follow the Hy4 preview configuration (hidden 6144, 256 routed experts,
top-8, one shared expert, expert intermediate 2048, routed_scaling_factor 2.827,
swiglu_limit 10, initializer_range 0.006, bf16) described in the Hy4 config.json walkthrough
(lshu.cn, section "MoE routed experts: 256 choose 8" and "length, vocabulary and training
details"; its architecture overview gives the first layer's dense FFN intermediate size 18432),
and the Hy3 router sketch's top-2 / 32-expert / hidden-7168 / capacity_factor 1.25
variant (Hy3 deep-dive, `SparseMoERouter`).

Recipe: every tensor is drawn as float32 N(0, std^2) from its own torch generator seeded with
``1000 * workload.seed + tensor_id`` and rounded to bf16 (round-to-nearest-even). Routed expert
weights are drawn one expert at a time. The optional router bias (Zipf-like popularity) is
``b_e = zipf * ln(1/(e+1))``, computed in float64 on the host and stored as float32.

FP8 workloads (``fp8=True``) store every expert weight matrix, routed and shared, as OCP FP8 E4M3
codes with one fp32 scale per row: the row is drawn as above in float32, its scale is
max|w| / 448 (448 being the largest finite E4M3 value), and the codes are torch's round-to-nearest
conversion of w / scale. This is checkpoint preparation, not part of the layer: the layer only
ever reads the codes and scales.

MX workloads (``mx=True``, with ``fp8`` and ``act_fp8``) store every expert weight matrix as E4M3
codes with one power-of-two scale per 32 consecutive elements of a row (E8M0 bytes, bias 127,
``<name>_mx`` of shape [..., rows, cols / 32]): per block, the smallest power of two 2^e with
max|w| / 2^e <= 448 (so no code saturates), and codes torch's round-to-nearest conversion of
w / 2^e. Checkpoint preparation again; the activations' block quantisation is the layer's own.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass

import torch

# tensor ids used in the per-tensor seeds
_TID = dict(x=1, w_router=2, w_gate=3, w_up=4, w_down=5, s_gate=6, s_up=7, s_down=8)


@dataclass(frozen=True)
class Workload:
    name: str
    T: int            # tokens (batch * sequence)
    H: int            # hidden size
    E: int            # routed experts
    K: int            # experts per token
    I: int            # expert intermediate size (also the shared expert's)
    n_shared: int = 1
    scale: float = 1.0          # routed_scaling_factor
    limit: float = 10.0         # swiglu_limit; <= 0 disables the clamp
    capacity: int = 0           # per-expert capacity; 0 = unlimited
    norm_topk: bool = True      # norm_topk_prob
    x_std: float = 1.0
    w_std: float = 0.02
    router_std: float = 0.02
    zipf: float = 0.0           # router bias b_e = zipf * ln(1/(e+1)); 0 = no bias
    seed: int = 0
    fp8: bool = False           # expert weights as FP8 E4M3 codes + per-row fp32 scales
    act_fp8: bool = False       # with fp8: expert activations quantised per row to E4M3 (W8A8)
    mx: bool = False            # with fp8 and act_fp8: MX block scales (32 elements) instead

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def capacity_for(T: int, K: int, E: int, num: int = 5, den: int = 4) -> int:
    """ceil(num/den * T*K/E) in integer arithmetic (capacity_factor 1.25 by default)."""
    return -(-(num * T * K) // (den * E))


WORKLOADS = {
    "tiny_t128_h512_e32_k2": Workload(
        "tiny_t128_h512_e32_k2", T=128, H=512, E=32, K=2, I=256, scale=1.0, limit=10.0,
        w_std=0.02, router_std=0.02, seed=0),
    "hy4_decode_t64": Workload(
        "hy4_decode_t64", T=64, H=6144, E=256, K=8, I=2048, scale=2.827, limit=10.0,
        w_std=0.006, router_std=0.006, seed=1),
    "hy4_prefill_t8192": Workload(
        "hy4_prefill_t8192", T=8192, H=6144, E=256, K=8, I=2048, scale=2.827, limit=10.0,
        w_std=0.006, router_std=0.006, seed=2),
    "capacity_t4096_h7168_e32_k2": Workload(
        "capacity_t4096_h7168_e32_k2", T=4096, H=7168, E=32, K=2, I=4096, scale=1.0,
        limit=0.0, capacity=capacity_for(4096, 2, 32), w_std=0.006, router_std=0.006, seed=3),
    "hy4_skew_t65536": Workload(
        "hy4_skew_t65536", T=65536, H=6144, E=256, K=8, I=2048, scale=2.827, limit=10.0,
        w_std=0.006, router_std=0.006, zipf=1.2, seed=4),
    # the dense FFN of the stack's first layer (intermediate 18432) as the E = 1, k = 1 layer with
    # no shared expert, over a prefill batch
    "dense_ffn_t8192_h6144_i18432": Workload(
        "dense_ffn_t8192_h6144_i18432", T=8192, H=6144, E=1, K=1, I=18432, n_shared=0, scale=1.0,
        limit=10.0, w_std=0.006, router_std=0.006, seed=6),
    # the decode and prefill batches with FP8 expert weights (the pages' deployment checkpoint is
    # FP8)
    "hy4_decode_t64_fp8": Workload(
        "hy4_decode_t64_fp8", T=64, H=6144, E=256, K=8, I=2048, scale=2.827, limit=10.0,
        w_std=0.006, router_std=0.006, seed=5, fp8=True),
    "hy4_prefill_t8192_fp8": Workload(
        "hy4_prefill_t8192_fp8", T=8192, H=6144, E=256, K=8, I=2048, scale=2.827, limit=10.0,
        w_std=0.006, router_std=0.006, seed=7, fp8=True),
    # the same FP8 deployment with the FP8 matrix cores doing the products: activations quantised
    # per row to E4M3 as well (W8A8)
    "hy4_decode_t64_w8a8": Workload(
        "hy4_decode_t64_w8a8", T=64, H=6144, E=256, K=8, I=2048, scale=2.827, limit=10.0,
        w_std=0.006, router_std=0.006, seed=8, fp8=True, act_fp8=True),
    "hy4_prefill_t8192_w8a8": Workload(
        "hy4_prefill_t8192_w8a8", T=8192, H=6144, E=256, K=8, I=2048, scale=2.827, limit=10.0,
        w_std=0.006, router_std=0.006, seed=9, fp8=True, act_fp8=True),
    "hy4_skew_t65536_w8a8": Workload(
        "hy4_skew_t65536_w8a8", T=65536, H=6144, E=256, K=8, I=2048, scale=2.827, limit=10.0,
        w_std=0.006, router_std=0.006, zipf=1.2, seed=10, fp8=True, act_fp8=True),
    # the FP8 deployment with MX block scales (one power of two per 32 elements, OCP MXFP8) on
    # weights and activations
    "hy4_decode_t64_mx": Workload(
        "hy4_decode_t64_mx", T=64, H=6144, E=256, K=8, I=2048, scale=2.827, limit=10.0,
        w_std=0.006, router_std=0.006, seed=11, fp8=True, act_fp8=True, mx=True),
    "hy4_prefill_t8192_mx": Workload(
        "hy4_prefill_t8192_mx", T=8192, H=6144, E=256, K=8, I=2048, scale=2.827, limit=10.0,
        w_std=0.006, router_std=0.006, seed=12, fp8=True, act_fp8=True, mx=True),
    "hy4_skew_t65536_mx": Workload(
        "hy4_skew_t65536_mx", T=65536, H=6144, E=256, K=8, I=2048, scale=2.827, limit=10.0,
        w_std=0.006, router_std=0.006, zipf=1.2, seed=13, fp8=True, act_fp8=True, mx=True),
}
WORKLOAD_ORDER = list(WORKLOADS)


def router_bias(wl: Workload):
    if wl.zipf == 0.0:
        return None
    vals = [wl.zipf * math.log(1.0 / (e + 1)) for e in range(wl.E)]
    return torch.tensor(vals, dtype=torch.float64).to(torch.float32)


def _gen(wl: Workload, name: str, device):
    g = torch.Generator(device=device)
    g.manual_seed(1000 * wl.seed + _TID[name])
    return g


def _randn_bf16(shape, std, gen, device):
    return (torch.randn(*shape, generator=gen, device=device, dtype=torch.float32) * std).to(
        torch.bfloat16)


def _randn_fp8(shape, std, gen, device):
    """(E4M3 codes as uint8, fp32 per-row scale) of a float32 N(0, std^2) matrix."""
    w = torch.randn(*shape, generator=gen, device=device, dtype=torch.float32) * std
    scale = w.abs().amax(dim=-1) / 448.0
    scale = torch.where(scale > 0, scale, torch.ones_like(scale))
    q = (w / scale.unsqueeze(-1)).to(torch.float8_e4m3fn).view(torch.uint8)
    return q, scale


def _randn_mx(shape, std, gen, device):
    """(E4M3 codes as uint8, E8M0 scale bytes [rows, cols / 32]) of a float32 N(0, std^2) matrix."""
    w = torch.randn(*shape, generator=gen, device=device, dtype=torch.float32) * std
    blk = w.view(*shape[:-1], shape[-1] // 32, 32)
    amax = blk.abs().amax(dim=-1)
    e = torch.ceil(torch.log2(torch.clamp(amax, min=2.0 ** -100) / 448.0))
    e = torch.clamp(e, -127, 127)
    q = (blk / torch.exp2(e).unsqueeze(-1)).to(torch.float8_e4m3fn).view(torch.uint8).view(*shape)
    return q, (e + 127).to(torch.uint8)


def generate(wl: Workload, device="cpu", shared: bool = True):
    """Return a dict of torch tensors on ``device``:
    x [T,H], w_router [E,H], router_bias [E] fp32 or None, w_gate/w_up [E,I,H], w_down [E,H,I],
    s_gate/s_up [I,H], s_down [H,I] (None without a shared expert). bf16 unless noted. For FP8
    workloads the expert weights are uint8 E4M3 codes and each has a ``<name>_scale`` fp32 tensor
    of its leading dimensions ([E,I], [E,H], [I], [H])."""
    dev = torch.device(device)
    out = {}
    out["x"] = _randn_bf16((wl.T, wl.H), wl.x_std, _gen(wl, "x", dev), dev)
    out["w_router"] = _randn_bf16((wl.E, wl.H), wl.router_std, _gen(wl, "w_router", dev), dev)
    b = router_bias(wl)
    out["router_bias"] = None if b is None else b.to(dev)
    for name, shp in (("w_gate", (wl.I, wl.H)), ("w_up", (wl.I, wl.H)), ("w_down", (wl.H, wl.I))):
        g = _gen(wl, name, dev)
        if wl.mx:
            w = torch.empty((wl.E,) + shp, dtype=torch.uint8, device=dev)
            sc = torch.empty((wl.E, shp[0], shp[1] // 32), dtype=torch.uint8, device=dev)
            for e in range(wl.E):
                w[e], sc[e] = _randn_mx(shp, wl.w_std, g, dev)
            out[name + "_mx"] = sc
        elif wl.fp8:
            w = torch.empty((wl.E,) + shp, dtype=torch.uint8, device=dev)
            sc = torch.empty((wl.E, shp[0]), dtype=torch.float32, device=dev)
            for e in range(wl.E):
                w[e], sc[e] = _randn_fp8(shp, wl.w_std, g, dev)
            out[name + "_scale"] = sc
        else:
            w = torch.empty((wl.E,) + shp, dtype=torch.bfloat16, device=dev)
            for e in range(wl.E):
                w[e] = _randn_bf16(shp, wl.w_std, g, dev)
        out[name] = w
    out["act_fp8"] = wl.act_fp8
    out["mx"] = wl.mx
    for name, shp in (("s_gate", (wl.I, wl.H)), ("s_up", (wl.I, wl.H)), ("s_down", (wl.H, wl.I))):
        if shared and wl.n_shared:
            g = _gen(wl, name, dev)
            if wl.mx:
                out[name], out[name + "_mx"] = _randn_mx(shp, wl.w_std, g, dev)
            elif wl.fp8:
                out[name], out[name + "_scale"] = _randn_fp8(shp, wl.w_std, g, dev)
            else:
                out[name] = _randn_bf16(shp, wl.w_std, g, dev)
        else:
            out[name] = None
            if wl.mx:
                out[name + "_mx"] = None
            elif wl.fp8:
                out[name + "_scale"] = None
    return out


def as_u16(t: torch.Tensor):
    """bf16 torch tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view("uint16")


def from_u16(a, device="cpu") -> torch.Tensor:
    """numpy uint16 bit patterns -> bf16 torch tensor."""
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
