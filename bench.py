#!/usr/bin/env python3
"""Benchmark of the sparse MoE FFN layer forward on one MI355X.

One step = one moe_layer_forward (router GEMM + softmax/top-k/renorm/scale, dispatch, routed and
shared SwiGLU expert FFNs, combine) over one batch of synthetic, seeded inputs already resident
in HBM. The headline workload (``value``) is the Hy4-shape decode batch (T=64, H=6144, 256
experts, top-8, one shared expert, intermediate 2048, bf16); the same JSON line also carries,
under ``workloads``, the other workloads of the layer's configuration list, each timed in a
region of its own: the tiny layer, the Hy4 prefill batch (T=8192), the capacity-limited top-2
layer and the long skewed prefill (T=65536), the last three bound by the matrix cores. Every
workload reports its roofline fractions and the CPU oracle timed on a bounded token sample
(all host threads; the tiny and decode layers also on one thread). ``--workload NAME`` changes
the headline (e.g. ``hy4_decode_t64_fp8``), ``--extra ''`` drops the other workloads.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--extra A,B] [--no-cpu-baseline]
  python bench.py --copy-calibration     # plain device copy, for scaling HBM counters
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "MoE-layer tokens/s at Hy4 shape; % of bf16 MFMA or HBM roofline"
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, GB/s
PEAK_MFMA_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, TFLOP/s
PEAK_MFMA_FP8_TFLOPS = 5000.0  # MI355X dense FP8 MFMA, TFLOP/s (the W8A8 expert products)
# the other workloads of the layer's configuration list, timed after the headline
EXTRA = ("tiny_t128_h512_e32_k2", "hy4_prefill_t8192", "capacity_t4096_h7168_e32_k2",
         "hy4_skew_t65536")
# workloads whose CPU baseline also runs on one thread
SINGLE_THREAD = ("tiny_t128_h512_e32_k2", "hy4_decode_t64")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="hy4_decode_t64")
    ap.add_argument("--extra", default=",".join(EXTRA),
                    help="comma-separated workloads timed after the headline ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0, help="oracle sample size (0 = auto)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--mode", choices=("forward", "train"), default="forward",
                    help="train: one step = forward + backward (bf16 weights)")
    return ap.parse_args()


def algorithmic(wl, counts):
    """Per-call algorithmic work from the run's actual routing (implementation buffers such as
    the permuted h and y rows are not counted for the layer)."""
    T, H, E, K, I, S = wl.T, wl.H, wl.E, wl.K, wl.I, wl.n_shared
    R = int(counts.sum())
    touched = int((counts > 0).sum())
    # bytes of one expert's gate+up and down weights: bf16, or one-byte E4M3 codes plus one fp32
    # scale per weight row, or (MX) plus one scale byte per 32 codes
    if wl.mx:
        w_gu, w_dn = 2 * H * I + 2 * H * I // 32, H * I + H * I // 32
    elif wl.fp8:
        w_gu, w_dn = 2 * H * I + 4 * 2 * I, H * I + 4 * H
    else:
        w_gu, w_dn = 4 * H * I, 2 * H * I
    layer_flops = 2 * T * H * E + 6 * H * I * (R + S * T)
    layer_bytes = (touched + S) * (w_gu + w_dn) + 2 * E * H + 2 * 2 * T * H + 4 * T * E + 8 * T * K
    # gate/up grouped GEMM launch: its weights, x in, h out
    gu_flops = 4 * H * I * (R + S * T)
    # activations read by the projections: bf16, or E4M3 codes plus one fp32 scale per row, or
    # (MX) plus one scale byte per 32 codes of each GEMM row
    if wl.mx:
        a_x, a_h = T * H + (R + S * T) * H // 32, (R + S * T) * (I + I // 32)
    elif wl.act_fp8:
        a_x, a_h = T * (H + 4), (R + S * T) * (I + 4)
    else:
        a_x, a_h = 2 * T * H, 2 * (R + S * T) * I
    gu_bytes = (touched + S) * w_gu + a_x + 2 * (R + S * T) * I
    # down grouped GEMM launch: its weights, h in, y out
    dn_flops = 2 * H * I * (R + S * T)
    dn_bytes = (touched + S) * w_dn + a_h + 2 * (R + S * T) * H
    return dict(R=R, touched=touched, layer_flops=layer_flops, layer_bytes=layer_bytes,
                gu_flops=gu_flops, gu_bytes=gu_bytes, dn_flops=dn_flops, dn_bytes=dn_bytes)


def roofline(flops, nbytes, seconds, peak_mfma=PEAK_MFMA_TFLOPS):
    ai = flops / nbytes
    ridge = peak_mfma * 1e12 / (PEAK_HBM_GBS * 1e9)
    if ai >= ridge:
        a = flops / seconds / 1e12
        return dict(bound="mfma", achieved=round(a, 2), peak=peak_mfma, unit="TFLOP/s",
                    frac=round(a / peak_mfma, 4))
    a = nbytes / seconds / 1e9
    return dict(bound="hbm", achieved=round(a, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                frac=round(a / PEAK_HBM_GBS, 4))


def recorded_traffic(workload, kernel):
    """HBM bytes per launch from profiles/traffic.txt (rocprofv3 PMC, copy-calibrated), or None
    when there is no record or the kernel source changed since the counters were taken."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", "traffic.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        f = line.split()
        if len(f) != 6 or line.startswith("#") or f[0] != workload or f[1] != kernel.replace(" ", ""):
            continue
        src = os.path.join(root, f[2])
        if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != f[3]:
            return None
        return int(f[4]) + int(f[5])
    return None


def cpu_baseline(wl, dev, n_tok, min_seconds=10.0, max_reps=50, threads=0):
    """The CPU oracle, timed on a bounded sample of the workload's tokens (every step of the
    layer for those tokens: router logits, routing, their routed and shared expert FFNs, combine),
    repeated until at least min_seconds have passed. Weights are copied to host memory before the
    clock starts. threads: OpenMP threads (0 = all the host offers)."""
    import numpy as np
    import torch

    import oracle
    from sparse_moe_layer_softmax_amd.workloads import as_u16

    rng = np.random.default_rng(99)
    toks = np.sort(rng.choice(wl.T, min(n_tok, wl.T), replace=False))
    x = as_u16(dev["x"][torch.from_numpy(toks).to(dev["x"].device)])
    wr = as_u16(dev["w_router"])
    bias = None if dev["router_bias"] is None else dev["router_bias"].cpu().numpy()
    # routing of the sample decides which expert weights the timed region needs
    lg = oracle.router_logits(x, wr, bias)
    idx, _ = oracle.route_from_logits(lg, wl.K, wl.scale, wl.norm_topk)
    experts = sorted(set(int(e) for e in idx.ravel()))
    def host_w(name, e=None):
        t = dev[name] if e is None else dev[name][e]
        if wl.mx:
            sc = dev[name + "_mx"] if e is None else dev[name + "_mx"][e]
            return oracle.Mx(t.cpu().numpy(), sc.cpu().numpy())
        if wl.fp8:
            sc = dev[name + "_scale"] if e is None else dev[name + "_scale"][e]
            return oracle.Fp8(t.cpu().numpy(), sc.cpu().numpy())
        return as_u16(t)

    def ffn_w8a8(x_rows, wg, wu, wd, limit):
        xq, sx = oracle.quant_rows_e4m3(x_rows)
        h = oracle.gateup_rows_w8a8(xq, sx, wg, wu, limit)
        hq, sh = oracle.quant_rows_e4m3(h)
        return h, oracle.down_rows_w8a8(hq, sh, wd)

    def ffn_mx(x_rows, wg, wu, wd, limit):
        xq, xs = oracle.mx_quant_rows(x_rows)
        h = oracle.gateup_rows_mx(xq, xs, wg, wu, limit)
        hq, hs = oracle.mx_quant_rows(h)
        return h, oracle.down_rows_mx(hq, hs, wd)

    ffn = (ffn_mx if wl.mx else ffn_w8a8 if wl.act_fp8 else
           oracle.expert_ffn_rows_fp8 if wl.fp8 else oracle.expert_ffn_rows)
    W = {e: tuple(host_w(n, e) for n in ("w_gate", "w_up", "w_down")) for e in experts}
    SW = tuple(host_w(n) for n in ("s_gate", "s_up", "s_down")) if wl.n_shared else None
    all_threads = oracle.num_threads()
    if threads:
        oracle.set_num_threads(threads)
    cores = oracle.num_threads()
    reps = 0
    t0 = time.perf_counter()
    while True:
        lg = oracle.router_logits(x, wr, bias)
        idx, w = oracle.route_from_logits(lg, wl.K, wl.scale, wl.norm_topk)
        counts, offsets, r2s, s2r = oracle.dispatch(idx, wl.E, 0)
        y = np.zeros((len(toks) * wl.K, wl.H), np.uint16)
        for e in experts:  # expert-major, as the oracle's layer does
            a, b = offsets[e], offsets[e + 1]
            _, y[a:b] = ffn(x[r2s[a:b] // wl.K], *W[e], wl.limit)
        ys = ffn(x, *SW, wl.limit)[1] if SW else None
        oracle.combine(w, s2r, y, ys)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or reps >= max_reps:
            break
    oracle.set_num_threads(all_threads)
    return {"value": round(reps * len(toks) / dt, 3), "unit": "tokens/s",
            "cores": cores, "nproc": len(os.sched_getaffinity(0)), "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": "%d of the workload's %d tokens, %d pass(es): all steps of the layer for them "
                      "(%d distinct routed experts%s), fp64 C++ oracle, %d thread(s)"
                      % (len(toks), wl.T, reps, len(experts), " + shared" if wl.n_shared else "",
                         cores)}


def copy_calibration():
    import torch
    n = 1 << 30  # 1 GiB
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "reads_bytes": n, "writes_bytes": n}))


def measure(wl, args):
    """Generate the workload's inputs in HBM, run W warm-up steps, time K plain forward steps
    between two events, then K more with an event between the phases for the per-kernel split.
    Returns the step time, the phase times, the roofline objects and the layer's fractions."""
    import ctypes

    import numpy as np
    import torch

    import sparse_moe_layer_softmax_amd as moe

    dev = generate_inputs(wl)
    shape = moe.Shape.of(wl)
    layer = moe.MoELayer.from_inputs(shape, dev)
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        layer.forward(dev["x"], out)
    torch.cuda.synchronize()

    # phase events: one set per step, created once (a first record makes the HIP event)
    nph = moe.MOE_LAYER_PHASE_EVENTS
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nph)] for _ in range(args.steps)]
    for row in evs:
        for e in row:
            e.record(stream)
    handles = [(ctypes.c_void_p * nph)(*[e.cuda_event for e in row]) for row in evs]
    torch.cuda.synchronize()

    # the timed steps are the plain forward calls; the per-phase split comes from a second pass
    # of the same steps with an event recorded between the phases (each record is a stream packet
    # of its own, which would otherwise add to the step time)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        layer.forward(dev["x"], out, stream=stream)
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    for i in range(args.steps):
        layer.forward(dev["x"], out, stream=stream, phase_events=handles[i])
    torch.cuda.synchronize()

    names = ["route", "permute", "tile_table", "gate_up_gemm", "down_gemm", "combine"]
    phase_ms = {n: float(np.mean([row[j].elapsed_time(row[j + 1]) for row in evs]))
                for j, n in enumerate(names)}
    counts = layer.intermediate("counts", torch.int32, (wl.E,)).cpu().numpy()
    alg = algorithmic(wl, counts)
    gu_s = phase_ms["gate_up_gemm"] / 1e3
    dn_s = phase_ms["down_gemm"] / 1e3
    peak_mfma = PEAK_MFMA_FP8_TFLOPS if wl.act_fp8 else PEAK_MFMA_TFLOPS
    rf = roofline(alg["gu_flops"], alg["gu_bytes"], gu_s, peak_mfma)
    # the tiled MFMA kernel runs when the groups hold at least 64 rows each on average (bf16 or
    # FP8 weights alike); below that the weights stream through the skinny kernel
    rows = wl.T * wl.K + wl.n_shared * wl.T
    groups = wl.E + wl.n_shared
    if rows >= 64 * groups:
        gu, dn = (("kEpiSwigluMx", "kEpiBf16Mx") if wl.mx else
                  ("kEpiSwiglu88", "kEpiBf16_88") if wl.act_fp8 else
                  ("kEpiSwiglu8", "kEpiBf16_8") if wl.fp8 else ("kEpiSwiglu", "kEpiBf16"))
        # second template argument: the buffer-descriptor form, which the library picks when the
        # activation operand and each weight matrix hold at most 4 GiB
        ab, wb = (1 if wl.act_fp8 else 2), (1 if wl.fp8 else 2)
        lim = 0xFFFFFFFF
        gu_buf = wl.T * wl.H * ab <= lim and wl.I * wl.H * wb <= lim
        dn_buf = (wl.T + wl.T * wl.K) * wl.I * ab <= lim and wl.H * wl.I * wb <= lim
        kname = "ffn_tiled_kernel<%s,%s>" % (gu, str(gu_buf).lower())
        dname = "ffn_tiled_kernel<%s,%s>" % (dn, str(dn_buf).lower())
    else:
        # the weight-streaming kernel; 16-row tiles (one sub-block) when the groups average at
        # most 16 rows
        maxns = 1 if rows <= 16 * groups else 4
        # <gated, FP8 weights, FP8 activations, 16-row sub-blocks per tile, MX scales>
        fl = ("true" if wl.fp8 else "false", "true" if wl.act_fp8 else "false", maxns,
              "true" if wl.mx else "false")
        kname = "ffn_skinny_kernel<true, %s, %s, %d, %s>" % fl
        dname = "ffn_skinny_kernel<false, %s, %s, %d, %s>" % fl
    rf["traffic"] = recorded_traffic(wl.name, kname)
    rf["kernel"] = kname + " (routed+shared gate/up grouped GEMM, clamped SwiGLU epilogue)"
    rf["algorithmic_bytes"] = alg["gu_bytes"]
    rf["algorithmic_flops"] = alg["gu_flops"]
    rf["avg_launch_ms"] = round(phase_ms["gate_up_gemm"], 4)
    dn = roofline(alg["dn_flops"], alg["dn_bytes"], dn_s, peak_mfma)
    dn["traffic"] = recorded_traffic(wl.name, dname)
    dn["kernel"] = dname + " (routed+shared down grouped GEMM)"
    dn["avg_launch_ms"] = round(phase_ms["down_gemm"], 4)
    layer_s = ms / 1e3
    layer_obj = {"algorithmic_bytes": alg["layer_bytes"], "algorithmic_flops": alg["layer_flops"],
                 "hbm_GBs": round(alg["layer_bytes"] / layer_s / 1e9, 1),
                 "hbm_frac": round(alg["layer_bytes"] / layer_s / 1e9 / PEAK_HBM_GBS, 4),
                 "mfma_TFLOPs": round(alg["layer_flops"] / layer_s / 1e12, 2),
                 "mfma_frac": round(alg["layer_flops"] / layer_s / 1e12 / peak_mfma, 4),
                 "routed_rows": alg["R"], "touched_experts": alg["touched"],
                 "max_rows_per_expert": int(counts.max())}
    config = {"workload": wl.name, "T": wl.T, "H": wl.H, "E": wl.E, "K": wl.K, "I": wl.I,
              "n_shared": wl.n_shared, "routed_scaling": wl.scale, "swiglu_limit": wl.limit,
              "capacity": wl.capacity, "router_bias": "zipf %.1f" % wl.zipf if wl.zipf else "none",
              "parallelism": "none (1 GPU)",
              "expert_weights": ("mxfp8: fp8_e4m3 + e8m0 scale per 32" if wl.mx else
                                 "fp8_e4m3 + fp32 row scale" if wl.fp8 else "bf16"),
              "expert_activations": ("mxfp8: fp8_e4m3 + e8m0 scale per 32 (dynamic)" if wl.mx else
                                     "fp8_e4m3 + fp32 row scale (dynamic)" if wl.act_fp8
                                     else "bf16")}
    return dict(dev=dev, ms=ms, tokens_per_s=wl.T / layer_s, roofline=rf, down_gemm=dn,
                layer=layer_obj, phases_ms={k: round(v, 4) for k, v in phase_ms.items()},
                config=config)


def cpu_baselines(wl, dev, args, min_seconds):
    """The oracle's timing on the workload's token sample: all host threads, and one thread for
    the tiny and decode layers."""
    if args.no_cpu_baseline:
        return None, None
    n_tok = args.cpu_tokens or min(wl.T, 64)
    full = cpu_baseline(wl, dev, n_tok, min_seconds=min_seconds)
    one = cpu_baseline(wl, dev, n_tok, min_seconds=min_seconds, threads=1) \
        if wl.name in SINGLE_THREAD else None
    return full, one


def release(m):
    import torch
    m.pop("dev", None)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the MoE layer here runs on a single MI355X, so "
              "--gpus %d (WORLD_SIZE=%d) is not supported" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import torch

    from sparse_moe_layer_softmax_amd.workloads import WORKLOADS

    wl = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    if args.mode == "train":
        import sparse_moe_layer_softmax_amd as moe
        dev = generate_inputs(wl)
        layer = moe.MoELayer.from_inputs(moe.Shape.of(wl), dev)
        return train_step(args, wl, dev, layer)
    m = measure(wl, args)
    res = {
        "metric": METRIC,
        "value": round(m["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3" if wl.act_fp8 else "bf16",
        "data": "synthetic",
        "config": m["config"],
        "roofline": m["roofline"],
        "layer": m["layer"],
        "down_gemm": m["down_gemm"],
        "phases_ms": m["phases_ms"],
    }
    full, one = cpu_baselines(wl, m["dev"], args, 10.0)
    res["cpu_baseline"] = full
    if one is not None:
        res["cpu_baseline_single_thread"] = one
    release(m)
    extra = [n for n in args.extra.split(",") if n and n != wl.name]
    if extra:
        res["workloads"] = {}
    for name in extra:
        w2 = WORKLOADS[name]
        m2 = measure(w2, args)
        obj = {"ms_per_step": round(m2["ms"], 4), "value": round(m2["tokens_per_s"], 1),
               "unit": "tokens/s", "steps": args.steps, "warmup": args.warmup,
               "config": m2["config"], "roofline": m2["roofline"], "down_gemm": m2["down_gemm"],
               "layer": m2["layer"], "phases_ms": m2["phases_ms"]}
        full, one = cpu_baselines(w2, m2["dev"], args, 6.0)
        obj["cpu_baseline"] = full
        if one is not None:
            obj["cpu_baseline_single_thread"] = one
        res["workloads"][name] = obj
        release(m2)
        print("[bench] %s: %.4f ms/step, %.1f tokens/s, gate/up %.1f%% of %s peak"
              % (name, m2["ms"], m2["tokens_per_s"], 100 * m2["roofline"]["frac"],
                 m2["roofline"]["bound"]), file=sys.stderr, flush=True)
    print(json.dumps(res), flush=True)


def train_flops(wl, counts):
    """Algorithmic FLOPs of one training step from the run's routing: the forward, and a backward
    of dh, dx rows, dWd, dWg/dWu (2+4+2+4 H I per row) and the router's two products (2 T E H
    each). The training forward stores the gate/up sums, so the backward recomputes nothing."""
    T, H, E, I, S = wl.T, wl.H, wl.E, wl.I, wl.n_shared
    rows = int(counts.sum()) + S * T
    fwd = 2 * T * H * E + 6 * H * I * rows
    bwd = 12 * H * I * rows + 4 * T * E * H
    return fwd, bwd


def cpu_baseline_train(wl, dev, n_tok, min_seconds=10.0, max_reps=50):
    """The oracle's forward and backward steps over a sample of the workload's tokens, taken as a
    layer of their own (their routing, their experts' rows): router, routing, dispatch, expert
    FFNs and combine, then the combine, down, SwiGLU, gate/up and weight-gradient backward of the
    touched experts and the shared expert, the router backward and dx. Repeated until at least
    min_seconds have passed."""
    import numpy as np
    import torch

    import oracle
    from sparse_moe_layer_softmax_amd.workloads import as_u16

    rng = np.random.default_rng(99)
    toks = np.sort(rng.choice(wl.T, min(n_tok, wl.T), replace=False))
    sel = torch.from_numpy(toks).to(dev["x"].device)
    x = as_u16(dev["x"][sel])
    wr = as_u16(dev["w_router"])
    bias = None if dev["router_bias"] is None else dev["router_bias"].cpu().numpy()
    g = torch.Generator()
    g.manual_seed(7)
    dout = as_u16(torch.randn(len(toks), wl.H, generator=g).to(torch.bfloat16))
    lg = oracle.router_logits(x, wr, bias)
    idx, _ = oracle.route_from_logits(lg, wl.K, wl.scale, wl.norm_topk)
    experts = sorted(set(int(e) for e in idx.ravel()))
    W = {e: tuple(as_u16(dev[n][e]) for n in ("w_gate", "w_up", "w_down")) for e in experts}
    SW = tuple(as_u16(dev[n]) for n in ("s_gate", "s_up", "s_down")) if wl.n_shared else None
    f64 = oracle.bf16_to_f64
    Ts, K, H = len(toks), wl.K, wl.H
    all_threads = oracle.num_threads()
    if threads:
        oracle.set_num_threads(threads)
    cores = oracle.num_threads()
    reps = 0
    t0 = time.perf_counter()
    while True:
        lg = oracle.router_logits(x, wr, bias)
        idx, w = oracle.route_from_logits(lg, K, wl.scale, wl.norm_topk)
        counts, offsets, r2s, s2r = oracle.dispatch(idx, wl.E, 0)
        R = int(offsets[-1])
        y = np.zeros((max(R, 1), H), np.uint16)
        hh = {}
        for e in experts:
            a, b = offsets[e], offsets[e + 1]
            hh[e], y[a:b] = oracle.expert_ffn_rows(x[r2s[a:b] // K], *W[e], wl.limit)
        hs, ys = oracle.expert_ffn_rows(x, *SW, wl.limit) if SW else (None, None)
        oracle.combine(w, s2r, y, ys)
        dy, dw = oracle.combine_bwd(w, s2r, f64(y), dout)
        dx = np.zeros((Ts, H))
        for e in experts:
            a, b = offsets[e], offsets[e + 1]
            xr = x[r2s[a:b] // K]
            dh = oracle.down_bwd_rows(dy[a:b], W[e][2])
            dg, du = oracle.swiglu_bwd_rows(xr, W[e][0], W[e][1], dh, wl.limit)
            dxr = oracle.gateup_dgrad_rows(dg, du, W[e][0], W[e][1])
            oracle.wgrad(dy[a:b], f64(hh[e]))
            oracle.wgrad(dg, f64(xr))
            oracle.wgrad(du, f64(xr))
            np.add.at(dx, r2s[a:b] // K, dxr)
        if SW:
            dys = f64(dout)
            dh = oracle.down_bwd_rows(dys, SW[2])
            dg, du = oracle.swiglu_bwd_rows(x, SW[0], SW[1], dh, wl.limit)
            dx += oracle.gateup_dgrad_rows(dg, du, SW[0], SW[1])
            oracle.wgrad(dys, f64(hs))
            oracle.wgrad(dg, f64(x))
            oracle.wgrad(du, f64(x))
        dl = oracle.router_bwd(lg, idx, dw, wl.scale, wl.norm_topk, 0.0)
        oracle.wgrad(dl, f64(x))
        dx += dl @ f64(wr)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or reps >= max_reps:
            break
    return {"value": round(reps * Ts / dt, 3), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": "%d of the workload's %d tokens as a layer of their own, %d pass(es): forward "
                      "and backward steps (%d distinct routed experts + shared), fp64 C++ oracle"
                      % (Ts, wl.T, reps, len(experts))}


def train_step(args, wl, dev, layer):
    """One step = moe_layer_forward_train + moe_layer_backward (d_aux 0.01), HIP events around
    each."""
    import torch

    if wl.fp8:
        print("train mode takes bf16 expert weights", file=sys.stderr)
        sys.exit(2)
    stream = torch.cuda.current_stream()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4242)
    dout = torch.randn(wl.T, wl.H, generator=gen, device="cuda").to(torch.bfloat16)
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")
    for _ in range(args.warmup):
        layer.forward(dev["x"], out, train=True)
        layer.backward(dout, 0.01)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        layer.forward(dev["x"], out, train=True)
        layer.backward(dout, 0.01)
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    # forward / backward split from a second pass of the same steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record(stream)
        layer.forward(dev["x"], out, train=True)
        ev[i][1].record(stream)
        layer.backward(dout, 0.01)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    import numpy as np
    f_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    b_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    counts = layer.intermediate("counts", torch.int32, (wl.E,)).cpu().numpy()
    fwd_f, bwd_f = train_flops(wl, counts)
    a = bwd_f / (b_ms / 1e3) / 1e12
    res = {
        "metric": "MoE-layer training step (forward + backward) tokens/s at Hy4 shape",
        "value": round(wl.T / (ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "E": wl.E, "K": wl.K, "I": wl.I,
                   "n_shared": wl.n_shared, "mode": "train", "d_aux": 0.01,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(a, 2), "peak": PEAK_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(a / PEAK_MFMA_TFLOPS, 4), "traffic": None,
                     "kernel": "moe_layer_backward (all its kernels)", "algorithmic_flops": bwd_f,
                     "avg_launch_ms": round(b_ms, 4)},
        "phases_ms": {"forward": round(f_ms, 4), "backward": round(b_ms, 4)},
        "forward_mfma_frac": round(fwd_f / (f_ms / 1e3) / 1e12 / PEAK_MFMA_TFLOPS, 4),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_train(wl, dev, args.cpu_tokens or min(wl.T, 16))
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def generate_inputs(wl):
    from sparse_moe_layer_softmax_amd.workloads import generate
    return generate(wl, "cuda")


if __name__ == "__main__":
    main()
