#!/usr/bin/env python3
"""Benchmark of the MXFP4 W4A4 linear-layer path on one MI355X.

Default workload (the decode-shaped dense linear): an NVFP4 weight
[N=12288, K=4096] from bf16 N(0, 0.02) is requantized to MXFP4, then for each
M in {1, 8, 32, 64} bf16 activations [M, 4096] ~ N(0, 1) with 1% outlier
channels (x50) are quantized to MXFP4 and multiplied with the weight (bf16
out).  One step = requant + the four (act-quant, GEMM) pairs.  Weight sources
and destinations rotate over copies totalling > 768 MiB so that the bytes
come from HBM, not the 256 MiB Infinity Cache.

Other workloads (``--workload prefill|moe|layerwise``) print their own JSON
line; they are measurements of the remaining configurations.

Prints ONE JSON line.  ``value`` = GEMM TFLOP/s including activation
quantization (sum of 2MNK over the time of the act-quant + GEMM launches);
requant GB/s and roofline fractions are extra fields.  Each phase of a step
(the whole step, the act-quant + GEMM pairs, the GEMMs alone, ...) is captured
into HIP graphs, one per rotated weight copy, and timed by replaying them back
to back between two HIP events recorded on the stream the kernels run on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import pathlib
import sys
import time

ROOT = pathlib.Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "MXFP4 W4A4 GEMM TFLOP/s (incl. act quant) + requant GB/s, % of roofline"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MXFP4_PEAK_TFLOPS = 10100.0     # MI355X dense MXFP4 MFMA
ROTATE_BYTES = 1 << 30          # > 3x the 256 MiB MALL
CALIBRATION_BYTES = 512 << 20   # copy kernel of known size for the HBM counters
PREFILL_SLOTS = 16              # activation copies: 16 x 176 MiB over the three shapes
MOE_SLOTS = 8                   # token / down-input copies for the MoE workload


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="decode",
                   choices=["decode", "prefill", "moe", "layerwise", "w4a8"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--eager", type=int, default=0, metavar="N",
                   help="counter-collection pass: no graphs and no timing; run a "
                        "%d MiB copy (the calibration kernel), then every phase "
                        "N times eagerly" % (CALIBRATION_BYTES >> 20))
    return p.parse_args()


# ---- algorithmic bytes (per launch) ---------------------------------------------
def requant_bytes(T, N, K):          # codes+E4M3 in, codes+E8M0 out, one g per tensor
    return T * N * K * (0.5 + 1 / 16 + 0.5 + 1 / 32) + 4 * T


def act_quant_bytes(M, K):           # bf16 in, codes + E8M0 out
    return M * K * (2 + 0.5 + 1 / 32)


def gemm_bytes(M, N, K, out_bytes=2):  # both MXFP4 operands in, Y out
    return (M + N) * K * (0.5 + 1 / 32) + M * N * out_bytes


# The source files each measured kernel is built from (its traffic record is
# valid only while these hash to the digest stored with it).
KERNEL_SOURCES = {
    "requant": ("quant_kernels.hip", "mx_device.h"),
    "act_quant": ("quant_kernels.hip", "mx_device.h"),
    "gemm_decode": ("gemm_skinny.hip", "mx_device.h"),
    "gemm_prefill": ("gemm_tiled.hip", "mx_device.h"),
    "grouped_gemm_moe": ("gemm_tiled.hip", "mx_device.h"),
    "grouped_gemm_moe_step": ("gemm_tiled.hip", "mx_device.h"),
    "gemm_w4a8_decode": ("gemm_skinny.hip", "mx_device.h"),
}


def kernel_source_digest(tag=None):
    csrc = ROOT / "w4a4_mxfp4_gemm_amd" / "csrc"
    files = ([csrc / n for n in KERNEL_SOURCES[tag]] if tag else sorted(csrc.glob("*")))
    h = hashlib.sha256()
    for f in files:
        h.update(f.read_bytes())
    return h.hexdigest()[:16]


def recorded_traffic(kernel_tag):
    """HBM bytes per dispatch measured by rocprofv3 PMC runs (profiles/), valid
    only while the kernel's sources hash to the digest stored with them."""
    f = ROOT / "profiles" / f"{kernel_tag}_traffic.txt"
    if not f.exists():
        return None
    kv = {}
    for line in f.read_text().splitlines():
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_digest") != kernel_source_digest(kernel_tag):
        return None
    try:
        return float(kv["hbm_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


class Phases:
    """Named launch sequences captured into HIP graphs and timed by replaying
    the graphs back to back between two HIP events recorded on the stream the
    kernels run on.  The step phase gets one graph per rotation slot (one
    replay = one step); every other phase gets a single graph holding all slots
    in turn, repeated until it holds at least `min_launches` passes, so short
    kernels run back to back on the GPU and the time per pass is not bounded
    by the host's graph-launch rate."""

    def __init__(self, torch, slots, min_launches=20):
        self.torch = torch
        self.slots = slots
        self.rounds = max(1, math.ceil(min_launches / slots))
        self.fns = {}
        self.graphs = {}

    def add(self, name, fn):           # fn(slot) enqueues the phase's launches
        self.fns[name] = fn

    def capture(self):
        torch = self.torch
        for name, fn in self.fns.items():
            for r in range(self.slots):
                fn(r)                  # eager run first (also a correctness warm-up)
            torch.cuda.synchronize()
            if name == "step":
                gs = []
                for r in range(self.slots):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g):
                        fn(r)
                    gs.append(g)
            else:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for _ in range(self.rounds):
                        for r in range(self.slots):
                            fn(r)
                gs = [g]
            self.graphs[name] = gs
        torch.cuda.synchronize()

    def time(self, name, reps, warmup):
        """Average milliseconds per slot (per step for the step phase)."""
        torch = self.torch
        gs = self.graphs[name]
        per_replay = 1 if name == "step" else self.slots * self.rounds
        for i in range(warmup):
            gs[i % len(gs)].replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            gs[i % len(gs)].replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * per_replay)


# ---- workloads ------------------------------------------------------------------------
def decode_workload(torch, mx, synth):
    N, K, Ms = 12288, 4096, (1, 8, 32, 64)
    d = torch.device("cuda:0")
    w = synth.bf16_normal((N, K), 0.02, seed=11, device=d)
    codes, scales, g = synth.nvfp4_from_bf16(w)
    g = g.reshape(1)
    R = max(2, math.ceil(ROTATE_BYTES / requant_bytes(1, N, K)))
    src = [(codes.clone(), scales.clone(), g.clone()) for _ in range(R)]
    dst = [(torch.empty((N, K // 2), dtype=torch.uint8, device=d),
            torch.empty((N, K // 32), dtype=torch.uint8, device=d)) for _ in range(R)]
    x = synth.activations(64, K, seed=12, outlier_seed=13, device="cpu").to(d)
    xs = {M: x[:M].contiguous() for M in Ms}
    xq = {M: (torch.empty((M, K // 2), dtype=torch.uint8, device=d),
              torch.empty((M, K // 32), dtype=torch.uint8, device=d)) for M in Ms}
    ys = {M: torch.empty((M, N), dtype=torch.bfloat16, device=d) for M in Ms}

    def requant(r):
        c, s, gg = src[r]
        mx.mxfp4_requant_from_nvfp4(c, s, gg, *dst[r])

    def pair(r, M):
        mx.mxfp4_quantize_act(xs[M], *xq[M])
        mx.mxfp4_gemm(xq[M][0], xq[M][1], dst[r][0], dst[r][1], ys[M])

    ws_bytes = max(mx.mxfp4_linear_workspace_size(M, N, K) for M in Ms)
    ws = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=d)

    def linear(r, M):               # the same pair as one call
        mx.mxfp4_linear_bf16(xs[M], dst[r][0], dst[r][1], ys[M], workspace=ws)

    ph = Phases(torch, R)
    ph.add("step", lambda r: (requant(r), [linear(r, M) for M in Ms]))
    ph.add("linears", lambda r: [linear(r, M) for M in Ms])
    ph.add("pairs", lambda r: [pair(r, M) for M in Ms])
    ph.add("gemm", lambda r: [mx.mxfp4_gemm(xq[M][0], xq[M][1], dst[r][0], dst[r][1], ys[M])
                              for M in Ms])
    ph.add("requant", requant)
    for M in Ms:
        ph.add(f"linear_M{M}", lambda r, M=M: linear(r, M))
        ph.add(f"act_quant_M{M}", lambda r, M=M: mx.mxfp4_quantize_act(xs[M], *xq[M]))
        ph.add(f"gemm_M{M}", lambda r, M=M: mx.mxfp4_gemm(xq[M][0], xq[M][1], dst[r][0],
                                                           dst[r][1], ys[M]))

    def report(t, steps):
        flops = sum(2 * M * N * K for M in Ms)
        value = flops / (t["linears"] * 1e-3) / 1e12
        gb_req = requant_bytes(1, N, K) / (t["requant"] * 1e-3) / 1e9
        gemm_b = sum(gemm_bytes(M, N, K) for M in Ms)
        gemm_gbps = gemm_b / (t["gemm"] * 1e-3) / 1e9
        per_m = {}
        for M in Ms:
            ta, tg = t[f"act_quant_M{M}"], t[f"gemm_M{M}"]
            tl = t[f"linear_M{M}"]
            per_m[str(M)] = {
                "linear_us": round(tl * 1e3, 2),
                "linear_one_launch": mx.mxfp4_linear_workspace_size(M, N, K) == 0,
                "TFLOPs_linear": round(2 * M * N * K / (tl * 1e-3) / 1e12, 3),
                "act_quant_us": round(ta * 1e3, 2), "gemm_us": round(tg * 1e3, 2),
                "gemm_GBps": round(gemm_bytes(M, N, K) / (tg * 1e-3) / 1e9, 1),
                "gemm_frac_hbm": round(gemm_bytes(M, N, K) / (tg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "TFLOPs_incl_act_quant": round(2 * M * N * K / ((ta + tg) * 1e-3) / 1e12, 3),
            }
        roof = {"kernel": "mxfp4_gemm, decode (M=1,8,32,64)", "bound": "hbm",
                "achieved": round(gemm_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(gemm_gbps / HBM_PEAK_GBPS, 4),
                "traffic": recorded_traffic("gemm_decode"),
                "algorithmic_bytes_per_launch": round(gemm_b / len(Ms)),
                "avg_launch_us": round(t["gemm"] / len(Ms) * 1e3, 3)}
        extra = {"requant_GBps": round(gb_req, 1),
                 "requant_frac_hbm": round(gb_req / HBM_PEAK_GBPS, 4),
                 "requant_us": round(t["requant"] * 1e3, 2),
                 "linear_calls_us": round(t["linears"] * 1e3, 2),
                 "act_quant_plus_gemm_us": round(t["pairs"] * 1e3, 2),
                 "per_M": per_m, "weight_copies_rotated": R}
        cfg = {"workload": "decode-shaped dense linear: NVFP4->MXFP4 requant of W "
                           "[12288,4096] + act-quant + W4A4 GEMM for M in {1,8,32,64} "
                           "(mxfp4_linear_bf16), bf16 out",
               "N": N, "K": K, "M": list(Ms)}
        return value, "TFLOP/s", roof, extra, cfg

    def cpu_baseline():
        import numpy as np
        import oracle
        wc, ws, gg = codes.cpu().numpy(), scales.cpu().numpy(), g.cpu().numpy()
        xb = x.cpu().view(torch.int16).numpy().view(np.uint16)
        t0 = time.perf_counter()
        oc, os_ = oracle.requant(wc, ws, gg)
        t1 = time.perf_counter()
        reps = 0
        while True:
            for M in Ms:
                ac, as_ = oracle.quantize_act(xb[:M])
                oracle.gemm(ac, as_, oc, os_)
            reps += 1
            t2 = time.perf_counter()
            if t2 - t1 > 10.0:
                break
        flops = sum(2 * M * N * K for M in Ms) * reps
        return {"value": round(flops / (t2 - t1) / 1e12, 6), "unit": "TFLOP/s",
                "cores": oracle.num_threads(), "kind": "oracle",
                "sample": f"the whole workload: oracle requant of W [12288,4096] once "
                          f"({requant_bytes(1, N, K) / (t1 - t0) / 1e9:.3f} GB/s), then act-quant "
                          f"+ fp64 GEMM for M in {{1,8,32,64}} repeated {reps}x over >= 10 s",
                "seconds": round(t2 - t0, 2)}

    return ph, report, cpu_baseline


def prefill_workload(torch, mx, synth):
    M = 4096
    shapes = [(4096, 4096), (28672, 4096), (4096, 14336)]
    d = torch.device("cuda:0")
    data = []
    for (N, K), ws, xs_, os_ in zip(shapes, (21, 22, 23), (24, 24, 25), (26, 26, 27)):
        w = synth.bf16_normal((N, K), 0.02, seed=ws, device=d)
        c, s, g = synth.nvfp4_from_bf16(w)
        del w
        wc, wsc = mx.mxfp4_requant_from_nvfp4(c, s, g.reshape(1))
        x0 = synth.activations(M, K, seed=xs_, outlier_seed=os_, device=d)
        # rotated copies of the activations and their quantized form, so the
        # activation bytes come from HBM rather than the Infinity Cache
        x = [x0.clone() for _ in range(PREFILL_SLOTS)]
        xq = [(torch.empty((M, K // 2), dtype=torch.uint8, device=d),
               torch.empty((M, K // 32), dtype=torch.uint8, device=d))
              for _ in range(PREFILL_SLOTS)]
        y = torch.empty((M, N), dtype=torch.bfloat16, device=d)
        data.append((N, K, wc, wsc, x, xq, y))

    ph = Phases(torch, PREFILL_SLOTS)

    def step(r):
        for N, K, wc, wsc, x, xq, y in data:
            mx.mxfp4_quantize_act(x[r], *xq[r])
            mx.mxfp4_gemm(xq[r][0], xq[r][1], wc, wsc, y)

    ph.add("step", step)
    for N, K, wc, wsc, x, xq, y in data:
        ph.add(f"aq_{N}x{K}", lambda r, x=x, xq=xq: mx.mxfp4_quantize_act(x[r], *xq[r]))
        ph.add(f"gemm_{N}x{K}", lambda r, xq=xq, wc=wc, wsc=wsc, y=y:
               mx.mxfp4_gemm(xq[r][0], xq[r][1], wc, wsc, y))

    def report(t, steps):
        flops = sum(2 * M * N * K for N, K in shapes)
        value = flops / (t["step"] * 1e-3) / 1e12
        per = {}
        tg_all = 0.0
        for N, K in shapes:
            ta, tg = t[f"aq_{N}x{K}"], t[f"gemm_{N}x{K}"]
            tg_all += tg
            per[f"{N}x{K}"] = {"act_quant_us": round(ta * 1e3, 2), "gemm_us": round(tg * 1e3, 2),
                               "gemm_TFLOPs": round(2 * M * N * K / (tg * 1e-3) / 1e12, 1),
                               "TFLOPs_incl_act_quant": round(2 * M * N * K / ((ta + tg) * 1e-3) / 1e12, 1),
                               "act_quant_GBps": round(act_quant_bytes(M, K) / (ta * 1e-3) / 1e9, 1)}
        ach = flops / (tg_all * 1e-3) / 1e12
        roof = {"kernel": "mxfp4_gemm, prefill", "bound": "mfma", "achieved": round(ach, 1),
                "peak": MXFP4_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / MXFP4_PEAK_TFLOPS, 4),
                "traffic": recorded_traffic("gemm_prefill")}
        cfg = {"workload": "prefill dense linears M=4096, (N,K) in (4096,4096),(28672,4096),"
                           "(4096,14336): act-quant + W4A4 GEMM, bf16 out"}
        return value, "TFLOP/s", roof, {"per_shape": per}, cfg

    return ph, report, None


def moe_workload(torch, mx, synth):
    """One MoE layer's expert path: act-quant of the tokens, each written to its
    routed expert-sorted rows; the grouped gate_up GEMM with the expert
    activation + act-quant of the down input (silu(gate) * up) in its
    epilogue; the grouped down GEMM.  The top-k combine that ends the layer
    is timed beside it, and so is the step with the gate_up stage as two
    launches (grouped GEMM to bf16, then the activation kernel).  The fused
    call reads the gate_up weights as rows interleaved by 32 (gate, up); the
    synthetic weights are the same bytes either way."""
    E, T, TOPK = 128, 2048, 8
    d = torch.device("cuda:0")
    perm, offsets, rows, weights = synth.route_topk_full(T, E, TOPK, seed=34, device="cpu")
    perm, offsets, rows, weights = perm.to(d), offsets.to(d), rows.to(d), weights.to(d)
    tokens = synth.activations(T, 4096, seed=33, device=d)
    W = {}
    for name, (N, K), seed in (("gate_up", (2048, 4096), 31), ("down", (4096, 1024), 32)):
        wc = torch.empty((E, N, K // 2), dtype=torch.uint8, device=d)
        ws = torch.empty((E, N, K // 32), dtype=torch.uint8, device=d)
        for e in range(E):
            w = synth.bf16_normal((N, K), 0.02, seed=seed * 1000 + e, device=d)
            c, s, g = synth.nvfp4_from_bf16(w)
            mx.mxfp4_requant_from_nvfp4(c, s, g.reshape(1), wc[e], ws[e])
        W[name] = (N, K, wc, ws)
    Mtot = T * TOPK
    # rotated copies of the activation-side buffers (the expert weights,
    # 855 MB, exceed the Infinity Cache on their own)
    R = MOE_SLOTS
    tokens = [tokens.clone() for _ in range(R)]
    aq1 = [(torch.empty((Mtot, 2048), dtype=torch.uint8, device=d),
            torch.empty((Mtot, 128), dtype=torch.uint8, device=d)) for _ in range(R)]
    aq2 = [(torch.empty((Mtot, 512), dtype=torch.uint8, device=d),
            torch.empty((Mtot, 32), dtype=torch.uint8, device=d)) for _ in range(R)]
    y1 = [torch.empty((Mtot, 2048), dtype=torch.bfloat16, device=d) for _ in range(R)]
    y2 = [torch.empty((Mtot, 4096), dtype=torch.bfloat16, device=d) for _ in range(R)]
    out = [torch.empty((T, 4096), dtype=torch.bfloat16, device=d) for _ in range(R)]

    def aq_gate_up(r):
        # each token quantized once, written to its top-k expert-sorted rows
        mx.mxfp4_quantize_act_scatter(tokens[r], rows, *aq1[r])

    def aq_gate_up_gather(r):
        mx.mxfp4_quantize_act(tokens[r], *aq1[r], row_index=perm)

    def gemm_gate_up(r):
        mx.mxfp4_grouped_gemm(aq1[r][0], aq1[r][1], W["gate_up"][2], W["gate_up"][3], offsets,
                              y1[r])

    def act_down(r):
        mx.mxfp4_silu_mul_quantize(y1[r], *aq2[r])

    def gemm_down(r):
        mx.mxfp4_grouped_gemm(aq2[r][0], aq2[r][1], W["down"][2], W["down"][3], offsets, y2[r])

    def combine(r):
        mx.mxfp4_moe_combine(y2[r], rows, weights, out[r])

    def gate_up_glu(r):
        mx.mxfp4_grouped_gemm_silu_quantize(aq1[r][0], aq1[r][1], W["gate_up"][2],
                                            W["gate_up"][3], offsets, *aq2[r])

    def step(r):
        aq_gate_up(r), gate_up_glu(r), gemm_down(r)

    def step_two_call(r):
        aq_gate_up(r), gemm_gate_up(r), act_down(r), gemm_down(r)

    ph = Phases(torch, R)
    ph.add("step", step)
    ph.add("step_two_call", step_two_call)
    ph.add("layer", lambda r: (step(r), combine(r)))
    for f in (aq_gate_up, aq_gate_up_gather, gate_up_glu, gemm_gate_up, act_down, gemm_down,
              combine):
        ph.add(f.__name__, f)

    def report(t, steps):
        flops = 2 * Mtot * (2048 * 4096 + 4096 * 1024)
        value = flops / (t["step"] * 1e-3) / 1e12
        # the step's two grouped GEMMs: gate_up with the activation in its
        # epilogue (writes MXFP4 h), then down
        tg = t["gate_up_glu"] + t["gemm_down"]
        mx4 = 0.5 + 1 / 32
        gb = (E * 2048 * 4096 * mx4 + Mtot * 4096 * mx4 + Mtot * 1024 * mx4 +
              E * 4096 * 1024 * mx4 + Mtot * 1024 * mx4 + Mtot * 4096 * 2)
        ach = gb / (tg * 1e-3) / 1e9
        tg2 = t["gemm_gate_up"] + t["gemm_down"]
        gb2 = gb - Mtot * 1024 * mx4 + Mtot * 2048 * 2
        per = {k: round(t[k] * 1e3, 2) for k in ("aq_gate_up", "aq_gate_up_gather", "gate_up_glu",
                                                 "gemm_gate_up", "act_down", "gemm_down",
                                                 "combine")}
        # algorithmic bytes of the two epilogue kernels
        act_b = Mtot * 2048 * 2 + Mtot * 1024 * mx4
        comb_b = Mtot * 4096 * 2 + T * 4096 * 2 + T * TOPK * 8
        roof = {"kernel": "mxfp4_grouped_gemm_silu_quantize (gate_up) + mxfp4_grouped_gemm "
                          "(down)", "bound": "hbm",
                "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBPS, 4),
                "traffic": recorded_traffic("grouped_gemm_moe_step"),
                "algorithmic_bytes_per_launch": round(gb / 2),
                "avg_launch_us": round(tg / 2 * 1e3, 2),
                "gemm_TFLOPs": round(flops / (tg * 1e-3) / 1e12, 1)}
        extra = {"per_kernel_us": per,
                 "step_two_call_us": round(t["step_two_call"] * 1e3, 2),
                 "step_two_call_TFLOPs": round(flops / (t["step_two_call"] * 1e-3) / 1e12, 1),
                 "two_call_grouped_gemms_GBps": round(gb2 / (tg2 * 1e-3) / 1e9, 1),
                 "two_call_grouped_gemms_traffic": recorded_traffic("grouped_gemm_moe"),
                 "layer_us": round(t["layer"] * 1e3, 2),
                 "layer_TFLOPs": round(flops / (t["layer"] * 1e-3) / 1e12, 1),
                 "act_down_GBps": round(act_b / (t["act_down"] * 1e-3) / 1e9, 1),
                 "combine_GBps": round(comb_b / (t["combine"] * 1e-3) / 1e9, 1)}
        cfg = {"workload": "MoE 128 experts, 2048 tokens top-8: act-quant scattered to the "
                           "routed rows + grouped GEMM gate_up [2048,4096] with silu(gate)*up "
                           "act-quant in its epilogue + grouped GEMM down [4096,1024] "
                           "(layer_us adds the top-k combine)"}
        return value, "TFLOP/s", roof, extra, cfg

    return ph, report, None


def w4a8_workload(torch, mx, synth):
    """W4A8 (MXFP8 activations x the same MXFP4 weights): the decode-shaped
    layer W [12288, 4096] for M in {1, 8, 32, 64} through mxfp4_linear_w4a8_bf16
    with a bf16 row bias, weight copies rotated past the Infinity Cache; a
    prefill-shaped [4096, 4096] x [4096, 4096] W4A8 GEMM is timed beside it."""
    N, K, Ms = 12288, 4096, (1, 8, 32, 64)
    d = torch.device("cuda:0")
    w = synth.bf16_normal((N, K), 0.02, seed=11, device=d)
    codes, scales, g = synth.nvfp4_from_bf16(w)
    wc, ws = mx.mxfp4_requant_from_nvfp4(codes, scales, g.reshape(1))
    del w, codes, scales
    R = max(2, math.ceil(ROTATE_BYTES / gemm_bytes(0, N, K)))
    W = [(wc.clone(), ws.clone()) for _ in range(R)]
    bias = (torch.randn(N, generator=torch.Generator().manual_seed(3)) * 0.5).to(
        torch.bfloat16).to(d)
    x = synth.activations(64, K, seed=12, outlier_seed=13, device="cpu").to(d)
    xs = {M: x[:M].contiguous() for M in Ms}
    xq = {M: (torch.empty((M, K), dtype=torch.uint8, device=d),
              torch.empty((M, K // 32), dtype=torch.uint8, device=d)) for M in Ms}
    ys = {M: torch.empty((M, N), dtype=torch.bfloat16, device=d) for M in Ms}
    wsp = torch.empty((max(mx.mxfp4_linear_w4a8_workspace_size(M, N, K) for M in Ms),),
                      dtype=torch.uint8, device=d)
    PM, PN, PK = 4096, 4096, 4096
    xp = synth.activations(PM, PK, seed=24, outlier_seed=26, device=d)
    xpq = mx.mxfp8_quantize_act(xp)
    wp = synth.bf16_normal((PN, PK), 0.02, seed=21, device=d)
    cp, sp, gp = synth.nvfp4_from_bf16(wp)
    wpc, wps = mx.mxfp4_requant_from_nvfp4(cp, sp, gp.reshape(1))
    del wp, cp, sp
    yp = torch.empty((PM, PN), dtype=torch.bfloat16, device=d)

    def linear(r, M):
        mx.mxfp4_linear_w4a8_bf16(xs[M], W[r][0], W[r][1], ys[M], bias=bias, workspace=wsp)

    def gemm(r, M):
        mx.mxfp4_gemm_w4a8(xq[M][0], xq[M][1], W[r][0], W[r][1], ys[M], bias=bias)

    ph = Phases(torch, R)
    ph.add("step", lambda r: [linear(r, M) for M in Ms])
    ph.add("gemm", lambda r: [gemm(r, M) for M in Ms])
    for M in Ms:
        ph.add(f"linear_M{M}", lambda r, M=M: linear(r, M))
        ph.add(f"act_quant_M{M}", lambda r, M=M: mx.mxfp8_quantize_act(xs[M], *xq[M]))
        ph.add(f"gemm_M{M}", lambda r, M=M: gemm(r, M))
    ph.add("prefill_gemm", lambda r: mx.mxfp4_gemm_w4a8(xpq[0], xpq[1], wpc, wps, yp))

    def report(t, steps):
        flops = sum(2 * M * N * K for M in Ms)
        value = flops / (t["step"] * 1e-3) / 1e12
        wbytes = N * K * (0.5 + 1 / 32)
        gb = [wbytes + M * K * (1 + 1 / 32) + M * N * 2 + N * 2 for M in Ms]
        gemm_gbps = sum(gb) / (t["gemm"] * 1e-3) / 1e9
        per_m = {str(M): {"linear_us": round(t[f"linear_M{M}"] * 1e3, 2),
                          "linear_one_launch": mx.mxfp4_linear_w4a8_workspace_size(M, N, K) == 0,
                          "act_quant_us": round(t[f"act_quant_M{M}"] * 1e3, 2),
                          "gemm_us": round(t[f"gemm_M{M}"] * 1e3, 2),
                          "gemm_GBps": round(b / (t[f"gemm_M{M}"] * 1e-3) / 1e9, 1)}
                 for M, b in zip(Ms, gb)}
        pf = 2 * PM * PN * PK / (t["prefill_gemm"] * 1e-3) / 1e12
        roof = {"kernel": "mxfp4_gemm_w4a8, decode (M=1,8,32,64)", "bound": "hbm",
                "achieved": round(gemm_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(gemm_gbps / HBM_PEAK_GBPS, 4),
                "traffic": recorded_traffic("gemm_w4a8_decode"),
                "algorithmic_bytes_per_launch": round(sum(gb) / len(Ms)),
                "avg_launch_us": round(t["gemm"] / len(Ms) * 1e3, 3)}
        extra = {"dtype": "w4a8 (e4m3 x e2m1, e8m0 scales, fp32 acc)", "per_M": per_m,
                 "prefill_gemm_us": round(t["prefill_gemm"] * 1e3, 2),
                 "prefill_gemm_TFLOPs": round(pf, 1),
                 "prefill_gemm_frac_fp8_peak": round(pf / 5000.0, 4),
                 "weight_copies_rotated": R}
        cfg = {"workload": "W4A8 decode-shaped linear W [12288,4096], M in {1,8,32,64} "
                           "(mxfp4_linear_w4a8_bf16 with bf16 bias, bf16 out); beside it a "
                           "[4096,4096]x[4096,4096] W4A8 GEMM",
               "N": N, "K": K, "M": list(Ms)}
        return value, "TFLOP/s", roof, extra, cfg

    return ph, report, None


def layerwise_workload(torch, mx, synth):
    """One MoE layer's NVFP4 tensors resident in a one-layer scratch buffer,
    requantized into a 48-layer preallocated destination, layer after layer
    (kernel time only; 5% of tensors excluded and skipped)."""
    E, L = 128, 48
    d = torch.device("cuda:0")
    gen = torch.Generator().manual_seed(42)
    excluded = torch.rand((L, 2, E), generator=gen) < 0.05
    shapes = {0: (2048, 4096), 1: (4096, 1024)}
    src = {}
    for k, (N, K) in shapes.items():
        w = synth.bf16_normal((E, N, K), 0.02, seed=41 + k, device=d)
        src[k] = synth.nvfp4_from_bf16(w)
        del w
    dst = {k: (torch.empty((L, E, N, K // 2), dtype=torch.uint8, device=d),
               torch.empty((L, E, N, K // 32), dtype=torch.uint8, device=d))
           for k, (N, K) in shapes.items()}
    # one launch per layer and tensor kind: the experts not excluded, passed
    # as a tensor list (excluded slots of the destination stay untouched)
    calls = [(l, k, (~excluded[l, k]).nonzero().flatten().tolist())
             for l in range(L) for k in shapes]
    n_tensors = sum(len(keep) for _, _, keep in calls)

    def step(r):
        for l, k, keep in calls:
            c, s, g = src[k]
            mc, ms = dst[k]
            mx.mxfp4_requant_from_nvfp4(c, s, g, mc[l], ms[l], tensors=keep)

    ph = Phases(torch, 1)
    ph.add("step", step)

    def report(t, steps):
        tt = t["step"]
        b = sum(requant_bytes(len(keep), *shapes[k]) for _, k, keep in calls)
        gbps = b / (tt * 1e-3) / 1e9
        roof = {"kernel": "mxfp4_requant_from_nvfp4_subset", "bound": "hbm",
                "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": recorded_traffic("requant"),
                "algorithmic_bytes_per_launch": round(b / len(calls)),
                "avg_launch_us": round(tt / len(calls) * 1e3, 3)}
        cfg = {"workload": "layerwise load: 48 MoE layers x 128 experts x ([2048,4096] + "
                           "[4096,1024]) NVFP4 -> MXFP4, 5% of tensors excluded",
               "tensors_requantized": n_tensors, "launches": len(calls)}
        return gbps, "GB/s", roof, {"ms_all_layers": round(tt, 3)}, cfg

    return ph, report, None


def eager_pass(torch, ph, n):
    """For rocprofv3 --pmc runs: an elementwise kernel that reads and writes
    CALIBRATION_BYTES once each (torch's bitwise_not on u8; its FETCH_SIZE /
    WRITE_SIZE per byte calibrate the counters), then each phase other than
    the whole step, n times, eagerly."""
    src = torch.full((CALIBRATION_BYTES,), 1, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(n):
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    names = [k for k in ph.fns if k != "step"] or ["step"]
    for name in names:
        for i in range(n):
            ph.fns[name](i % ph.slots)
        torch.cuda.synchronize()
        print(f"eager phase {name}: {n} runs", flush=True)
    print(json.dumps({"eager": n, "calibration_copy_bytes": CALIBRATION_BYTES,
                      "phases": names}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this path has no multi-GPU mode "
              f"(--gpus {args.gpus} requested). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(2)
    import synth
    import w4a4_mxfp4_gemm_amd as mx

    make = {"decode": decode_workload, "prefill": prefill_workload, "moe": moe_workload,
            "layerwise": layerwise_workload, "w4a8": w4a8_workload}[args.workload]
    ph, report, cpu_baseline = make(torch, mx, synth)
    if args.eager:
        eager_pass(torch, ph, args.eager)
        return
    ph.capture()
    # the contract's timed region: exactly `steps` steps after `warmup` untimed ones
    t = {"step": ph.time("step", args.steps, args.warmup)}
    total_ms = t["step"] * args.steps
    reps = max(3, args.steps // max(1, ph.slots))
    for name in ph.fns:
        if name != "step":
            t[name] = ph.time(name, reps, 1)
    value, unit, roof, extra, cfg = report(t, args.steps)

    out = {"metric": METRIC, "value": round(value, 4), "unit": unit, "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(total_ms / args.steps, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "mxfp4 (e2m1 x e8m0, fp32 acc)",
           "data": "synthetic (seeded; NVFP4 weights from bf16 N(0,0.02), bf16 activations "
                   "N(0,1) with 1% outlier channels x50)",
           "config": cfg, "roofline": roof, **extra,
           "kernel_source_digest": kernel_source_digest()}
    if cpu_baseline is not None and not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
