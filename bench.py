#!/usr/bin/env python3
"""Benchmark of the MXFP4 W4A4 linear-layer path on one MI355X.

Headline workload (the largest single-GPU configuration): the prefill-shaped
dense linears, M = 4096 tokens of bf16 activations ~ N(0, 1) with 1% outlier
channels (x50), times MXFP4 weights requantized from NVFP4 (bf16 N(0, 0.02)),
for (N, K) in (4096, 4096), (28672, 4096), (4096, 14336).  One step = the
three act-quant + GEMM pairs (bf16 out); ``value`` = their 2MNK flops over the
step's time, i.e. GEMM TFLOP/s including the activation quantization.

The default run (``--workload all``) measures every other configuration in the
same process and adds it to the same JSON line:
* ``decode``: requant of W [12288, 4096] + act-quant + GEMM for M in
  {1, 8, 32, 64} (weight-streaming, HBM-bound);
* ``moe``: 128 experts, 2048 tokens top-8: dispatch act-quant, gate_up GEMM
  with the expert activation in its epilogue, down GEMM, top-k combine;
* ``layerwise``: 48 MoE layers x 128 experts x ([2048, 4096] + [4096, 1024])
  NVFP4 -> MXFP4, 5% excluded: kernel-only requant rate, and the end-to-end
  load from pinned host memory through the layerwise driver;
* ``w4a8``: MXFP8 activations with the same weights (decode and a 4096^3 GEMM);
* ``measured_peaks``: this GPU's own MFMA-loop and copy ceilings, with the
  clock the MFMAs ran at; every fraction is also given against them.

Each phase is captured into HIP graphs and timed by replaying them back to
back between two HIP events recorded on the stream the kernels run on (the
current torch stream, which the binding launches on).  Inputs are resident in
HBM before the timed region; the rotating copies exceed the 256 MiB Infinity
Cache, so the bytes come from HBM.  ``cpu_baseline`` times the CPU oracle, as
it stands, on a row sample of the headline workload on this host's cores.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import pathlib
import platform
import sys
import time

ROOT = pathlib.Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "MXFP4 W4A4 GEMM TFLOP/s (incl. act quant) + requant GB/s, % of roofline"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MXFP4_PEAK_TFLOPS = 10100.0     # MI355X dense MXFP4 MFMA
FP8_PEAK_TFLOPS = 5000.0        # MI355X dense FP8 MFMA (W4A8's E4M3 x E2M1 runs at this rate)
ROTATE_BYTES = 1 << 30          # > 3x the 256 MiB MALL
CALIBRATION_BYTES = 512 << 20   # copy kernel of known size for the HBM counters
PREFILL_SLOTS = 16              # activation copies: 16 x 176 MiB over the three shapes
MOE_SLOTS = 8                   # token / down-input copies for the MoE workload
MX4 = 0.5 + 1 / 32              # MXFP4 bytes per element (codes + E8M0)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="all",
                   choices=["all", "prefill", "decode", "moe", "layerwise", "w4a8"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--eager", type=int, default=0, metavar="N",
                   help="counter-collection pass for one workload: no graphs and no "
                        "timing; run a %d MiB copy (the calibration kernel), then every "
                        "phase N times eagerly" % (CALIBRATION_BYTES >> 20))
    return p.parse_args()


def say(msg):
    print(msg, file=sys.stderr, flush=True)


# ---- algorithmic bytes (per launch) ---------------------------------------------
def requant_bytes(T, N, K):          # codes+E4M3 in, codes+E8M0 out, one g per tensor
    return T * N * K * (0.5 + 1 / 16 + 0.5 + 1 / 32) + 4 * T


def act_quant_bytes(M, K):           # bf16 in, codes + E8M0 out
    return M * K * (2 + MX4)


def gemm_bytes(M, N, K, out_bytes=2):  # both MXFP4 operands in, Y out
    return (M + N) * K * MX4 + M * N * out_bytes


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


def recorded_traffic(kernel_tag, key="hbm_bytes_per_dispatch"):
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
        return float(kv[key])
    except (KeyError, ValueError):
        return None


class Phases:
    """Named launch sequences captured into HIP graphs and timed by replaying
    the graphs back to back between two HIP events recorded on the stream the
    kernels run on.  The step phase gets one graph per rotation slot (one
    replay = one step) for the warm-up and the per-step distribution, and its
    timed steps replay graphs that each hold G consecutive steps (G = gcd of
    the step count and the slot count), since each graph launch leaves the GPU
    idle for a few microseconds.  Every other phase gets a single graph holding
    all slots in turn, repeated until it holds at least `min_launches` passes,
    so short kernels run back to back on the GPU and the time per pass is not
    bounded by the host's graph-launch rate."""

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

    def chained_steps(self, g):
        """Graphs of g consecutive steps, slots / g of them, covering the slots
        in order (g divides the slot count)."""
        torch = self.torch
        fn = self.fns["step"]
        gs = []
        for b in range(self.slots // g):
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for r in range(b * g, b * g + g):
                    fn(r)
            gs.append(graph)
        torch.cuda.synchronize()
        return gs

    def time(self, name, reps, warmup, per_rep=None):
        """Average milliseconds per slot (per step for the step phase).  With
        `per_rep` (a list, step phase only), a second pass of `reps` steps, one
        graph and one event per step, appends each step's milliseconds to it;
        the average comes from the first pass alone."""
        torch = self.torch
        gs = self.graphs[name]
        per_replay = 1 if name == "step" else self.slots * self.rounds
        timed, n = gs, reps
        if name == "step":
            self.steps_per_graph = g = math.gcd(reps, self.slots)
            if g > 1:
                timed, n = self.chained_steps(g), reps // g
        for i in range(warmup):
            gs[i % len(gs)].replay()
        # A graph's first replay carries one-time set-up work of the runtime
        # (building its launch packets); run each chained graph once, untimed,
        # so the timed steps are steady-state ones like the warm-up's.
        self.first_replay_steps = 0
        if timed is not gs:
            for graph in timed:
                graph.replay()
            self.first_replay_steps = len(timed) * (reps // n)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            timed[i % len(timed)].replay()
        e1.record()
        torch.cuda.synchronize()
        if per_rep is not None:
            marks = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
            marks[0].record()
            for i in range(reps):
                gs[i % len(gs)].replay()
                marks[i + 1].record()
            torch.cuda.synchronize()
            per_rep.extend(a.elapsed_time(b) / per_replay for a, b in zip(marks, marks[1:]))
        return e0.elapsed_time(e1) / (reps * per_replay)

    def time_all(self, reps):
        return {name: self.time(name, reps, 1) for name in self.fns if name != "step"}


def roofline(kernel, bound, achieved, peak, unit, traffic, per_launch, avg_us, measured=None):
    r = {"kernel": kernel, "bound": bound, "achieved": round(achieved, 1), "peak": peak,
         "unit": unit, "frac": round(achieved / peak, 4), "traffic": traffic,
         "algorithmic_per_launch": per_launch, "avg_launch_us": round(avg_us, 3)}
    if measured:
        r["measured_peak"] = round(measured, 1)
        r["frac_of_measured_peak"] = round(achieved / measured, 4)
    return r


# ---- host / CPU description for the CPU baselines ----------------------------------
def host_info():
    model = platform.processor() or "unknown"
    try:
        for line in pathlib.Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    aff = sorted(os.sched_getaffinity(0))
    runs, start = [], aff[0] if aff else 0
    for a, b in zip(aff, aff[1:] + [None]):
        if b != a + 1:
            runs.append(f"{start}-{a}" if a != start else f"{a}")
            start = b
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity": ",".join(runs),
            "affinity_cpus": len(aff)}


# ---- workloads ------------------------------------------------------------------------
def prefill_workload(torch, mx, synth):
    M = 4096
    shapes = [(4096, 4096), (28672, 4096), (4096, 14336)]
    d = torch.device("cuda:0")
    data, nv_host = [], []
    for (N, K), ws, xs_, os_ in zip(shapes, (21, 22, 23), (24, 24, 25), (26, 26, 27)):
        w = synth.bf16_normal((N, K), 0.02, seed=ws, device=d)
        c, s, g = synth.nvfp4_from_bf16(w)
        del w
        wc, wsc = mx.mxfp4_requant_from_nvfp4(c, s, g.reshape(1))
        nv_host.append((c.cpu(), s.cpu(), g.reshape(1).cpu()))
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

    def vendor_library():
        """The platform's MXFP4 GEMM (hipBLASLt, through torch._scaled_mm with
        E2M1 operands and E8M0 scales) on the same quantized operands, beside
        this library's GEMM, both timed the same way: eager launches between
        two events, after a warm-up, interleaved.  Context only, outside the
        timed region: hipBLASLt reads the scale tensors in a layout of its own,
        so its outputs differ (max_rel_diff) and only its time compares."""
        out = {"how": "torch._scaled_mm (hipBLASLt) vs mxfp4_gemm, 10 eager launches "
                      "between events after 3, medians of 5 interleaved rounds; timing only"}
        try:
            f4, e8 = torch.float4_e2m1fn_x2, torch.float8_e8m0fnu
            for N, K, wc, wsc, x, xq, y in data:
                a, sa = xq[0]
                lt = lambda: torch._scaled_mm(a.view(f4), wc.view(f4).t(), scale_a=sa.view(e8),
                                              scale_b=wsc.view(e8), out_dtype=torch.bfloat16)
                ours = lambda: mx.mxfp4_gemm(a, sa, wc, wsc, y)
                times = {"hipblaslt": [], "ours": []}
                for fn in (lt, ours):
                    for _ in range(3):
                        fn()
                for _ in range(5):
                    for name, fn in (("hipblaslt", lt), ("ours", ours)):
                        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                        e0.record()
                        for _ in range(10):
                            fn()
                        e1.record()
                        torch.cuda.synchronize()
                        times[name].append(e0.elapsed_time(e1) / 10 * 1e3)
                yl = lt().float()
                ours()
                torch.cuda.synchronize()
                tl, to = sorted(times["hipblaslt"])[2], sorted(times["ours"])[2]
                out[f"{N}x{K}"] = {
                    "hipblaslt_us": round(tl, 2), "ours_us": round(to, 2),
                    "hipblaslt_TFLOPs": round(2 * M * N * K / (tl * 1e-6) / 1e12, 1),
                    "ours_TFLOPs": round(2 * M * N * K / (to * 1e-6) / 1e12, 1),
                    "max_rel_diff": float(((yl - y.float()).abs().max() / y.float().abs().max()).item())}
                del yl
        except Exception as ex:                 # the vendor path is optional context
            out["error"] = repr(ex)[:300]
        return out

    def report(t, peaks):
        flops = sum(2 * M * N * K for N, K in shapes)
        value = flops / (t["step"] * 1e-3) / 1e12
        per = {}
        tg_all = 0.0
        for N, K in shapes:
            ta, tg = t[f"aq_{N}x{K}"], t[f"gemm_{N}x{K}"]
            tg_all += tg
            gb = act_quant_bytes(M, K) / (ta * 1e-3) / 1e9
            per[f"{N}x{K}"] = {
                "act_quant_us": round(ta * 1e3, 2), "gemm_us": round(tg * 1e3, 2),
                "gemm_TFLOPs": round(2 * M * N * K / (tg * 1e-3) / 1e12, 1),
                "TFLOPs_incl_act_quant": round(2 * M * N * K / ((ta + tg) * 1e-3) / 1e12, 1),
                "act_quant_GBps": round(gb, 1), "act_quant_frac_hbm": round(gb / HBM_PEAK_GBPS, 4)}
        # the dominant kernel: the 28672 x 4096 GEMM (seven rounds of 256 x 256 tiles)
        N, K = 28672, 4096
        tg = t[f"gemm_{N}x{K}"]
        ach = 2 * M * N * K / (tg * 1e-3) / 1e12
        roof = roofline("mxfp4_gemm M=4096 N=28672 K=4096 (gemm_dense_kernel), bf16 out",
                        "mfma", ach, MXFP4_PEAK_TFLOPS, "TFLOP/s",
                        recorded_traffic("gemm_prefill", "hbm_bytes_per_dispatch_28672x4096"),
                        {"flop": 2 * M * N * K, "bytes": gemm_bytes(M, N, K)}, tg * 1e3,
                        peaks.get("mfma_TFLOPs"))
        extra = {"per_shape": per,
                 "three_gemms_TFLOPs": round(flops / (tg_all * 1e-3) / 1e12, 1),
                 "step_frac_mfma_peak": round(value / MXFP4_PEAK_TFLOPS, 4)}
        if peaks.get("mfma_TFLOPs"):
            extra["step_frac_of_measured_mfma_peak"] = round(value / peaks["mfma_TFLOPs"], 4)
        extra["vendor_library"] = vendor_library()
        cfg = {"workload": "prefill dense linears M=4096, (N,K) in (4096,4096),(28672,4096),"
                           "(4096,14336): act-quant + W4A4 GEMM, bf16 out",
               "M": M, "NK": [list(s) for s in shapes]}
        return value, "TFLOP/s", roof, extra, cfg

    def cpu_baseline():
        """The oracle on a row sample of the step: act-quant of the sampled
        rows, then the exact GEMM against each whole weight (requantized by
        the oracle beforehand, not timed), all threads on 1024 rows and one
        thread on 32 rows, each scaled to TFLOP/s of the same flops."""
        import numpy as np
        import oracle
        ops = []
        for (N, K), (c, s, g), (_, _, _, _, x, _, _) in zip(shapes, nv_host, data):
            oc, os_ = oracle.requant(c.numpy(), s.numpy(), g.numpy())
            xb = x[0].cpu().view(torch.int16).numpy().view(np.uint16)
            ops.append((N, K, oc, os_, xb))

        def run(rows, threads):
            oracle.set_num_threads(threads)
            t0 = time.perf_counter()
            flops = 0
            for N, K, oc, os_, xb in ops:
                ac, as_ = oracle.quantize_act(xb[rows])
                oracle.gemm(ac, as_, oc, os_)
                flops += 2 * len(rows) * N * K
            return flops, time.perf_counter() - t0

        all_threads = oracle.num_threads()
        rows_all = np.arange(0, M, M // 1024)
        f_all, t_all = run(rows_all, all_threads)
        f_one, t_one = run(np.arange(0, M, M // 32), 1)
        oracle.set_num_threads(all_threads)
        return {"value": round(f_all / t_all / 1e12, 6), "unit": "TFLOP/s",
                "cores": all_threads, "kind": "oracle",
                "sample": f"{len(rows_all)} of the 4096 rows (every 4th) through act-quant + "
                          f"exact GEMM for the three (N,K), all {all_threads} threads: "
                          f"{t_all:.2f} s; scaled by flops",
                "seconds": round(t_all, 2),
                "single_thread": {"value": round(f_one / t_one / 1e12, 6), "unit": "TFLOP/s",
                                  "sample": "32 rows (every 128th), 1 thread",
                                  "seconds": round(t_one, 2)},
                **host_info()}

    return ph, report, cpu_baseline


def decode_workload(torch, mx, synth):
    N, K, Ms = 12288, 4096, (1, 8, 32, 64)
    d = torch.device("cuda:0")
    w = synth.bf16_normal((N, K), 0.02, seed=11, device=d)
    codes, scales, g = synth.nvfp4_from_bf16(w)
    del w
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
    ws_bytes = max(mx.mxfp4_linear_workspace_size(M, N, K) for M in Ms)
    ws = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=d)

    def requant(r):
        c, s, gg = src[r]
        mx.mxfp4_requant_from_nvfp4(c, s, gg, *dst[r])

    def linear(r, M):
        mx.mxfp4_linear_bf16(xs[M], dst[r][0], dst[r][1], ys[M], workspace=ws)

    def gemm(r, M):
        mx.mxfp4_gemm(xq[M][0], xq[M][1], dst[r][0], dst[r][1], ys[M])

    ph = Phases(torch, R)
    ph.add("step", lambda r: (requant(r), [linear(r, M) for M in Ms]))
    ph.add("linears", lambda r: [linear(r, M) for M in Ms])
    ph.add("gemm", lambda r: [gemm(r, M) for M in Ms])
    ph.add("requant", requant)
    for M in Ms:
        ph.add(f"linear_M{M}", lambda r, M=M: linear(r, M))
        ph.add(f"act_quant_M{M}", lambda r, M=M: mx.mxfp4_quantize_act(xs[M], *xq[M]))
        ph.add(f"gemm_M{M}", lambda r, M=M: gemm(r, M))

    def report(t, peaks):
        flops = sum(2 * M * N * K for M in Ms)
        gemm_b = sum(gemm_bytes(M, N, K) for M in Ms)
        gemm_gbps = gemm_b / (t["gemm"] * 1e-3) / 1e9
        gb_req = requant_bytes(1, N, K) / (t["requant"] * 1e-3) / 1e9
        copy = peaks.get("copy_GBps")
        per_m = {}
        for M in Ms:
            ta, tg, tl = t[f"act_quant_M{M}"], t[f"gemm_M{M}"], t[f"linear_M{M}"]
            gb = gemm_bytes(M, N, K) / (tg * 1e-3) / 1e9
            per_m[str(M)] = {
                "linear_us": round(tl * 1e3, 2),
                "linear_one_launch": mx.mxfp4_linear_workspace_size(M, N, K) == 0,
                "TFLOPs_linear": round(2 * M * N * K / (tl * 1e-3) / 1e12, 3),
                "act_quant_us": round(ta * 1e3, 2), "gemm_us": round(tg * 1e3, 2),
                "gemm_GBps": round(gb, 1), "gemm_frac_hbm": round(gb / HBM_PEAK_GBPS, 4)}
        return {
            "workload": "decode-shaped dense linear: requant of W [12288,4096] + act-quant + "
                        "W4A4 GEMM for M in {1,8,32,64} (mxfp4_linear_bf16), bf16 out",
            "step_ms": round(t["step"], 4),
            "TFLOPs_incl_act_quant": round(flops / (t["linears"] * 1e-3) / 1e12, 3),
            "roofline": roofline("mxfp4_gemm decode (M=1,8,32,64), gemm_skinny", "hbm",
                                 gemm_gbps, HBM_PEAK_GBPS, "GB/s", recorded_traffic("gemm_decode"),
                                 {"bytes": round(gemm_b / len(Ms))},
                                 t["gemm"] / len(Ms) * 1e3, copy),
            "requant": roofline("mxfp4_requant_from_nvfp4 W [12288,4096]", "hbm", gb_req,
                                HBM_PEAK_GBPS, "GB/s", recorded_traffic("requant"),
                                {"bytes": requant_bytes(1, N, K)}, t["requant"] * 1e3, copy),
            "per_M": per_m, "weight_copies_rotated": R}

    def cpu_baseline():
        import numpy as np
        import oracle
        wc, wsc, gg = codes.cpu().numpy(), scales.cpu().numpy(), g.cpu().numpy()
        xb = x.cpu().view(torch.int16).numpy().view(np.uint16)
        t0 = time.perf_counter()
        oc, os_ = oracle.requant(wc, wsc, gg)
        t1 = time.perf_counter()
        for M in Ms:
            ac, as_ = oracle.quantize_act(xb[:M])
            oracle.gemm(ac, as_, oc, os_)
        t2 = time.perf_counter()
        return {"TFLOPs": round(sum(2 * M * N * K for M in Ms) / (t2 - t1) / 1e12, 6),
                "requant_GBps": round(requant_bytes(1, N, K) / (t1 - t0) / 1e9, 3),
                "cores": oracle.num_threads(), "kind": "oracle",
                "sample": "the whole workload once: requant, then act-quant + exact GEMM for "
                          "M in {1,8,32,64}", "seconds": round(t2 - t0, 2)}

    return ph, report, cpu_baseline


def moe_workload(torch, mx, synth):
    """One MoE layer's expert path: act-quant of the tokens, each written to its
    routed expert-sorted rows; the grouped gate_up GEMM with the expert
    activation + act-quant of the down input (silu(gate) * up) in its
    epilogue; the grouped down GEMM.  The top-k combine that ends the layer
    is timed beside it, and so is the step with the gate_up stage as two
    launches (grouped GEMM to bf16, then the activation kernel).  The fused
    call reads the gate_up weights as rows interleaved by 32 (gate, up); the
    synthetic weights are the same bytes either way.  The expert weight codes
    are pre-shuffled into the grouped GEMMs' operand order at load time."""
    E, T, TOPK = 128, 2048, 8
    d = torch.device("cuda:0")
    perm, offsets, rows, weights = synth.route_topk_full(T, E, TOPK, seed=34, device="cpu")
    perm, offsets, rows, weights = perm.to(d), offsets.to(d), rows.to(d), weights.to(d)
    tokens = synth.activations(T, 4096, seed=33, device=d)
    W = {}
    SAMPLE_EXPERTS = (0, 41, 87, 127)              # the CPU baseline's experts
    W_rows = {}                                    # their row-major codes, on the host
    for name, (N, K), seed in (("gate_up", (2048, 4096), 31), ("down", (4096, 1024), 32)):
        wc = torch.empty((E, N, K // 2), dtype=torch.uint8, device=d)
        ws = torch.empty((E, N, K // 32), dtype=torch.uint8, device=d)
        for e in range(E):
            w = synth.bf16_normal((N, K), 0.02, seed=seed * 1000 + e, device=d)
            c, s, g = synth.nvfp4_from_bf16(w)
            mx.mxfp4_requant_from_nvfp4(c, s, g.reshape(1), wc[e], ws[e])
        W_rows[name] = wc[list(SAMPLE_EXPERTS)].cpu()
        # load time: the codes go into the grouped GEMMs' operand order
        W[name] = (N, K, mx.mxfp4_preshuffle_weights(wc), ws)
        del wc
    Mtot = T * TOPK
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
        mx.mxfp4_quantize_act_scatter(tokens[r], rows, *aq1[r])

    def aq_gate_up_gather(r):
        mx.mxfp4_quantize_act(tokens[r], *aq1[r], row_index=perm)

    def gemm_gate_up(r):
        mx.mxfp4_grouped_gemm(aq1[r][0], aq1[r][1], W["gate_up"][2], W["gate_up"][3], offsets,
                              y1[r], b_preshuffled=True)

    def act_down(r):
        mx.mxfp4_silu_mul_quantize(y1[r], *aq2[r])

    def gemm_down(r):
        mx.mxfp4_grouped_gemm(aq2[r][0], aq2[r][1], W["down"][2], W["down"][3], offsets, y2[r],
                              b_preshuffled=True)

    def combine(r):
        mx.mxfp4_moe_combine(y2[r], rows, weights, out[r])

    def gate_up_glu(r):
        mx.mxfp4_grouped_gemm_silu_quantize(aq1[r][0], aq1[r][1], W["gate_up"][2],
                                            W["gate_up"][3], offsets, *aq2[r],
                                            b_preshuffled=True)

    def step(r):
        aq_gate_up(r), gate_up_glu(r), gemm_down(r)

    ph = Phases(torch, R)
    ph.add("step", step)
    ph.add("step_two_call", lambda r: (aq_gate_up(r), gemm_gate_up(r), act_down(r),
                                       gemm_down(r)))
    ph.add("layer", lambda r: (step(r), combine(r)))
    for f in (aq_gate_up, aq_gate_up_gather, gate_up_glu, gemm_gate_up, act_down, gemm_down,
              combine):
        ph.add(f.__name__, f)

    def report(t, peaks):
        flops = 2 * Mtot * (2048 * 4096 + 4096 * 1024)
        tg = t["gate_up_glu"] + t["gemm_down"]
        gb = (E * 2048 * 4096 * MX4 + Mtot * 4096 * MX4 + Mtot * 1024 * MX4 +
              E * 4096 * 1024 * MX4 + Mtot * 1024 * MX4 + Mtot * 4096 * 2)
        ach = gb / (tg * 1e-3) / 1e9
        tg2 = t["gemm_gate_up"] + t["gemm_down"]
        gb2 = gb - Mtot * 1024 * MX4 + Mtot * 2048 * 2
        act_b = Mtot * 2048 * 2 + Mtot * 1024 * MX4
        comb_b = Mtot * 4096 * 2 + T * 4096 * 2 + T * TOPK * 8
        return {
            "workload": "MoE 128 experts, 2048 tokens top-8: act-quant scattered to the routed "
                        "rows + grouped GEMM gate_up [2048,4096] with silu(gate)*up act-quant in "
                        "its epilogue + grouped GEMM down [4096,1024]; layer adds the combine",
            "step_us": round(t["step"] * 1e3, 2),
            "TFLOPs_incl_act_quant": round(flops / (t["step"] * 1e-3) / 1e12, 1),
            "roofline": roofline("mxfp4_grouped_gemm_silu_quantize (gate_up) + "
                                 "mxfp4_grouped_gemm (down)", "hbm", ach, HBM_PEAK_GBPS, "GB/s",
                                 recorded_traffic("grouped_gemm_moe_step"), {"bytes": round(gb / 2)},
                                 tg / 2 * 1e3, peaks.get("copy_GBps")),
            "grouped_gemms_TFLOPs": round(flops / (tg * 1e-3) / 1e12, 1),
            "per_kernel_us": {k: round(t[k] * 1e3, 2) for k in (
                "aq_gate_up", "aq_gate_up_gather", "gate_up_glu", "gemm_gate_up", "act_down",
                "gemm_down", "combine")},
            "step_two_call_us": round(t["step_two_call"] * 1e3, 2),
            "two_call_grouped_gemms_GBps": round(gb2 / (tg2 * 1e-3) / 1e9, 1),
            "layer_us": round(t["layer"] * 1e3, 2),
            "layer_TFLOPs": round(flops / (t["layer"] * 1e-3) / 1e12, 1),
            "act_down_GBps": round(act_b / (t["act_down"] * 1e-3) / 1e9, 1),
            "combine_GBps": round(comb_b / (t["combine"] * 1e-3) / 1e9, 1)}

    def cpu_baseline():
        """Four experts' rows through the oracle's act-quant + exact gate_up and
        down GEMMs, scaled by flops."""
        import numpy as np
        import oracle
        off = offsets.cpu().numpy()
        tok = tokens[0].cpu().view(torch.int16).numpy().view(np.uint16)
        pm = perm.cpu().numpy()
        gu_s = W["gate_up"][3].cpu().numpy()
        dn_s = W["down"][3].cpu().numpy()
        gu_c, dn_c = W_rows["gate_up"].numpy(), W_rows["down"].numpy()
        t0 = time.perf_counter()
        flops = 0
        for i, e in enumerate(SAMPLE_EXPERTS):
            r0, r1 = int(off[e]), int(off[e + 1])
            ac, as_ = oracle.quantize_act(tok, row_index=pm[r0:r1])
            oracle.gemm(ac, as_, gu_c[i], gu_s[e])
            hc = np.zeros((r1 - r0, 512), np.uint8)
            hs = np.full((r1 - r0, 32), 127, np.uint8)
            oracle.gemm(hc, hs, dn_c[i], dn_s[e])
            flops += 2 * (r1 - r0) * (2048 * 4096 + 4096 * 1024)
        dt = time.perf_counter() - t0
        return {"TFLOPs": round(flops / dt / 1e12, 6), "cores": oracle.num_threads(),
                "kind": "oracle", "sample": "4 experts' routed rows: act-quant + exact gate_up "
                "and down GEMMs, scaled by flops", "seconds": round(dt, 2)}

    return ph, report, cpu_baseline


def w4a8_workload(torch, mx, synth):
    """W4A8 (MXFP8 activations x the same MXFP4 weights): the decode-shaped
    layer W [12288, 4096] for M in {1, 8, 32, 64} through mxfp4_linear_w4a8_bf16
    with a bf16 row bias, weight copies rotated past the Infinity Cache; a
    prefill-shaped [4096, 4096] x [4096, 4096] W4A8 GEMM beside it."""
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

    def report(t, peaks):
        flops = sum(2 * M * N * K for M in Ms)
        wbytes = N * K * MX4
        gb = [wbytes + M * K * (1 + 1 / 32) + M * N * 2 + N * 2 for M in Ms]
        gemm_gbps = sum(gb) / (t["gemm"] * 1e-3) / 1e9
        per_m = {str(M): {"linear_us": round(t[f"linear_M{M}"] * 1e3, 2),
                          "linear_one_launch": mx.mxfp4_linear_w4a8_workspace_size(M, N, K) == 0,
                          "act_quant_us": round(t[f"act_quant_M{M}"] * 1e3, 2),
                          "gemm_us": round(t[f"gemm_M{M}"] * 1e3, 2),
                          "gemm_GBps": round(b / (t[f"gemm_M{M}"] * 1e-3) / 1e9, 1)}
                 for M, b in zip(Ms, gb)}
        pf = 2 * PM * PN * PK / (t["prefill_gemm"] * 1e-3) / 1e12
        return {"workload": "W4A8 decode-shaped linear W [12288,4096], M in {1,8,32,64} "
                            "(mxfp4_linear_w4a8_bf16 with bf16 bias); a [4096]^3 W4A8 GEMM",
                "dtype": "w4a8 (e4m3 x e2m1, e8m0 scales, fp32 acc)",
                "TFLOPs_incl_act_quant": round(flops / (t["step"] * 1e-3) / 1e12, 3),
                "roofline": roofline("mxfp4_gemm_w4a8 decode (M=1,8,32,64)", "hbm", gemm_gbps,
                                     HBM_PEAK_GBPS, "GB/s", recorded_traffic("gemm_w4a8_decode"),
                                     {"bytes": round(sum(gb) / len(Ms))},
                                     t["gemm"] / len(Ms) * 1e3, peaks.get("copy_GBps")),
                "per_M": per_m, "prefill_gemm_us": round(t["prefill_gemm"] * 1e3, 2),
                "prefill_gemm_TFLOPs": round(pf, 1),
                "prefill_gemm_frac_fp8_peak": round(pf / FP8_PEAK_TFLOPS, 4)}

    return ph, report, None


def layerwise_workload(torch, mx, synth):
    """The layerwise load, 48 MoE layers x 128 experts x ([2048,4096] +
    [4096,1024]) with 5% of the tensors excluded, measured two ways:
    * kernel only: one layer's NVFP4 source resident in HBM, requantized into
      the 48-layer destination one launch per layer and tensor kind (the
      subset requant), timed like the other phases;
    * end to end: the layerwise driver streaming every layer from pinned host
      memory (a pool of 2 distinct layers, layer l = pool[l % 2]) through a
      one-layer scratch into the same destination, copies on their own
      stream overlapping the requant, timed by the host around one call."""
    E, L, P = 128, 48, 2
    d = torch.device("cuda:0")
    gen = torch.Generator().manual_seed(42)
    excluded = torch.rand((L, 2, E), generator=gen) < 0.05
    shapes = {0: (2048, 4096), 1: (4096, 1024)}
    src, pool = {}, []
    for p in range(P):
        layer = []
        for k, (N, K) in shapes.items():
            w = synth.bf16_normal((E, N, K), 0.02, seed=41 + 10 * p + k, device=d)
            c, s, g = synth.nvfp4_from_bf16(w)
            del w
            if p == 0:
                src[k] = (c, s, g)
            host = []
            for t in (c, s, g):
                h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
                h.copy_(t)
                host.append(h)
            layer.append(host)
        pool.append(layer)
    dst = {k: (torch.empty((L, E, N, K // 2), dtype=torch.uint8, device=d),
               torch.empty((L, E, N, K // 32), dtype=torch.uint8, device=d))
           for k, (N, K) in shapes.items()}
    calls = [(l, k, (~excluded[l, k]).nonzero().flatten().tolist())
             for l in range(L) for k in shapes]
    n_tensors = sum(len(keep) for _, _, keep in calls)
    layer_bytes = sum(E * (N * K // 2 + N * K // 16) for N, K in shapes.values())
    scratch = torch.empty(layer_bytes, dtype=torch.uint8, device=d)
    parts = [dict(nv_codes=pool[l % P][k][0], nv_scales=pool[l % P][k][1],
                  nv_global=pool[l % P][k][2], excluded=excluded[l, k].to(torch.uint8),
                  mx_codes=dst[k][0][l], mx_scales=dst[k][1][l])
             for l in range(L) for k in shapes]
    copied = sum(int((~excluded[l, k]).sum()) * (N * K // 2 + N * K // 16)
                 for l in range(L) for k, (N, K) in shapes.items())

    def step(r):
        for l, k, keep in calls:
            c, s, g = src[k]
            mc, ms = dst[k]
            mx.mxfp4_requant_from_nvfp4(c, s, g, mc[l], ms[l], tensors=keep)

    ph = Phases(torch, 1, min_launches=1)
    ph.add("step", step)

    def end_to_end(runs=2):
        cs = torch.cuda.Stream(d)
        best = None
        for _ in range(runs):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            mx.mxfp4_requant_layers_from_host(parts, scratch, copy_stream=cs)
            torch.cuda.synchronize()
            dt = time.perf_counter() - t0
            best = dt if best is None else min(best, dt)
        return best

    def report(t, peaks):
        tt = t["step"]
        b = sum(requant_bytes(len(keep), *shapes[k]) for _, k, keep in calls)
        gbps = b / (tt * 1e-3) / 1e9
        e2e = end_to_end()
        return {"workload": "layerwise load: 48 MoE layers x 128 experts x ([2048,4096] + "
                            "[4096,1024]) NVFP4 -> MXFP4, 5% of tensors excluded",
                "tensors_requantized": n_tensors, "launches": len(calls),
                "roofline": roofline("mxfp4_requant_from_nvfp4_subset (kernel only, source "
                                     "resident)", "hbm", gbps, HBM_PEAK_GBPS, "GB/s",
                                     recorded_traffic("requant"),
                                     {"bytes": round(b / len(calls))}, tt / len(calls) * 1e3,
                                     peaks.get("copy_GBps")),
                "kernel_ms_all_layers": round(tt, 3),
                "end_to_end": {"seconds": round(e2e, 3),
                               "host_to_device_GB": round(copied / 1e9, 2),
                               "host_to_device_GBps": round(copied / e2e / 1e9, 1),
                               "scratch_bytes": layer_bytes, "pool_layers": P,
                               "how": "mxfp4_requant_layers_from_host over all 48 layers, "
                                      "pinned host source, copies on a second stream; best "
                                      "of 2 runs"}}

    def cpu_baseline():
        import oracle
        c, s, g = (u.cpu().numpy() for u in src[0])
        t0 = time.perf_counter()
        oracle.requant(c[:8], s[:8], g[:8])
        dt = time.perf_counter() - t0
        return {"GBps": round(requant_bytes(8, 2048, 4096) / dt / 1e9, 3),
                "cores": oracle.num_threads(), "kind": "oracle",
                "sample": "8 gate_up tensors [2048,4096]", "seconds": round(dt, 2)}

    return ph, report, cpu_baseline


WORKLOADS = {"prefill": prefill_workload, "decode": decode_workload, "moe": moe_workload,
             "layerwise": layerwise_workload, "w4a8": w4a8_workload}


# ---- this GPU's own ceilings ------------------------------------------------------------
def measure_peaks(torch):
    """MFMA-loop TFLOP/s with its clock, and copy GB/s (read + write), from
    libmxfp4_calibrate.so; {} if that library is missing."""
    lib_path = ROOT / "w4a4_mxfp4_gemm_amd" / "libmxfp4_calibrate.so"
    if not lib_path.exists():
        return {}
    lib = ctypes.CDLL(str(lib_path))
    lib.mxfp4_calibrate_mfma.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p]
    lib.mxfp4_calibrate_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                         ctypes.c_int, ctypes.c_void_p]
    lib.mxfp4_calibrate_mfma_flop_per_round.restype = ctypes.c_double
    d = torch.device("cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream(d).cuda_stream)
    waves = lib.mxfp4_calibrate_mfma_waves()
    clocks = torch.zeros(2 * waves, dtype=torch.int64, device=d)
    sink = torch.zeros(256 * 256, dtype=torch.float32, device=d)
    iters = 40000
    out = {}

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms = timed(lambda: lib.mxfp4_calibrate_mfma(iters, ctypes.c_void_p(clocks.data_ptr()),
                                                ctypes.c_void_p(sink.data_ptr()), stream), 3)
    flop = waves * iters * lib.mxfp4_calibrate_mfma_flop_per_round()
    c = clocks.cpu().view(-1, 2).double()
    ghz = float((c[:, 0] / (c[:, 1] / 100e6)).mean() / 1e9)
    out["mfma_TFLOPs"] = round(flop / (ms * 1e-3) / 1e12, 1)
    out["mfma_clock_GHz"] = round(ghz, 3)
    out["mfma_how"] = ("one wavefront per SIMD, back-to-back 32x32x64 E2M1 scaled MFMAs on "
                       "operands that change every round; clock from the shader and 100 MHz "
                       "counters of each wave")
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=d)
    b = torch.empty(n, dtype=torch.uint8, device=d)
    a.fill_(1)
    best = None
    for cfg in range(lib.mxfp4_calibrate_copy_configs()):
        ms = timed(lambda: lib.mxfp4_calibrate_copy(ctypes.c_void_p(a.data_ptr()),
                                                    ctypes.c_void_p(b.data_ptr()), n, cfg,
                                                    stream), 5)
        best = ms if best is None else min(best, ms)
    out["copy_GBps"] = round(2 * n / (best * 1e-3) / 1e9, 1)
    out["copy_how"] = ("1 GiB copy, 16-byte loads and stores, fastest of a few launch shapes "
                       "(plain and non-temporal), read + write counted")
    del a, b
    return out


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

    headline = "prefill" if args.workload == "all" else args.workload
    extras = [w for w in WORKLOADS if w != headline] if args.workload == "all" else []
    if args.eager:
        ph, _, _ = WORKLOADS[headline](torch, mx, synth)
        eager_pass(torch, ph, args.eager)
        return

    peaks = measure_peaks(torch) if args.workload == "all" else {}
    say(f"measured peaks: {peaks}")
    ph, report, cpu_baseline = WORKLOADS[headline](torch, mx, synth)
    ph.capture()
    # the contract's timed region: exactly `steps` steps after `warmup` untimed ones,
    # synchronised on both sides (one process, one GPU)
    per_step = []
    t = {"step": ph.time("step", args.steps, args.warmup, per_step)}
    steps_per_graph = ph.steps_per_graph
    first_replay_steps = ph.first_replay_steps
    total_ms = t["step"] * args.steps
    q = sorted(per_step)
    pick = lambda f: q[min(len(q) - 1, int(round(f * (len(q) - 1))))]
    reps = max(3, args.steps // max(1, ph.slots))
    t.update(ph.time_all(reps))
    rep = report(t, peaks)
    if isinstance(rep, dict):
        # another workload as the headline (--workload decode, moe, ...): its
        # report's own rate and roofline
        roof = rep["roofline"]
        value = rep.get("TFLOPs_incl_act_quant")
        unit = "TFLOP/s"
        if value is None:
            value, unit = roof["achieved"], roof["unit"]
        cfg = {"workload": rep["workload"]}
        extra = {k: v for k, v in rep.items() if k not in ("roofline", "workload")}
    else:
        value, unit, roof, extra, cfg = rep
    say(f"{headline}: {value:.1f} {unit}")
    del ph
    torch.cuda.synchronize()

    more = {}
    for name in extras:
        wph, wreport, wcpu = WORKLOADS[name](torch, mx, synth)
        wph.capture()
        wt = {"step": wph.time("step", max(3, args.steps // 2), 2)}
        wt.update(wph.time_all(max(2, args.steps // (2 * max(1, wph.slots)))))
        more[name] = wreport(wt, peaks)
        if wcpu is not None and not args.no_cpu_baseline:
            more[name]["cpu_baseline"] = wcpu()
        say(f"{name}: done")
        del wph, wreport, wcpu
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    out = {"metric": METRIC, "value": round(value, 4), "unit": unit, "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(total_ms / args.steps, 4),
           "steps_per_graph": steps_per_graph,
           "untimed_first_replay_steps": first_replay_steps,
           "step_ms_median_p10_p90": [round(pick(0.5), 4), round(pick(0.1), 4), round(pick(0.9), 4)],
           "step_ms_median_p10_p90_pass": "a second pass of the same steps, one graph and "
                                          "one event per step",
           "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "mxfp4 (e2m1 x e8m0, fp32 acc)",
           "data": "synthetic (seeded; NVFP4 weights from bf16 N(0,0.02), bf16 activations "
                   "N(0,1) with 1% outlier channels x50)",
           "config": cfg, "roofline": roof, **extra, **more}
    if peaks:
        out["measured_peaks"] = peaks
    out["kernel_source_digest"] = kernel_source_digest()
    if cpu_baseline is not None and not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
