#!/usr/bin/env python3
"""Benchmark of the quantized-linear hot path on one MI355X.

A call is one pass of the per-call path over one batch of synthetic input,
inputs resident in HBM: ``quantize_act`` (smoothing, FWHT-64, per-token
quantization), the branch projection where a workload has a low-rank
branch, then the GEMM with its dequant epilogue and fused 16-bit branch.
Weight packing is offline and outside every timed region.

Headline ("value"): the batch-1 64-token action-expert step, a W4A4
projection 64x2048x2048 plus a W8A8 down projection 64x2048x8192, as
effective TOPS = sum 2*M*N*K / step time.

"configs": every workload of the scope, each timed
* warm: a HIP graph of G back-to-back calls on one input set, replayed;
  the set stays in the caches between calls;
* cold: a HIP graph whose calls rotate over S independent input sets
  (activations, codes, packed weights, outputs) totalling at least
  640 MB, more than the 256 MB last-level cache, so every call finds its
  operands evicted by the other sets' traffic; no flush sits inside the
  timed region;
and, the same two ways, each kernel of the call alone.  HIP events on the
replay stream bracket each replay; figures are the median and the 10th /
90th percentile over replays of the per-call average.

Prints one JSON line.  ``--summarize-profiles DIR`` turns rocprofv3 output
of this script into the summaries under profiles/ (no GPU).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
PEAK_CLOCK_GHZ = 2.4           # MI355X peak engine clock
# dense matrix-core peaks (TFLOP/s, TOP/s for int8)
PEAK_T = {"i8": 5000.0, "fp8": 5000.0, "f16": 2500.0, "bf16": 2500.0, "fp4": 10100.0, "fp6": 10100.0}
COLD_BYTES = 640e6             # input sets per cold rotation: more than twice the 256 MB last-level cache
METRIC = "W4A4 linear effective TOPS + us/call (batch-1 64-token and 4096-token shapes)"

# The scope's workloads: id, workload name, what it is
CONFIGS = [
    ("C1", "tiny", "W4A4 16x256x256, fp32 in/out, smoothing + FWHT-64"),
    ("C2a", "decode_w4a4", "batch-1 step, W4A4 projection 64x2048x2048"),
    ("C2b", "decode_w8a8", "batch-1 step, W8A8 down projection 64x2048x8192"),
    ("C3-gu", "prefill_gate_up", "512-token prefill, fused gate/up W4A4 512x16384x2048"),
    ("C3-dn", "prefill_down", "512-token prefill, down W4A4 512x2048x8192"),
    ("C4", "lowrank", "1024-token W4A4 1024x3072x3072 + rank-32 bf16 branch"),
    ("C5", "video_nvfp4", "4096-token video-latent NVFP4 4096x5120x5120 + 64 kept bf16 channels"),
]
HEADLINE = ("batch1", ["decode_w4a4", "decode_w8a8"],
            "batch-1 64-token action-expert step: W4A4 64x2048x2048 + W8A8 64x2048x8192, "
            "smoothing + FWHT-64 + per-token quantization")
# further workloads, measured alone with --workload
EXTRA = {
    "batch1_a8": (["decode_w4a8", "decode_w4a8_down"], "batch-1 step at 8-bit activations: W4A8 64x2048x2048 "
                                                       "+ W4A8 64x2048x8192"),
    "video4096_a8": (["video_w4a8"], "4096-token video projection at 8-bit activations, W4A8 4096x5120x5120"),
    "batch1_fp8": (["decode_w4a4", "decode_fp8"], "batch-1 step with the down projection in FP8 (E4M3) W8A8"),
    "video4096_fp8": (["video_fp8"], "4096-token video projection in FP8 (E4M3) W8A8 4096x5120x5120"),
}
# the ranked next rows' workloads, measured in the default run after the
# configurations: id, workload name, row
NEXT = [
    ("N1a", "decode_w4a8", "W4A8 (8-bit activations, 4-bit weights) 64x2048x2048"),
    ("N1b", "decode_w4a8_down", "W4A8 64x2048x8192"),
    ("N1c", "video_w4a8", "W4A8 4096x5120x5120 + 64 kept bf16 channels"),
    ("N3a", "decode_fp8", "FP8 (E4M3) W8A8 64x2048x8192"),
    ("N3b", "video_fp8", "FP8 (E4M3) W8A8 4096x5120x5120 + 64 kept bf16 channels"),
]
REPLAYS, WARMUP_REPLAYS = 20, 3


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200, help="calls per timed region of the headline step")
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default=None, choices=[c[0] for c in CONFIGS] + list(EXTRA),
                   help="measure one workload only (no headline, no CPU baseline)")
    p.add_argument("--replays", type=int, default=REPLAYS)
    p.add_argument("--no-configs", action="store_true", help="headline step only")
    p.add_argument("--no-next", action="store_true", help="skip the next rows' workloads (W4A8, FP8)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain elementwise copy of 256 MiB five times (hardware-counter scale)")
    p.add_argument("--summarize-profiles", metavar="DIR",
                   help="turn rocprofv3 outputs under DIR into the summaries under profiles/ and exit (no GPU)")
    return p.parse_args()


# ---------------------------------------------------------------------------
# Algorithmic work per kernel
# ---------------------------------------------------------------------------
def gemm_bytes(case):
    """Algorithmic HBM bytes of one GEMM launch: packed weight and activation
    codes, their scales, the output and the branch operands."""
    M, N, K = case.M, case.N, case.K
    code_a = {"int4": 0.5, "int8": 1.0, "nvfp4": 0.5, "w4a8": 1.0, "fp8": 1.0}[case.fmt]
    code_w = {"int4": 0.5, "int8": 1.0, "nvfp4": 0.5, "w4a8": 0.5, "fp8": 1.0}[case.fmt]
    scales = (M + N) * K / 16 if case.fmt == "nvfp4" else 4 * (M + N)
    out = M * N * (4 if case.y_dtype == "f32" else 2)
    br = 0
    if case.branch is not None:
        r = case.branch["lw"].shape[1]
        ra = 2 * r if case.branch["kind"] == "lowrank" else r
        br = 2 * (M * ra + N * r)
    return code_a * M * K + code_w * N * K + scales + out + br


def quant_bytes(case, fused_branch_cols=0):
    """Algorithmic bytes of quantize_act: X in, codes and scales out (+ a
    branch operand written from the same pass)."""
    M, K = case.M, case.K
    xin = M * K * (2 if case.x_dtype == "bf16" else 4)
    codes = M * K * (1.0 if case.fmt in ("int8", "w4a8", "fp8") else 0.5)
    scales = M * K / 16 if case.fmt == "nvfp4" else 4 * M
    return xin + codes + scales + 2 * M * fused_branch_cols


def proj_bytes(case):
    r = case.branch["lw"].shape[1]
    return 2 * case.M * case.K + 2 * r * case.K + 2 * case.M * 2 * r


def mfma_type(fmt):
    return {"int4": "i8", "int8": "i8", "nvfp4": "f16", "w4a8": "i8", "fp8": "fp8"}[fmt]


def gemm_roof(case, us):
    """Roofline of the GEMM launch: HBM below the matrix type's ridge, else the
    matrix-core peak of the instruction actually issued."""
    flop = 2.0 * case.M * case.N * case.K
    byt = gemm_bytes(case)
    t = mfma_type(case.fmt)
    ridge = PEAK_T[t] * 1e12 / (HBM_PEAK_GBS * 1e9)
    if flop / byt < ridge:
        a = byt / (us * 1e-6) / 1e9
        return {"bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": a / HBM_PEAK_GBS,
                "algorithmic_bytes": byt}
    a = flop / (us * 1e-6) / 1e12
    r = {"bound": "mfma", "mfma": t, "achieved": a, "peak": PEAK_T[t], "unit": "TOP/s" if t == "i8" else "TFLOP/s",
         "frac": a / PEAK_T[t], "algorithmic_ops": flop}
    if case.fmt == "nvfp4":
        r["frac_of_fp4_peak"] = a / PEAK_T["fp4"]
    return r


def hbm_roof(byt, us):
    a = byt / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": a / HBM_PEAK_GBS,
            "algorithmic_bytes": byt}


# ---------------------------------------------------------------------------
# Timing
# ---------------------------------------------------------------------------
PHASE_LOG = []


def marker(torch, name=None):
    """A short spin kernel before and after each timed phase: the profiler's
    kernel trace splits into the phases listed under ``profile_phases``
    (dispatches between an end and the next start are set-up)."""
    torch.cuda.synchronize()
    torch.cuda._sleep(100)
    torch.cuda.synchronize()
    if name is not None:
        PHASE_LOG.append(name)


def pct(v, q):
    s = sorted(v)
    if not s:
        return None
    i = (len(s) - 1) * q
    lo, hi = int(math.floor(i)), int(math.ceil(i))
    return s[lo] + (s[hi] - s[lo]) * (i - lo)


def time_graph(torch, fns, replays, name):
    """Per-call microseconds of ``fns`` (a list of zero-argument callables, one
    per call, run in order) captured into one HIP graph and replayed; one
    pair of HIP events per replay.  Returns {median, p10, p90, mean}."""
    marker(torch, name)
    for f in fns[:2]:
        f()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fns[0]()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for f in fns:
            f()
    stream = torch.cuda.current_stream()
    for _ in range(WARMUP_REPLAYS):
        graph.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(replays)]
    for e0, e1 in ev:
        e0.record(stream)
        graph.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    per = [e0.elapsed_time(e1) * 1e3 / len(fns) for e0, e1 in ev]
    marker(torch)
    del graph
    return {"median": pct(per, 0.5), "p10": pct(per, 0.1), "p90": pct(per, 0.9), "mean": sum(per) / len(per)}


def set_bytes(case, layer):
    """Bytes one independent input set holds on the device."""
    b = layer.buffers(case.M, "cuda")
    n = case.M * case.K * (2 if case.x_dtype == "bf16" else 4)
    for t in [b["codes"], b["scales"], b["y"], b["br_a"], layer.w_codes, layer.w_scales]:
        if t is not None:
            n += t.numel() * t.element_size()
    if layer.branch is not None:
        n += layer.branch["lw"].numel() * 2
    return n


def build(name):
    from w4a4_post_quantized_channel_amd import pipeline, workloads as WL
    case = WL.workload(name)
    layer, t = pipeline.build_layer(case, device="cuda")
    layer.buffers(case.M, t["x"].device)
    return case, layer, t


def measure_case(torch, cid, name, replays, cold=True, built=None):
    """Warm and cold per-call and per-kernel times of one workload."""
    case, layer, t = built or build(name)
    x = t["x"]
    M = case.M
    proj = layer.has_projection(x.dtype)
    kernels = {"call": lambda L, xx: L.forward(xx), "quantize": lambda L, xx: L.quantize(xx)}
    if proj:
        kernels["project"] = lambda L, xx: L.project(xx)
    kernels["gemm"] = lambda L, xx: L.gemm(M, xx.device)
    layer.forward(x)                       # every buffer filled once
    torch.cuda.synchronize()
    G = 20 if M * case.N * case.K >= 1 << 30 else 100
    res = {"id": cid, "workload": name, "M": case.M, "N": case.N, "K": case.K, "fmt": case.fmt,
           "warm": {}, "cold": None}
    for k, f in kernels.items():
        res["warm"][k] = time_graph(torch, [lambda f=f: f(layer, x)] * G, replays, f"{cid} warm {k}")
    if layer.branch is not None and layer.branch["kind"] == "lowrank" and not layer.fuse_lowrank:
        # the single-read alternative (quantize_act_lowrank), timed beside the default two kernels
        layer.fuse_lowrank = True
        res["warm"]["fused_quantize_project"] = time_graph(torch, [lambda: layer.quantize(x)] * G, replays,
                                                           f"{cid} warm fused_quantize_project")
        layer.fuse_lowrank = False
        layer.forward(x)
    if cold:
        S = max(2, int(math.ceil(COLD_BYTES / set_bytes(case, layer))))
        sets = [(layer, x)] + [(layer.replica(), x.clone()) for _ in range(S - 1)]
        for L, xx in sets:
            L.forward(xx)
        torch.cuda.synchronize()
        res["cold"] = {"sets": S, "set_MB": set_bytes(case, layer) / 1e6}
        for k, f in kernels.items():
            res["cold"][k] = time_graph(torch, [lambda f=f, L=L, xx=xx: f(L, xx) for L, xx in sets], replays,
                                        f"{cid} cold {k}")
        del sets
        torch.cuda.synchronize()
    return case, layer, res


def vendor_gemm(torch, case):
    """The vendor library's dense GEMM at the workload's shape, for context:
    int8 x int8 -> int32 (torch._int_mm) for the integer formats, bf16
    (torch.matmul) for NVFP4 and FP8, whose matrix type here is 16-bit /
    8-bit float.  Warm graph replays; None when the library refuses."""
    M, N, K = case.M, case.N, case.K
    try:
        if case.fmt in ("int4", "int8", "w4a8"):
            a = torch.randint(-128, 127, (max(M, 32), K), device="cuda", dtype=torch.int8)
            b = torch.randint(-128, 127, (K, N), device="cuda", dtype=torch.int8)
            f, kind = (lambda: torch._int_mm(a, b)), "int8 torch._int_mm"
        else:
            a = torch.randn(M, K, device="cuda", dtype=torch.bfloat16)
            b = torch.randn(K, N, device="cuda", dtype=torch.bfloat16)
            f, kind = (lambda: torch.matmul(a, b)), "bf16 torch.matmul"
        f()
        torch.cuda.synchronize()
        r = time_graph(torch, [f] * 10, 10, f"vendor {case.name}")
        return {"kind": kind, "us": r["median"], "TOPS": 2.0 * max(M, 32 if "int8" in kind else M) * N * K
                / (r["median"] * 1e-6) / 1e12}
    except Exception as e:
        return {"kind": "unavailable", "note": str(e)[:100]}


def summarize_case(case, layer, res):
    """Effective TOPS and roofline fractions from the measured medians."""
    flop = 2.0 * case.M * case.N * case.K
    out = {"id": res["id"], "workload": res["workload"], "shape": f"{case.M}x{case.N}x{case.K}", "fmt": case.fmt}
    fused_cols, fused_extra = 0, 0
    if layer.branch is not None and not layer.has_projection():
        r = layer.branch["lw"].shape[1]
        if layer.branch["kind"] == "lowrank":   # T hi/lo written, L1 read by the same launch
            fused_cols, fused_extra = 2 * r, 2 * r * case.K
        else:                                   # the kept channels gathered from the same pass
            fused_cols = r
    for mode in ("warm", "cold"):
        r = res[mode]
        if r is None:
            continue
        m = {"us_per_call": r["call"], "effective_TOPS": flop / (r["call"]["median"] * 1e-6) / 1e12}
        ks = {}
        ks["quantize"] = {"us": r["quantize"], **hbm_roof(quant_bytes(case, fused_cols) + fused_extra,
                                                          r["quantize"]["median"])}
        if "project" in r:
            ks["project"] = {"us": r["project"], **hbm_roof(proj_bytes(case), r["project"]["median"])}
        if "fused_quantize_project" in r:   # not part of the call: the single-read alternative
            ks["fused_quantize_project"] = {"us": r["fused_quantize_project"], "in_call": False,
                                            **hbm_roof(quant_bytes(case, 2 * layer.branch["lw"].shape[1])
                                                       + 2 * layer.branch["lw"].shape[1] * case.K,
                                                       r["fused_quantize_project"]["median"])}
        ks["gemm"] = {"us": r["gemm"], **gemm_roof(case, r["gemm"]["median"])}
        m["kernels"] = ks
        if mode == "cold":
            m["sets"], m["set_MB"] = r["sets"], round(r["set_MB"], 2)
        out[mode] = m
    return out


def measure_headline(torch, names, steps, replays):
    from w4a4_post_quantized_channel_amd import pipeline, workloads as WL
    built = []
    for n in names:
        case = WL.workload(n)
        layer, t = pipeline.build_layer(case, device="cuda")
        layer.buffers(case.M, t["x"].device)
        built.append((case, layer, t))
    torch.cuda.synchronize()

    def step():
        for case, layer, t in built:
            layer.forward(t["x"])
    G = max(1, min(steps, 200))
    warm = time_graph(torch, [step] * G, replays, "headline warm step")
    flops = sum(2.0 * c.M * c.N * c.K for c, _, _ in built)
    return built, warm, flops


# ---------------------------------------------------------------------------
# Measured ceilings
# ---------------------------------------------------------------------------
def ceilings(torch):
    """What the chip sustains on plain work, measured the same way: a device
    copy (read + write), and the vendor library's dense GEMMs."""
    out = {}
    n = 256 << 20                                    # 1 GiB of fp32 per buffer
    a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    r = time_graph(torch, [lambda: b.copy_(a)] * 5, 10, "ceiling copy")
    out["copy_GBs"] = 2 * 4 * n / (r["median"] * 1e-6) / 1e9
    del a, b
    x = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    y = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    r = time_graph(torch, [lambda: torch.matmul(x, y)] * 5, 10, "ceiling bf16 gemm")
    out["bf16_gemm_TFLOPs"] = 2 * 8192 ** 3 / (r["median"] * 1e-6) / 1e12
    try:
        xi = torch.randint(-128, 127, (8192, 8192), device="cuda", dtype=torch.int8)
        yi = torch.randint(-128, 127, (8192, 8192), device="cuda", dtype=torch.int8)
        torch._int_mm(xi, yi)
        torch.cuda.synchronize()
        r = time_graph(torch, [lambda: torch._int_mm(xi, yi)] * 5, 10, "ceiling int8 gemm")
        out["int8_gemm_TOPs"] = 2 * 8192 ** 3 / (r["median"] * 1e-6) / 1e12
    except Exception as e:                           # the library may not offer it
        out["int8_gemm_TOPs"] = None
        out["int8_gemm_note"] = str(e)[:120]
    out["how"] = ("graph replays of 5 launches, median of 10: copy of 1 GiB fp32 (bytes read + written), "
                  "torch.matmul bf16 8192^3, torch._int_mm int8 8192^3")
    return out


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on the host cores
# ---------------------------------------------------------------------------
def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(names_ops, rows=32, min_s=0.3):
    """The oracle as it stands (NumPy; BLAS for the products) timing one call
    of every workload -- activation transform and quantization, GEMM,
    epilogue, branch; weights quantized (and, for NVFP4, decoded)
    beforehand -- on the first ``rows`` and ``2 rows`` rows; the call's cost
    is fitted as fixed + per-row and evaluated at the full M.  Two legs: one
    thread, and BLAS on every core of this process's CPU share (at most 16)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import w4a4_oracle as O
    from w4a4_post_quantized_channel_amd import workloads as WL
    host = len(os.sched_getaffinity(0))
    allc = min(host, 16)
    res = {}
    for cid, name in names_ops:
        c = WL.workload(name)
        fa, fw = O.OPERAND_FORMATS[c.fmt]
        W = O.quantize_operand(c.w, c.s, fw)
        g_a = O.nvfp4_tensor_scale(O.transformed_amax(c.x, c.inv_s)) if c.fmt == "nvfp4" else None
        w_dec = O.dequantize_nvfp4(W["codes"], W["scales"], W["g"]) if c.fmt == "nvfp4" else None

        def one(xs):
            A = O.quantize_operand(xs, c.inv_s, fa, g=g_a)
            if c.fmt in ("int4", "int8", "w4a8"):
                y = O.dequant_epilogue(O.int_gemm(A["codes"], W["codes"]), A["scales"], W["scales"])
            elif c.fmt == "fp8":
                y = O.dequant_epilogue(O.fp8_gemm(A["codes"], W["codes"]), A["scales"], W["scales"])
            else:
                y = O.dequantize_nvfp4(A["codes"], A["scales"], A["g"]) @ w_dec.T
            if c.branch is not None:
                if c.branch["kind"] == "lowrank":
                    y = y + O.lowrank_branch(xs, c.branch["l1"], c.branch["lw"])
                else:
                    y = y + O.outlier_branch(xs, c.branch["idx"], c.branch["lw"])
            return y

        ms = [c.M] if c.M <= 2 * rows else [rows, 2 * rows]
        entry = {"rows_timed": ms, "M": c.M}
        for leg, nthr in (("single", 1), ("all", allc)):
            with threadpool_limits(limits=nthr):
                used = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
                t = []
                for m in ms:
                    xs = np.ascontiguousarray(c.x[:m])
                    ts = []
                    t_end = time.perf_counter() + min_s
                    while len(ts) < 3 or (time.perf_counter() < t_end and len(ts) < 20):
                        t0 = time.perf_counter()
                        one(xs)
                        ts.append(time.perf_counter() - t0)
                    t.append(sorted(ts)[len(ts) // 2])
            if len(ms) == 1:
                us = t[0] * 1e6
            else:
                per_row = max(0.0, (t[1] - t[0]) / (ms[1] - ms[0]))
                us = (max(0.0, t[0] - per_row * ms[0]) + per_row * c.M) * 1e6
            entry[leg] = {"threads": int(used), "us_per_call": us,
                          "effective_TOPS": 2.0 * c.M * c.N * c.K / (us * 1e-6) / 1e12}
        res[cid] = entry
    return res, host, allc


# ---------------------------------------------------------------------------
# Copy calibration for the byte counters
# ---------------------------------------------------------------------------
def copy_calibration(torch):
    """Five launches of one elementwise kernel that reads and writes 256 MiB
    each: the known-size reference for the HBM byte counters."""
    n = 64 << 20
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"kernel": "elementwise mul by 1.0 (fp32)", "read_bytes": 4 * n,
                                           "write_bytes": 4 * n, "launches": 5}}), flush=True)


# ---------------------------------------------------------------------------
# Profile summaries (rocprofv3 outputs -> profiles/)
# ---------------------------------------------------------------------------
PROFILES = os.path.join(ROOT, "profiles")
# $OUT is the directory later given to --summarize-profiles
PROFILE_CMDS = {
    "trace": "BENCH_PHASE_LOG=$OUT/kt/phases.json rocprofv3 --kernel-trace --stats -f csv -d $OUT/kt "
             "-o run -- python3 bench.py",
    "pmc": "BENCH_PHASE_LOG=$OUT/pmc_{c}/phases.json rocprofv3 --pmc {c} -f csv -d $OUT/pmc_{c} -o run "
           "-- python3 bench.py --no-cpu-baseline --replays 2",
    "copy": "rocprofv3 --pmc {c} -f csv -d $OUT/pmc_copy_{c} -o run -- python3 bench.py --copy-calibration",
}
# one counter run: matrix-core busy cycles, VALU instructions and activity,
# wave cycles and waits, LDS bank conflicts (7 SQ counters + 1 GRBM)
CORE_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_WAVE_CYCLES SQ_WAIT_INST_ANY "
                 "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE GRBM_GUI_ACTIVE")
PROFILE_CMDS["core"] = ("BENCH_PHASE_LOG=$OUT/pmc_core/phases.json rocprofv3 --pmc " + CORE_COUNTERS +
                        " -f csv -d $OUT/pmc_core -o run -- python3 bench.py --no-cpu-baseline --replays 2")
KERNEL_SOURCES = ["quantize.hip", "gemm_int.hip", "gemm_wide.hip", "branch.hip", "epilogue.h", "device_common.h",
                  "lds_dma.h", "project_body.h"]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha1()
    for f in KERNEL_SOURCES:
        p = os.path.join(ROOT, "w4a4_post_quantized_channel_amd", "csrc", f)
        if os.path.exists(p):
            with open(p, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def _csv_rows(path):
    import csv
    with open(path) as fh:
        return list(csv.DictReader(fh))


def _is_marker(name):
    n = name.lower()
    return "spin" in n or "sleep" in n


def _phases_of(rows, phases, key):
    """Group dispatch rows (sorted in dispatch order) by the phase the marker
    kernels delimit: {phase name: {kernel name: [values]}}."""
    import re
    out, nmark = {}, 0
    for r in rows:
        name = r["Kernel_Name"]
        if _is_marker(name):
            nmark += 1
            continue
        cur = (nmark - 1) // 2 if nmark % 2 == 1 else -1    # inside start ... end of phase cur
        if 0 <= cur < len(phases):
            k = re.sub(r"\(.*", "", name)
            out.setdefault(phases[cur], {}).setdefault(k, []).append(key(r))
    return out


def _load_phases(d):
    with open(os.path.join(d, "phases.json")) as fh:
        return json.load(fh)


def _trace_rows(d, kind):
    import glob
    f = glob.glob(os.path.join(d, "**", f"run_{kind}.csv"), recursive=True)
    rows = _csv_rows(f[0])
    idk = "Dispatch_Id" if "Dispatch_Id" in rows[0] else "Correlation_Id"
    rows.sort(key=lambda r: int(r[idk]))
    return rows


def summarize_profiles(d):
    """profiles/bench_kernels.txt: per phase (workload, warm/cold, kernel) the
    kernel-trace median / mean duration of every kernel; with the counter
    runs, FETCH_SIZE / WRITE_SIZE per dispatch scaled by the copy
    calibration, and matrix-core busy fractions.  profiles/phase_kernels.json
    holds the same numbers for bench.py to quote."""
    os.makedirs(PROFILES, exist_ok=True)
    kt = os.path.join(d, "kt")
    phases = _load_phases(kt)
    rows = _trace_rows(kt, "kernel_trace")
    dur = _phases_of(rows, phases, lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    rec = {"source_hash": kernel_source_hash(), "command": PROFILE_CMDS["trace"], "phases": {}}
    lines = ["rocprofv3 kernel trace of the default benchmark run, split into its timed phases by the marker",
             "kernel bench.py launches before each phase (median and mean over every dispatch of the phase).",
             "command: " + PROFILE_CMDS["trace"], ""]
    factor = None
    pmc = {}
    if all(os.path.exists(os.path.join(d, f"pmc_copy_{c}")) for c in ("FETCH_SIZE", "WRITE_SIZE")):
        factor = {}
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            crow = [r for r in _trace_rows(os.path.join(d, f"pmc_copy_{c}"), "counter_collection")
                    if "MulFunctor" in r["Kernel_Name"]]
            kib = sum(float(r["Counter_Value"]) for r in crow) / len(crow)
            factor[c] = (256 * 1024) / kib
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            pd = os.path.join(d, f"pmc_{c}")
            if os.path.exists(pd):
                prow = [r for r in _trace_rows(pd, "counter_collection") if r.get("Counter_Name", c) == c]
                pmc[c] = _phases_of(prow, _load_phases(pd), lambda r: float(r["Counter_Value"]) * 1024 * factor[c])
        rec["copy_scale"] = factor
        rec["pmc_commands"] = [PROFILE_CMDS["pmc"].format(c=c) for c in ("FETCH_SIZE", "WRITE_SIZE")] + \
                              [PROFILE_CMDS["copy"].format(c=c) for c in ("FETCH_SIZE", "WRITE_SIZE")]
    core = {}
    cd = os.path.join(d, "pmc_core")
    if os.path.exists(cd):
        crow = _trace_rows(cd, "counter_collection")
        agent = [r for r in _csv_rows(os.path.join(cd, [f for f in os.listdir(cd) if f.endswith("agent_info.csv")][0]))
                 if int(r.get("Simd_Count") or 0) > 0][0]
        simds = int(agent["Simd_Count"])
        for cn in CORE_COUNTERS.split():
            rows_c = [r for r in crow if r["Counter_Name"] == cn]   # marker dispatches carry every counter too
            core[cn] = _phases_of(rows_c, _load_phases(cd), lambda r: float(r["Counter_Value"]))
        core["_dur"] = _phases_of([r for r in crow if r["Counter_Name"] == "GRBM_GUI_ACTIVE"], _load_phases(cd),
                                  lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        rec["core_command"] = PROFILE_CMDS["core"]
        rec["simds"] = simds
    for ph in phases:
        ks = dur.get(ph, {})
        if not ks:
            continue
        lines.append(f"[{ph}]")
        for k, v in sorted(ks.items(), key=lambda kv: -sum(kv[1])):
            e = {"n": len(v), "median_us": pct(v, 0.5), "mean_us": sum(v) / len(v)}
            extra = ""
            for c in ("FETCH_SIZE", "WRITE_SIZE"):
                pv = pmc.get(c, {}).get(ph, {}).get(k)
                if pv:
                    e[c.lower() + "_bytes"] = sum(pv) / len(pv)
                    extra += f"  {c} {e[c.lower() + '_bytes'] / 1e6:.2f} MB"
            if core and core.get("SQ_INSTS_VALU", {}).get(ph, {}).get(k):
                mean = lambda cn: sum(core[cn][ph][k]) / len(core[cn][ph][k])
                us_c = mean("_dur")
                e["mfma_busy"] = mean("SQ_VALU_MFMA_BUSY_CYCLES") / rec["simds"] / (us_c * 1e3 * PEAK_CLOCK_GHZ)
                e["valu_insts"] = mean("SQ_INSTS_VALU")
                e["valu_active_per_wave_cycle"] = mean("SQ_ACTIVE_INST_VALU") / max(1.0, mean("SQ_WAVE_CYCLES"))
                e["wait_per_wave_cycle"] = mean("SQ_WAIT_INST_ANY") / max(1.0, mean("SQ_WAVE_CYCLES"))
                e["lds_bank_conflict_frac"] = mean("SQ_LDS_BANK_CONFLICT") / max(1.0, mean("SQ_LDS_IDX_ACTIVE"))
                e["us_under_counters"] = us_c
                extra += (f"\n      MFMA busy {e['mfma_busy']:.1%}  VALU insts {e['valu_insts']:.3g}  "
                          f"VALU-active/wave-cycle {e['valu_active_per_wave_cycle']:.2f}  "
                          f"wait/wave-cycle {e['wait_per_wave_cycle']:.2f}  "
                          f"LDS conflict/active {e['lds_bank_conflict_frac']:.3f}  ({us_c:.2f} us under counters)")
            rec["phases"].setdefault(ph, {})[k] = e
            lines.append(f"  {k[:78]:78s} n={len(v):5d} median {e['median_us']:9.2f} us  mean {e['mean_us']:9.2f} us"
                         + extra)
        lines.append("")
    if core:
        lines.append("core counters (SIMDs " + str(rec["simds"]) + "; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / SIMDs over "
                     "the dispatch's duration at " + str(PEAK_CLOCK_GHZ) + " GHz): " + PROFILE_CMDS["core"])
    if factor:
        lines.append(f"byte counters scaled by the copy calibration: FETCH_SIZE x {factor['FETCH_SIZE']:.4f}, "
                     f"WRITE_SIZE x {factor['WRITE_SIZE']:.4f} (256 MiB read + 256 MiB written per launch)")
        for c in rec["pmc_commands"]:
            lines.append("  " + c)
    with open(os.path.join(PROFILES, "bench_kernels.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    with open(os.path.join(PROFILES, "phase_kernels.json"), "w") as fh:
        json.dump(rec, fh, indent=1)
    print(f"wrote {len(rec['phases'])} phases into {PROFILES}")


def profile_view(phase, kernel_prefix):
    """The committed profile's median for a kernel in a phase, or None when the
    kernel sources changed since the profile was taken."""
    try:
        with open(os.path.join(PROFILES, "phase_kernels.json")) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    ks = rec.get("phases", {}).get(phase, {})
    # trace names carry the full signature ("void w4a4::name<...>")
    hits = [(k, v) for k, v in ks.items() if kernel_prefix in k]
    if not hits:
        return None
    k, v = max(hits, key=lambda kv: kv[1]["median_us"])
    return {"kernel": k, **v}


GEMM_KERNELS = ("gemm_int_decode_kernel", "gemm_wide_kernel", "gemm_nvfp4_cb_kernel")


# ---------------------------------------------------------------------------
def main():
    a = parse()
    if a.summarize_profiles:
        summarize_profiles(a.summarize_profiles)
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported (every box here has one GPU)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if a.copy_calibration:
        copy_calibration(torch)
        return
    t_start = time.perf_counter()
    if a.workload:
        names = EXTRA[a.workload][0] if a.workload in EXTRA else [dict((c[0], c[1]) for c in CONFIGS)[a.workload]]
        res = []
        for n in names:
            case, layer, r = measure_case(torch, f"{a.workload}:{n}" if a.workload in EXTRA else a.workload, n,
                                          a.replays)
            res.append(summarize_case(case, layer, r))
        finish({"workload": a.workload, "configs": res}, t_start)
        return

    built, warm, flops = measure_headline(torch, HEADLINE[1], a.steps, a.replays)
    print("[bench] headline step measured", file=sys.stderr, flush=True)
    ms = warm["median"] * 1e-3
    # the headline's dominant kernel: the W8A8 down projection's GEMM (the larger projection)
    c2b = next(b for b in built if b[0].name == "decode_w8a8")
    _, _, r2b = measure_case(torch, "C2b", "decode_w8a8", a.replays, built=c2b)
    s2b = summarize_case(c2b[0], c2b[1], r2b)
    s2b["vendor_gemm"] = vendor_gemm(torch, c2b[0])
    configs = [s2b]
    if not a.no_configs:
        cached = {b[0].name: b for b in built}
        for cid, name, _ in CONFIGS:
            if cid == "C2b":
                continue
            case, layer, r = measure_case(torch, cid, name, a.replays, cold=(cid != "C1"), built=cached.get(name))
            print(f"[bench] {cid} measured", file=sys.stderr, flush=True)
            sc = summarize_case(case, layer, r)
            sc["vendor_gemm"] = vendor_gemm(torch, case)
            configs.append(sc)
            del layer
            torch.cuda.empty_cache()
        order = [c[0] for c in CONFIGS]
        configs.sort(key=lambda c: order.index(c["id"]))
    nexts = []
    if not a.no_configs and not a.no_next:
        for cid, name, what in NEXT:
            case, layer, r = measure_case(torch, cid, name, a.replays)
            print(f"[bench] {cid} measured", file=sys.stderr, flush=True)
            sc = summarize_case(case, layer, r)
            sc["row"] = what
            sc["vendor_gemm"] = vendor_gemm(torch, case)
            nexts.append(sc)
            del layer
            torch.cuda.empty_cache()
    ceil = ceilings(torch)
    g_cold = s2b["cold"]["kernels"]["gemm"]
    g_warm = s2b["warm"]["kernels"]["gemm"]
    roof = {k: g_cold[k] for k in ("bound", "achieved", "peak", "unit", "frac")}
    roof.update({"kernel": "w8a8_linear int8 64x2048x8192 (gemm_int_decode_kernel)",
                 "timing": "cold: graph replays rotating over independent input sets beyond the last-level cache",
                 "us": g_cold["us"]["median"], "algorithmic_bytes": g_cold["algorithmic_bytes"],
                 "frac_of_measured_copy": g_cold["achieved"] / ceil["copy_GBs"],
                 "warm": {"us": g_warm["us"]["median"], "achieved": g_warm["achieved"], "frac": g_warm["frac"]}})
    prof = profile_view("C2b cold gemm", "gemm_int_decode_kernel")
    roof["traffic"] = None
    if prof:
        roof["profile"] = {"median_us": prof["median_us"], "mean_us": prof["mean_us"],
                           "frac": g_cold["algorithmic_bytes"] / (prof["median_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS,
                           "source": "profiles/bench_kernels.txt [C2b cold gemm]"}
        if "fetch_size_bytes" in prof and "write_size_bytes" in prof:
            roof["traffic"] = prof["fetch_size_bytes"] + prof["write_size_bytes"]
    out = {
        "metric": METRIC,
        "value": flops / (ms * 1e-3) / 1e12,
        "unit": "TOPS",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": ms,
        "us_per_call": {"median": warm["median"], "p10": warm["p10"], "p90": warm["p90"]},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic (seeded; shapes and outlier statistics of the workload descriptions)",
        "config": {"workload": HEADLINE[2], "projections": HEADLINE[1],
                   "launch": f"HIP graph of {min(a.steps, 200)} steps, replayed {a.replays} times; median"},
        "roofline": roof,
        "configs": configs,
        "next": nexts,
        "ceilings": ceil,
    }
    if not a.no_cpu_baseline:
        cb, host, allc = cpu_baseline([(c[0], c[1]) for c in CONFIGS])
        step_us = {leg: cb["C2a"][leg]["us_per_call"] + cb["C2b"][leg]["us_per_call"] for leg in ("single", "all")}
        out["cpu_baseline"] = {
            "value": flops / (step_us["all"] * 1e-6) / 1e12, "unit": "TOPS", "cores": allc, "kind": "oracle",
            "sample": "the oracle (NumPy, BLAS products) on the first 32 and 64 rows of each workload's call "
                      "(quantize, GEMM, epilogue, branch; weights quantized beforehand), median of repeated "
                      "runs, fitted as fixed + per-row cost at the full row count; value = the batch-1 step "
                      "with BLAS on all cores of the CPU share",
            "single_thread_value": flops / (step_us["single"] * 1e-6) / 1e12,
            "host_cores": host, "cpu_model": cpu_model(), "configs": cb}
    finish(out, t_start)


def finish(out, t_start):
    out["wall_s"] = time.perf_counter() - t_start
    out["profile_phases"] = PHASE_LOG
    log = os.environ.get("BENCH_PHASE_LOG")
    if log:
        os.makedirs(os.path.dirname(log) or ".", exist_ok=True)
        with open(log, "w") as fh:
            json.dump(PHASE_LOG, fh)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
