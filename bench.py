#!/usr/bin/env python3
"""Benchmark of the quantized-linear hot path on one MI355X.

A step is one pass of the whole per-call path over one batch of synthetic
input, with inputs resident in HBM: ``quantize_act`` (smoothing, FWHT-64,
per-token quantization) then the GEMM with its dequant epilogue and, where
the workload has one, the fused 16-bit branch.  Weight packing is offline
and outside the timed region.

Default workload: the batch-1, 64-token action-expert step (a W4A4
projection 64x2048x2048 and a W8A8 down projection 64x2048x8192).  The
4096-token NVFP4 video-latent projection (4096x5120x5120 with 64 kept
bf16 channels) is measured in the same run and reported under "also".

Metric: effective TOPS = 2*M*N*K (summed over the step's projections) / time.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
PEAK_CLOCK_GHZ = 2.4           # MI355X peak engine clock
PEAK_TFLOPS = {"i8": 5000.0, "fp8": 5000.0, "f16": 2500.0, "bf16": 2500.0, "fp4": 10100.0}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="batch1", choices=["batch1", "video4096", "prefill", "lowrank", "tiny", "batch1_a8", "video4096_a8",
                                                      "batch1_fp8", "video4096_fp8"])
    p.add_argument("--no-also", action="store_true", help="skip the secondary 4096-token measurement")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU-oracle sample duration")
    p.add_argument("--eager", action="store_true", help="launch every call from Python (no HIP graph)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain elementwise copy of 256 MiB five times (hardware-counter scale)")
    p.add_argument("--summarize-profiles", metavar="DIR",
                   help="turn rocprofv3 outputs under DIR (kt_<workload>, pmc_<workload>_<counter>, "
                        "pmc_copy_<counter>) into the text summaries under profiles/ and exit (no GPU)")
    return p.parse_args()


def build_step(names, torch):
    from w4a4_post_quantized_channel_amd import pipeline, workloads as WL
    layers = []
    for n in names:
        case = WL.workload(n)
        layer, t = pipeline.build_layer(case, device="cuda")
        layer.buffers(case.M, t["x"].device)
        layers.append((case, layer, t))
    torch.cuda.synchronize()

    def step():
        for case, layer, t in layers:
            layer.forward(t["x"])
    return layers, step


def gemm_bytes(case):
    """Algorithmic HBM bytes of one GEMM launch: packed weight and activation
    codes, their scales, the output and the branch operands."""
    M, N, K = case.M, case.N, case.K
    code_a = {"int4": 0.5, "int8": 1.0, "nvfp4": 0.5, "w4a8": 1.0, "fp8": 1.0}[case.fmt]
    code_w = {"int4": 0.5, "int8": 1.0, "nvfp4": 0.5, "w4a8": 0.5, "fp8": 1.0}[case.fmt]
    if case.fmt == "nvfp4":
        scales = (M + N) * K / 16
    else:
        scales = 4 * (M + N)
    out = M * N * (4 if case.y_dtype == "f32" else 2)
    br = 0
    if case.branch is not None:
        r = case.branch["lw"].shape[1]
        ra = 2 * r if case.branch["kind"] == "lowrank" else r
        br = 2 * (M * ra + N * r)
    return code_a * M * K + code_w * N * K + scales + out + br


EAGER = False
PER_GRAPH = 20


def time_region(torch, step, steps, warmup):
    """ms per call of ``step``.  Default: the calls are captured once into a
    HIP graph of PER_GRAPH back-to-back calls and the graph is replayed, so
    host launch cost is not what is measured; HIP events on the replay
    stream bracket the timed replays.  With --eager every call is launched
    from Python."""
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    if EAGER:
        run, per = step, 1
    else:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(PER_GRAPH):
                step()
        run, per = graph.replay, PER_GRAPH
    reps = max(1, steps // per)
    for _ in range(max(1, warmup // per)):
        run()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        run()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / (reps * per)


def dominant_kernel_time(torch, case, layer, t, steps):
    """Average duration of the GEMM launch alone, HIP events on the launch stream."""
    b = layer.buffers(case.M, t["x"].device)
    layer.forward(t["x"])
    from w4a4_post_quantized_channel_amd import ops
    br = None
    if layer.branch is not None:
        br = ops.branch_desc(layer.branch_operand(case.M, t["x"].device), layer.branch["lw"])

    def gemm():
        if case.fmt in ("int8", "w4a8", "fp8"):
            fn = {"int8": ops.w8a8_linear, "w4a8": ops.w4a8_linear, "fp8": ops.fp8_linear}[case.fmt]
            fn(b["codes"], b["scales"], layer.w_codes, layer.w_scales, case.K, branch=br,
               y=b["y"], workspace=b["ws"])
        else:
            ops.w4a4_linear(b["codes"], b["scales"], layer.w_codes, layer.w_scales, case.K, case.fmt,
                            alpha=layer.alpha, branch=br, y=b["y"], workspace=b["ws"])
    return time_region(torch, gemm, steps, max(5, steps // 10))


def quant_kernel_time(torch, case, layer, t, steps):
    from w4a4_post_quantized_channel_amd import ops
    b = layer.buffers(case.M, t["x"].device)

    def q():
        ops.quantize_act(t["x"], layer.inv_s, layer.a_fmt, fwht_block=layer.fwht_block, order=layer.order,
                         tensor_scale=layer.g_a, codes=b["codes"], scales=b["scales"])
    return time_region(torch, q, steps, max(5, steps // 10))


def cpu_baseline(names, target_s):
    """The oracle as it stands, on the host cores: per-call path (activation
    transform + quantization, GEMM, epilogue, branch) with weights packed
    beforehand, repeated until about ``target_s`` seconds of CPU work."""
    import numpy as np
    from oracle import w4a4_oracle as O
    from w4a4_post_quantized_channel_amd import workloads as WL
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    prepared = []
    for n in names:
        c = WL.workload(n)
        W = O.quantize_operand(c.w, c.s, O.OPERAND_FORMATS[c.fmt][1])
        g_a = None
        if c.fmt == "nvfp4":
            g_a = O.nvfp4_tensor_scale(O.transformed_amax(c.x, c.inv_s))
        prepared.append((c, W, g_a))

    def one_call(c, W, g_a):
        A = O.quantize_operand(c.x, c.inv_s, O.OPERAND_FORMATS[c.fmt][0], g=g_a)
        if c.fmt in ("int4", "int8", "w4a8"):
            y = O.dequant_epilogue(O.int_gemm(A["codes"], W["codes"]), A["scales"], W["scales"])
        elif c.fmt == "fp8":
            y = O.dequant_epilogue(O.fp8_gemm(A["codes"], W["codes"]), A["scales"], W["scales"])
        else:
            y = O.dequantize_nvfp4(A["codes"], A["scales"], A["g"]) @ O.dequantize_nvfp4(
                W["codes"], W["scales"], W["g"]).T
        if c.branch is not None:
            if c.branch["kind"] == "lowrank":
                y = y + O.lowrank_branch(c.x, c.branch["l1"], c.branch["lw"])
            else:
                y = y + O.outlier_branch(c.x, c.branch["idx"], c.branch["lw"])
        return y

    ops_per = sum(2.0 * c.M * c.N * c.K for c, _, _ in prepared)
    t0 = time.perf_counter()
    reps = 0
    while True:
        for c, W, g_a in prepared:
            one_call(c, W, g_a)
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or reps >= 1000:
            break
    return {"value": ops_per * reps / el / 1e12, "unit": "TOPS", "cores": int(cores), "kind": "oracle",
            "sample": f"{reps} repetitions of the full step ({', '.join(names)}), "
                      f"{el:.1f} s, weights packed beforehand",
            "ms_per_step": el / reps * 1e3}


WORKLOADS = {
    "batch1": (["decode_w4a4", "decode_w8a8"],
               "batch-1 64-token action-expert step: W4A4 64x2048x2048 + W8A8 64x2048x8192, "
               "smoothing + FWHT-64 + per-token quantization"),
    "video4096": (["video_nvfp4"], "4096-token video-latent projection, NVFP4 W4A4 4096x5120x5120 "
                                   "+ 64 kept bf16 channels"),
    "prefill": (["prefill_gate_up", "prefill_down"], "512-token backbone prefill: gate/up W4A4 "
                                                     "512x16384x2048 + down W4A4 512x2048x8192"),
    "lowrank": (["lowrank"], "1024-token low-rank-protected W4A4 1024x3072x3072 + rank-32 bf16 branch"),
    "tiny": (["tiny"], "tiny W4A4 16x256x256 (fp32 in/out)"),
    "batch1_a8": (["decode_w4a8", "decode_w4a8_down"],
                  "batch-1 64-token action step at 8-bit activations (protected denoising step): "
                  "W4A8 64x2048x2048 + W4A8 64x2048x8192, smoothing + FWHT-64 + per-token int8"),
    "video4096_a8": (["video_w4a8"], "4096-token video-latent projection at 8-bit activations "
                                     "(protected denoising step), W4A8 4096x5120x5120 + 64 kept bf16 channels"),
    "batch1_fp8": (["decode_w4a4", "decode_fp8"],
                   "batch-1 64-token action-expert step with the upgraded projection in FP8: W4A4 64x2048x2048 "
                   "+ FP8 (E4M3) W8A8 64x2048x8192"),
    "video4096_fp8": (["video_fp8"], "4096-token video-latent projection upgraded to FP8 (E4M3) W8A8 "
                                     "4096x5120x5120 + 64 kept bf16 channels"),
}


def measure(torch, wl, steps, warmup):
    names, desc = WORKLOADS[wl]
    layers, step = build_step(names, torch)
    ms = time_region(torch, step, steps, warmup)
    flops = sum(2.0 * c.M * c.N * c.K for c, _, _ in layers)
    # dominant kernel = the GEMM of the largest projection
    c, layer, t = max(layers, key=lambda e: e[0].M * e[0].N * e[0].K)
    ksteps = max(20, steps)
    k_ms = dominant_kernel_time(torch, c, layer, t, ksteps)
    q_ms = quant_kernel_time(torch, c, layer, t, ksteps)
    flop_k = 2.0 * c.M * c.N * c.K
    bytes_k = gemm_bytes(c)
    mtype = {"int4": "i8", "int8": "i8", "nvfp4": "f16", "w4a8": "i8", "fp8": "fp8"}[c.fmt]
    intensity = flop_k / bytes_k
    ridge = PEAK_TFLOPS[mtype] * 1e12 / (HBM_PEAK_GBS * 1e9)
    if intensity < ridge:
        roof = {"bound": "hbm", "achieved": bytes_k / (k_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": flop_k / (k_ms * 1e-3) / 1e12, "peak": PEAK_TFLOPS[mtype],
                "unit": "TFLOP/s" if mtype != "i8" else "TOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = recorded_traffic(wl)
    entry = {"int8": "w8a8_linear", "w4a8": "w4a8_linear", "fp8": "fp8_linear"}.get(c.fmt, "w4a4_linear")
    roof["kernel"] = f"{entry} {c.fmt} {c.M}x{c.N}x{c.K}"
    roof["kernel_us"] = k_ms * 1e3
    roof["algorithmic_bytes"] = bytes_k
    qbytes = c.M * c.K * (2 if c.x_dtype == "bf16" else 4) + c.M * c.K * (1 if c.fmt in ("int8", "w4a8", "fp8") else 0.5) + (
        c.M * c.K / 16 if c.fmt == "nvfp4" else 4 * c.M)
    quant = {"kernel": f"quantize_act {layer.a_fmt} {c.M}x{c.K}", "us": q_ms * 1e3,
             "achieved_GBs": qbytes / (q_ms * 1e-3) / 1e9, "frac_hbm": qbytes / (q_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    return {"names": names, "desc": desc, "ms": ms, "flops": flops, "roofline": roof, "quantize": quant,
            "per_call_us": {n: None for n in names}}


def copy_calibration(torch):
    """Five launches of one elementwise kernel that reads and writes 256 MiB
    each: the known-size reference for the HBM byte counters."""
    n = 64 << 20                     # fp32 elements = 256 MiB
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"kernel": "elementwise mul by 1.0 (fp32)", "read_bytes": 4 * n,
                                           "write_bytes": 4 * n, "launches": 5}}), flush=True)



# ---------------------------------------------------------------------------
# Profile summaries (rocprofv3 outputs -> profiles/*.txt, profiles/traffic.json)
# ---------------------------------------------------------------------------
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["quantize.hip", "gemm_int.hip", "gemm_wide.hip", "branch.hip", "epilogue.h", "device_common.h"]

# The dominant call of each workload: the kernels one linear call launches.
DOMINANT = {
    "batch1": ("w8a8_linear int8 64x2048x8192", ["gemm_int_decode_kernel<1, 2, 1>"]),
    "batch1_a8": ("w4a8_linear w4a8 64x2048x8192", ["gemm_int_decode_kernel<2, 2, 1>"]),
    "video4096_a8": ("w4a8_linear w4a8 4096x5120x5120", ["gemm_wide_kernel<3,"]),
    "batch1_fp8": ("fp8_linear fp8 64x2048x8192", ["gemm_int_decode_kernel<3, 2, 1>"]),
    "video4096_fp8": ("fp8_linear fp8 4096x5120x5120", ["gemm_wide_kernel<4,"]),
    "video4096": ("w4a4_linear nvfp4 4096x5120x5120", ["gemm_nvfp4_cb_kernel"]),
    "prefill": ("w4a4_linear int4 512x16384x2048", ["gemm_wide_kernel<0, 4, 4, 2, 4, 1>"]),
    "lowrank": ("w4a4_linear int4 1024x3072x3072", ["gemm_wide_kernel<0, 2, 6, 4, 1, 2>"]),
}

PROFILE_CMDS = {
    "trace": "rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/kt_{w} -o run -- "
             "python3 bench.py --workload {w} --steps 100 --warmup 10 --no-cpu-baseline --no-also",
    "pmc": "rocprofv3 --pmc {c} -f csv -d gpurun_out/pmc_{w}_{c} -o run -- "
           "python3 bench.py --workload {w} --steps 5 --warmup 1 --eager --no-cpu-baseline --no-also",
    "copy": "rocprofv3 --pmc {c} -f csv -d gpurun_out/pmc_copy_{c} -o run -- python3 bench.py --copy-calibration",
    "group": "rocprofv3 --pmc {c} -f csv -d gpurun_out/pmc_{w}_{g} -o run -- "
             "python3 bench.py --workload {w} --steps 5 --warmup 1 --eager --no-cpu-baseline --no-also",
}

# Counter groups for the matrix-core view of the many-token calls, one run
# each: MFMA busy cycles (summed over SIMDs) against elapsed cycles (summed
# over XCDs), and the MFMA work in units of 512 operations.
COUNTER_GROUPS = {
    "MFMA": "SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE",
    "MOPS": "SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_INSTS_VALU_MFMA_MOPS_I8 SQ_INSTS_VALU_MFMA_MOPS_F8 "
            "SQ_INSTS_VALU_MFMA_MOPS_F6F4",
}
MFMA_WORKLOADS = ["video4096", "video4096_a8", "video4096_fp8", "prefill", "lowrank"]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha1()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "w4a4_post_quantized_channel_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(wl):
    """HBM bytes per dominant call from the committed counter summary, or
    None when there is none or the kernel sources changed since."""
    try:
        with open(os.path.join(PROFILES, "traffic.json")) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    e = rec.get("workloads", {}).get(wl)
    if not e or rec.get("source_hash") != kernel_source_hash():
        return None
    return {"fetch_bytes": e["fetch_bytes"], "write_bytes": e["write_bytes"],
            "total_bytes": e["fetch_bytes"] + e["write_bytes"]}


def _csv_rows(path):
    import csv
    with open(path) as fh:
        return list(csv.DictReader(fh))


def _quantizer_traffic(d, wl, stats, factor):
    """HBM bytes and average duration of each quantize kernel that runs every
    step (the activation quantizers; weight packing runs once)."""
    import re
    per = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        f = os.path.join(d, f"pmc_{wl}_{c}", "run_counter_collection.csv")
        if not os.path.exists(f):
            return None
        vals = {}
        for r in _csv_rows(f):
            if "quant" in r["Kernel_Name"]:
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        per[c] = {k: sum(v) / len(v) * factor[c] * 1024.0 for k, v in vals.items() if len(v) >= 5}
    out = {}
    for name in sorted(set(per["FETCH_SIZE"]) & set(per["WRITE_SIZE"])):
        us = [float(r["AverageNs"]) / 1e3 for r in stats if r["Name"] == name]
        if us:
            out[re.sub(r"\(.*", "", name)] = (per["FETCH_SIZE"][name], per["WRITE_SIZE"][name], us[0])
    return out


def _mfma_counters(d, wl, kernels):
    """Matrix-core busy fraction and MFMA work of the dominant call."""
    base = {g: os.path.join(d, f"pmc_{wl}_{g}") for g in COUNTER_GROUPS}
    if not all(os.path.exists(os.path.join(b, "run_counter_collection.csv")) for b in base.values()):
        return None
    agent = [r for r in _csv_rows(os.path.join(base["MFMA"], "run_agent_info.csv"))
             if int(r.get("Simd_Count") or 0) > 0][0]
    simds, xcc = int(agent["Simd_Count"]), int(agent["Num_Xcc"])

    def mean(g, counter):
        rows = [r for r in _csv_rows(os.path.join(base[g], "run_counter_collection.csv"))
                if r["Counter_Name"] == counter and any(k in r["Kernel_Name"] for k in kernels)]
        if not rows:
            return None, 0, 0.0
        dur = sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows) / len(rows)
        return sum(float(r["Counter_Value"]) for r in rows) / len(rows), len(rows), dur

    busy, calls, dur_ns = mean("MFMA", "SQ_VALU_MFMA_BUSY_CYCLES")
    active, _, _ = mean("MFMA", "GRBM_GUI_ACTIVE")
    if busy is None or not dur_ns:
        return None
    mops = sum(mean("MOPS", c)[0] or 0.0 for c in COUNTER_GROUPS["MOPS"].split())
    busy = busy / simds
    # GRBM_GUI_ACTIVE also counts dispatch set-up around short calls, so the
    # busy fraction is taken over the call's own duration at the peak clock
    return {"calls": calls, "us": dur_ns / 1e3, "busy": busy, "grbm_active_per_xcd": (active or 0.0) / xcc,
            "util": busy / (dur_ns * PEAK_CLOCK_GHZ), "gflop": mops * 512 / 1e9}


def summarize_profiles(d):
    """Write profiles/<kernel>_<workload>.txt (kernel-trace statistics) and
    profiles/traffic.json (FETCH_SIZE / WRITE_SIZE per dominant call and per
    step quantizer, scaled by the same counters read on a plain copy of known
    size; matrix-core busy fraction and MFMA work of the many-token calls)."""
    import re
    os.makedirs(PROFILES, exist_ok=True)
    factor = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        rows = [r for r in _csv_rows(os.path.join(d, f"pmc_copy_{c}", "run_counter_collection.csv"))
                if "MulFunctor" in r["Kernel_Name"]]
        kib = sum(float(r["Counter_Value"]) for r in rows) / len(rows)
        factor[c] = (256 * 1024) / kib          # known KiB per launch / counter KiB
    traffic = {"source_hash": kernel_source_hash(), "copy_scale": factor,
               "commands": {k: v for k, v in PROFILE_CMDS.items()}, "workloads": {}}
    for wl, (label, kernels) in DOMINANT.items():
        kt = os.path.join(d, f"kt_{wl}", "run_kernel_stats.csv")
        if not os.path.exists(kt):
            continue
        stats = _csv_rows(kt)
        lines = [f"rocprofv3 kernel-trace statistics, workload {wl} ({WORKLOADS[wl][1]})",
                 "command: " + PROFILE_CMDS["trace"].format(w=wl), "",
                 f"{'kernel':72s} {'calls':>6s} {'avg us':>9s} {'min us':>9s} {'max us':>9s}"]
        for r in stats:
            name = re.sub(r"\(.*", "", r["Name"])[:72]
            lines.append(f"{name:72s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} "
                         f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f}")
        dom_us = sum(float(r["AverageNs"]) / 1e3 for r in stats if any(k in r["Name"] for k in kernels))
        lines += ["", f"dominant call: {label} = {' + '.join(kernels)}; sum of average durations {dom_us:.2f} us"]
        per = {}
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            f = os.path.join(d, f"pmc_{wl}_{c}", "run_counter_collection.csv")
            if not os.path.exists(f):
                continue
            tot, found = 0.0, True
            for k in kernels:
                vals = [float(r["Counter_Value"]) for r in _csv_rows(f) if k in r["Kernel_Name"]]
                if not vals:
                    found = False
                    break
                tot += sum(vals) / len(vals)
            if not found:
                continue
            per[c] = tot * factor[c] * 1024.0
            lines.append(f"{c}: {tot:.1f} KiB per call (counter) x {factor[c]:.4f} (copy scale) = "
                         f"{per[c] / 1e6:.3f} MB   [" + PROFILE_CMDS["pmc"].format(w=wl, c=c) + "]")
        if len(per) == 2:
            traffic["workloads"][wl] = {"call": label, "fetch_bytes": per["FETCH_SIZE"],
                                        "write_bytes": per["WRITE_SIZE"], "avg_us": dom_us}
        q = _quantizer_traffic(d, wl, stats, factor)
        if q:
            lines += ["", "per-step quantize kernels (HBM bytes from the same FETCH_SIZE / WRITE_SIZE runs, "
                      "over the kernel-trace average):"]
            for name, (fb, wb, us) in q.items():
                lines.append(f"  {name}: {fb / 1e6:.2f} MB fetched + {wb / 1e6:.2f} MB written in {us:.2f} us = "
                             f"{(fb + wb) / us / 1e3:.0f} GB/s ({(fb + wb) / us / 1e3 / HBM_PEAK_GBS:.1%} of HBM peak)")
            traffic.setdefault("quantize", {})[wl] = {n: {"fetch_bytes": fb, "write_bytes": wb, "avg_us": us}
                                                      for n, (fb, wb, us) in q.items()}
        m = _mfma_counters(d, wl, kernels) if wl in MFMA_WORKLOADS else None
        if m:
            lines += ["", f"matrix cores ({m['calls']} calls under the counters, {m['us']:.2f} us each there):",
                      f"  SQ_VALU_MFMA_BUSY_CYCLES / SIMDs = {m['busy']:.0f} busy cycles per SIMD, "
                      f"{m['util']:.1%} of the call's {m['us'] * PEAK_CLOCK_GHZ * 1e3:.0f} cycles at "
                      f"{PEAK_CLOCK_GHZ} GHz",
                      f"  MFMA work {m['gflop']:.1f} G operations (512 per MOPS unit)",
                      "  [" + PROFILE_CMDS["group"].format(w=wl, g="MFMA", c=COUNTER_GROUPS["MFMA"]) + "]",
                      "  [" + PROFILE_CMDS["group"].format(w=wl, g="MOPS", c=COUNTER_GROUPS["MOPS"]) + "]"]
            traffic.setdefault("mfma", {})[wl] = m
        slug = re.sub(r"[^a-z0-9]+", "_", label.lower()).strip("_")
        with open(os.path.join(PROFILES, f"{slug}_{wl}.txt"), "w") as fh:
            fh.write("\n".join(lines) + "\n")
    traffic["copy_commands"] = [PROFILE_CMDS["copy"].format(c=c) for c in ("FETCH_SIZE", "WRITE_SIZE")]
    with open(os.path.join(PROFILES, "traffic.json"), "w") as fh:
        json.dump(traffic, fh, indent=1)
    print(f"wrote summaries for {sorted(traffic['workloads'])} into {PROFILES}")


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
    global EAGER
    EAGER = a.eager
    if a.copy_calibration:
        copy_calibration(torch)
        return
    r = measure(torch, a.workload, a.steps, a.warmup)
    out = {
        "metric": "W4A4 linear effective TOPS + us/call (batch-1 64-token and 4096-token shapes)",
        "value": r["flops"] / (r["ms"] * 1e-3) / 1e12,
        "unit": "TOPS",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": r["ms"],
        "us_per_call": r["ms"] * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"nvfp4": "f16", "fp8": "fp8"}.get(r["roofline"]["kernel"].split()[1], "i8"),
        "data": "synthetic (seeded; shapes and outlier statistics of the workload descriptions)",
        "config": {"workload": r["desc"], "projections": r["names"],
                   "launch": "eager" if a.eager else f"HIP graph of {PER_GRAPH} steps, replayed"},
        "roofline": r["roofline"],
        "quantize_kernel": r["quantize"],
    }
    if a.workload == "batch1" and not a.no_also:
        # five replays of the 20-step graph after two (about 30 ms): one replay
        # after one warm-up read the GPU before its clocks had settled
        v = measure(torch, "video4096", max(100, a.steps // 2), max(40, a.warmup))
        out["also"] = {"workload": v["desc"], "value": v["flops"] / (v["ms"] * 1e-3) / 1e12, "unit": "TOPS",
                       "us_per_call": v["ms"] * 1e3, "roofline": v["roofline"], "quantize_kernel": v["quantize"]}
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(r["names"], a.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
