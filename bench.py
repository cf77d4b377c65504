"""Benchmark of the microscaling hot path on one MI355X.

Default workload: the MXFP4 W4A4 DiT MLP-down layer, M=4608 tokens, K=12288,
N=3072, activations Laplace(0,1) with 0.5% outlier channels x100, weights
N(0,0.02) quantized beforehand. One step = quantize the bf16 activations to
MXFP4 (codes + E8M0 scales) and run the block-scaled GEMM against the
pre-quantized weights, bf16 output (operands in the K-panel layout of their
format: weights re-laid once by mx_pack, activations quantized straight into
it).
Everything in the timed region runs in libmx's HIP kernels; inputs are
resident in HBM before timing starts. After the warm-up steps the same steps
are replayed, untimed, for RAMP_S seconds: the GPU raises its clocks only
after tens of milliseconds of continuous load, and the timed steps should see
the clocks a sustained workload runs at.

Prints one JSON line. `value` is whole-step throughput, 2MNK / step time, in
TFLOP/s. The `roofline` object is for the dominant kernel (the GEMM), timed
with HIP events on its own stream; `quantize` reports the activation
quantizer's algorithmic GB/s, timed from a HIP-graph replay of quantize-only
steps; `cpu_baseline` times the oracle on the host cores (OpenMP) on a bounded
sample of the same step, and `parity` compares that sample with the GPU's
codes, scales and outputs.

Other workloads (--workload c1..c5, f1..f4, c5w) are for profiling; the
default is the one the headline metric is quoted on. c5w is a quantize-only
step (the decode weights, 470 MB of bf16), reported in GB/s.
"""
import argparse
import dataclasses
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks.
PEAK_HBM_GBPS = 8000.0
# Dense MFMA peaks (TFLOP/s). Each GEMM path is measured against the matrix
# instruction it runs on ("mfma") and against the rate of its element format
# ("format"): MXFP4 runs on the FP4 scaled MFMA (both 10.1 PF); MXFP8, E5M2 and
# E3M2 run on the exact bf16 expansion (bf16 2.5 PF; FP8 5.0, FP6 10.1);
# NVFP4 on the exact fp16 expansion (fp16 2.5 PF; FP4 10.1); W4A16 on bf16.
PEAK_MFMA = {"mxfp4": 10100.0, "mxfp8": 2500.0, "nvfp4": 2500.0, "w4a16": 2500.0,
             "mxfp8_e5m2": 2500.0, "mxfp6_e3m2": 2500.0, "mxfp4_mbs": 10100.0,
             "mxfp4_mbs16": 10100.0}
PEAK_FORMAT = {"mxfp4": 10100.0, "mxfp8": 5000.0, "nvfp4": 10100.0, "w4a16": 2500.0,
               "mxfp8_e5m2": 5000.0, "mxfp6_e3m2": 10100.0, "mxfp4_mbs": 10100.0,
               "mxfp4_mbs16": 10100.0}
MFMA_NAME = {"mxfp4": "fp4", "mxfp8": "bf16", "nvfp4": "fp16", "w4a16": "bf16",
             "mxfp8_e5m2": "bf16", "mxfp6_e3m2": "bf16", "mxfp4_mbs": "fp4", "mxfp4_mbs16": "fp4"}
FORMAT_NAME = {"mxfp4": "fp4", "mxfp8": "fp8", "nvfp4": "fp4", "w4a16": "bf16",
               "mxfp8_e5m2": "fp8", "mxfp6_e3m2": "fp6", "mxfp4_mbs": "fp4", "mxfp4_mbs16": "fp4"}
# fp32 vector lane-operations per second (one mul or one fma per lane per
# cycle, no packed math): 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz. The MBS GEMM
# is bound by its per-macro-block rescale on the vector ALU (2 operations per
# output element per 128 K), so it is measured against this.
PEAK_VALU_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
ROTATE_BYTES = 1 << 30  # activation copies cycled per step: > 256 MB MALL
RAMP_S = 0.2  # seconds of untimed replays before timing (GPU clock ramp)
# The K-panel layout per format (include/mx.h): panel width W in elements,
# code bytes and scale bytes of one row in one panel.
PANEL_GEOMETRY = {"mxfp4": (256, 128, 8), "mxfp8": (64, 64, 2), "mxfp8_e5m2": (64, 64, 2),
                  "mxfp6_e3m2": (64, 48, 2), "nvfp4": (64, 32, 4)}
WEIGHT_ROTATE_BYTES = 512 << 20  # weight copies cycled per step: > 256 MB MALL, so
                                 # every step streams its weights from HBM, as the
                                 # layers of a model would
CPU_BUDGET_MACS = 2.5e11  # bound on the oracle's CPU sample (multiply-adds)

# Algorithmic bytes per element of a quantizer: read bf16 once, write codes +
# scales (+ macro mantissas).
ELEM_BYTES = {"mxfp4": 0.5 + 1 / 32, "mxfp8": 1 + 1 / 32, "nvfp4": 0.5 + 1 / 16,
              "mxfp8_e5m2": 1 + 1 / 32, "mxfp6_e3m2": 0.75 + 1 / 32,
              "mxfp4_mbs": 0.5 + 1 / 32 + 1 / 128, "mxfp4_mbs16": 0.5 + 1 / 16 + 1 / 128}

DTYPE = {"mxfp4": "e2m1+e8m0 (fp32 accumulate)", "mxfp8": "e4m3+e8m0 via bf16 (fp32 accumulate)",
         "nvfp4": "e2m1+e4m3 via fp16 (fp32 accumulate)",
         "w4a16": "bf16 x e2m1+e8m0 (fp32 accumulate)",
         "mxfp8_e5m2": "e5m2+e8m0 via bf16 (fp32 accumulate)",
         "mxfp6_e3m2": "e3m2+e8m0 via bf16 (fp32 accumulate)",
         "mxfp4_mbs": "e2m1+e8m0/32, macro factor 1+m/256 (fp32 accumulate)",
         "mxfp4_mbs16": "e2m1+e8m0/16, macro factor 1+m/256 (fp32 accumulate)"}

METRIC = "block-scaled GEMM TFLOP/s + quantize GB/s, % of MXFP4/FP8 MFMA & HBM peak"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="c4")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--ramp-s", type=float, default=RAMP_S,
                   help="seconds of untimed replays between the warm-up and the timed steps")
    p.add_argument("--cpu-rows", type=int, default=0,
                   help="activation rows in the oracle's CPU sample (0: as many as fit "
                        f"{CPU_BUDGET_MACS:.2g} multiply-adds)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain device-to-device copy of 1 GiB, 5 times (reference "
                        "for scaling the HBM byte counters)")
    p.add_argument("--mfma-ceiling", action="store_true",
                   help="only measure what matrix instructions alone sustain on this device "
                        "(FP4 scaled, bf16, fp16; include/mx_calib.h)")
    p.add_argument("--hbm-ceiling", action="store_true",
                   help="only measure what plain 16-byte streams of loads and stores sustain "
                        "from HBM (read, write, copy, 4:1 read:write; include/mx_calib.h)")
    return p.parse_args()


def copy_calibration():
    """A plain copy of known size: each dispatch reads and writes exactly 1 GiB.
    rocprofv3's FETCH_SIZE / WRITE_SIZE for it give the scale factor applied
    to the same counters of the kernels."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_dispatch": n, "dispatches": 5}))


def mfma_ceiling():
    """The rate matrix instructions alone sustain (libmx_calib.so), on every CU
    and on the 216 CUs that the 256 x 256 tiles of the 4608 x 3072 MLP-down
    output occupy: the clock falls under a steady stream of them, so this, not
    the published peak, bounds what a GEMM can reach. About 0.2 s of launches
    per configuration: 40 launches of ~5 ms, the median of the last 20 (the
    clock settles within the first tens of milliseconds)."""
    import ctypes
    import torch
    torch.cuda.init()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    L = ctypes.CDLL(os.path.join(ROOT, "microscaling_precision_quantization_amd", "libmx_calib.so"))
    L.mx_calib_mfma.restype = ctypes.c_int
    L.mx_calib_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double)]
    res = {}
    for kind, name, peak, iters in ((0, "fp4_scaled_32x32x64", 10100.0, 15000),
                                    (1, "bf16_32x32x16", 2500.0, 15000),
                                    (2, "fp16_32x32x16", 2500.0, 15000)):
        for wgs in (cus, 216):
            ms, flop = ctypes.c_float(), ctypes.c_double()
            rc = L.mx_calib_mfma(kind, wgs, iters, 40, ctypes.byref(ms), ctypes.byref(flop))
            if rc != 0:
                raise RuntimeError(f"mx_calib_mfma({kind}) failed: {rc}")
            tf = flop.value / (ms.value * 1e-3) / 1e12
            res[f"{name}_{wgs}cu"] = {"TFLOP/s": round(tf, 1), "frac_of_peak": round(tf / peak, 4),
                                      "peak_TFLOP/s": peak, "ms_per_launch": round(ms.value, 3)}
    print(json.dumps({"mfma_ceiling": res, "cus": cus,
                      "method": "median of the last 20 of 40 back-to-back ~5 ms launches of "
                                "MFMA-only kernels on register operands with random bits "
                                "(include/mx_calib.h)"}))


def hbm_ceiling():
    """What plain streams of 16-byte loads and stores sustain from HBM
    (libmx_calib.so): 1 GiB per launch, four times the last-level cache, 20
    launches per configuration (the median of the last 10). Configurations:
    one pass over the data with 1 to 8 chunks per thread (each workgroup a
    contiguous run, as the quantizers are laid out), or a grid-stride loop
    over 1 to 8 workgroups per CU; plain or non-temporal accesses. The best
    configuration per kind is the ceiling."""
    import ctypes
    import torch
    torch.cuda.init()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    L = ctypes.CDLL(os.path.join(ROOT, "microscaling_precision_quantization_amd", "libmx_calib.so"))
    L.mx_calib_stream.restype = ctypes.c_int
    L.mx_calib_stream.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double)]
    nbytes = 1 << 30
    res = {}
    for kind, name in ((0, "read"), (1, "write"), (2, "copy"), (3, "read4_write1")):
        runs = {}
        for nt in (0, 1):
            for per_cu in (0, 1, 2, 4, 8):
                for unroll in (1, 2, 4, 8):
                    ms, moved = ctypes.c_float(), ctypes.c_double()
                    rc = L.mx_calib_stream(kind, nbytes, cus * per_cu, unroll, nt, 20, ctypes.byref(ms),
                                           ctypes.byref(moved))
                    if rc != 0:
                        raise RuntimeError(f"mx_calib_stream({kind}) failed: {rc}")
                    grid = "one_pass" if per_cu == 0 else f"{per_cu}_per_cu"
                    runs[f"{grid}_x{unroll}{'_nt' if nt else ''}"] = {
                        "GB/s": round(moved.value / (ms.value * 1e-3) / 1e9, 1), "ms_per_launch": round(ms.value, 4)}
        best = max(runs, key=lambda k: runs[k]["GB/s"])
        res[name] = {"best_GB/s": runs[best]["GB/s"], "frac_of_peak": round(runs[best]["GB/s"] / PEAK_HBM_GBPS, 4),
                     "best": best, "runs": runs}
    print(json.dumps({"hbm_ceiling": res, "cus": cus, "bytes_per_launch": nbytes, "peak_GB/s": PEAK_HBM_GBPS,
                      "method": "median of the last 10 of 20 back-to-back launches of 16-byte stream "
                                "kernels (include/mx_calib.h)"}))


def graph_ms_per_step(torch, fn, nsteps, stream, ramp_s):
    """fn(i) for i < nsteps captured once as a HIP graph; after ramp_s of
    untimed replays, five timed replays. Returns (ms per step of the first
    timed replay, the five, ramp replays, ramp seconds, graph)."""
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(nsteps):
            fn(i)
    graph.replay()
    torch.cuda.synchronize()
    t_ramp = time.perf_counter()
    ramp_replays = 0
    while time.perf_counter() - t_ramp < ramp_s:
        graph.replay()
        ramp_replays += 1
        torch.cuda.synchronize()
    ramp_s = time.perf_counter() - t_ramp
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    ms = []
    for _ in range(5):
        start.record(stream)
        graph.replay()
        end.record(stream)
        torch.cuda.synchronize()
        ms.append(start.elapsed_time(end) / nsteps)
    return ms[0], ms, ramp_replays, ramp_s, graph


def spread(ms):
    return {"min": min(ms), "median": sorted(ms)[len(ms) // 2], "max": max(ms), "n": len(ms)}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.mfma_ceiling:
        mfma_ceiling()
        return
    if args.hbm_ceiling:
        hbm_ceiling()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the kernels "
              "and their measurement cover one GPU's share; sharding over several GPUs is "
              "not implemented.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import microscaling_precision_quantization_amd as mx
    import synth

    name = synth.ALIASES.get(args.workload, args.workload)
    w = synth.WORKLOADS[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t0 = time.time()
    A_bits, B_bits = synth.workload(name)
    gen_s = time.time() - t0
    inputs = {"A": synth.digest(A_bits)}
    if B_bits is not None:
        inputs["B"] = synth.digest(B_bits)

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    if w.get("step") == "quantize":
        line = bench_quantize_only(args, name, w, A_bits, to_dev, mx, torch, np)
    else:
        line = bench_step(args, name, w, A_bits, B_bits, to_dev, mx, torch, np)
    line["inputs"] = {"digest_blake2b_64": inputs, "generated_s": round(gen_s, 2)}
    print(json.dumps(line), flush=True)


def bench_quantize_only(args, name, w, A_bits, to_dev, mx, torch, np):
    """One step = quantize the whole bf16 tensor to the workload's format (row
    layout), inputs in HBM (the tensor exceeds the last-level cache)."""
    fmt, M, K = w["fmt"], w["M"], w["K"]
    x = to_dev(A_bits)
    stream = torch.cuda.current_stream(x.device)
    for _ in range(args.warmup):
        mx.quantize(x, fmt)
    torch.cuda.synchronize()
    ms, ms_all, ramp_replays, ramp_s, _ = graph_ms_per_step(
        torch, lambda i: mx.quantize(x, fmt), args.steps, stream, args.ramp_s)
    q_bytes = M * K * (2 + ELEM_BYTES[fmt])
    gbps = q_bytes / (ms * 1e-3) / 1e9
    line = {
        "metric": METRIC, "value": gbps, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 -> " + DTYPE[fmt].split(" (")[0], "data": "synthetic",
        "config": {"workload": name, "format": fmt, "rows": M, "cols": K,
                   "step": "quantize (row layout)", "input_bytes": M * K * 2},
        "timing": {"ms_per_step": "HIP-graph replay of the timed steps",
                   "clock_ramp": f"{ramp_replays} untimed replays ({ramp_s * 1e3:.0f} ms)",
                   "replays_ms_per_step": spread(ms_all)},
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": gbps / PEAK_HBM_GBPS, "traffic": measured_traffic(name),
                     "kernel_ms": ms, "algorithmic_bytes": q_bytes},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"], line["parity"] = cpu_quantize_baseline(fmt, A_bits, x, mx, torch, np)
    return line


def bench_step(args, name, w, A_bits, B_bits, to_dev, mx, torch, np):
    fmt, M, N, K = w["fmt"], w["M"], w["N"], w["K"]
    dev = torch.device("cuda:0")
    A = to_dev(A_bits)
    Bx = to_dev(B_bits)
    wfmt = "mxfp4" if fmt == "w4a16" else fmt
    variant = dict(scale_rule=w.get("scale_rule", "ceil"), rotation=w.get("rotation"))
    # weights: pre-quantized, outside the timed step (rotated like A when the
    # step rotates, so that the product is unchanged; OAS is an activation-side
    # choice and W keeps the standard rule)
    qb = mx.quantize(Bx, wfmt, rotation=variant["rotation"])
    del Bx
    # Operands go to the GEMM in the K-panel layout where it has one: the
    # weights re-laid once with their quantization (mx_pack), the activations
    # quantized straight into it in the step, so each GEMM step reads one
    # contiguous range per operand tile; qb keeps the row layout for the CPU
    # baseline.
    panel = fmt in PANEL_GEOMETRY and K % PANEL_GEOMETRY[fmt][0] == 0
    qw = mx.pack(qb) if panel else qb
    wbytes = qw.codes.numel() * qw.codes.element_size() + qw.scales.numel() * qw.scales.element_size()
    nwcopies = max(2, -(-WEIGHT_ROTATE_BYTES // wbytes))
    weights = [qw] + [dataclasses.replace(qw, codes=qw.codes.clone(), scales=qw.scales.clone())
                      for _ in range(nwcopies - 1)]
    ncopies = max(1, min(8, ROTATE_BYTES // A.numel() // 2))
    acts = [A] + [A.clone() for _ in range(ncopies - 1)]
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    wsb = mx.mx_gemm_workspace_bytes(mx.FORMATS.get(fmt, mx.MX_FMT_BF16) if fmt != "w4a16" else mx.MX_FMT_BF16,
                                     mx.FORMATS[wfmt], M, N, K)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    quantize_a = fmt != "w4a16"
    layout = "kpanel" if panel else "rows"
    stream = torch.cuda.current_stream(dev)

    def quant(i):
        return mx.quantize(acts[i % len(acts)], fmt, layout=layout, **variant)

    def step(i, ev=None):
        a = acts[i % len(acts)]
        if ev is not None:
            ev[0].record(stream)
        qa = quant(i) if quantize_a else a
        if ev is not None:
            ev[1].record(stream)
        mx.gemm(qa, weights[i % len(weights)], torch.bfloat16, out=out, workspace=ws)
        if ev is not None:
            ev[2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Whole-step time: the K steps captured once as a HIP graph and replayed,
    # so host launch cost stays off the GPU's critical path (as in a serving
    # loop). The library enqueues kernels only (no allocation, memset or
    # synchronisation), so the steps capture as they run eagerly.
    ms_per_step, replay_ms, ramp_replays, ramp_s, graph = graph_ms_per_step(
        torch, step, args.steps, stream, args.ramp_s)
    graph_out = out.clone()

    # Per-kernel times: the same K steps run eagerly, each launch bracketed by
    # HIP events on the stream it runs on. Graph replays queued first keep the
    # GPU busy for at least 20 ms while the host enqueues those launches, so
    # the GPU runs them back to back and no host gap lands inside a bracket.
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for _ in range(max(1, math.ceil(20.0 / (ms_per_step * args.steps)))):
        graph.replay()
    start.record(stream)
    for i in range(args.steps):
        step(i, evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    eager_ms_per_step = start.elapsed_time(end) / args.steps
    graph_matches_eager = bool(torch.equal(graph_out.view(torch.int16), out.view(torch.int16)))
    q_ms_events = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    g_avg = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps

    flops = 2.0 * M * N * K
    value = flops / (ms_per_step * 1e-3) / 1e12
    gemm_tflops = flops / (g_avg * 1e-3) / 1e12
    if fmt == "w4a16":
        # Decode GEMM is HBM-bound: algorithmic bytes = weights + scales +
        # activations + output.
        g_bytes = N * K / 2 + N * K / 32 + M * K * 2 + M * N * 2
        roof = {"bound": "hbm", "achieved": g_bytes / (g_avg * 1e-3) / 1e9, "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "algorithmic_bytes": g_bytes}
    elif fmt in ("mxfp4_mbs", "mxfp4_mbs16"):
        # 2 vector operations (factor product, fma into the accumulator) per
        # output element per 128-element macro block.
        valu_ops = 2.0 * M * N * (K // 128)
        roof = {"bound": "alu", "achieved": valu_ops / (g_avg * 1e-3) / 1e12, "peak": PEAK_VALU_TOPS,
                "unit": "Top/s (fp32 vector lane operations)"}
    else:
        roof = {"bound": "mfma", "achieved": gemm_tflops, "peak": PEAK_MFMA[fmt], "unit": "TFLOP/s",
                "peak_is": MFMA_NAME[fmt] + " MFMA"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(name)
    roof["kernel_ms"] = g_avg

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE[fmt],
        "data": "synthetic",
        "config": {"workload": name, "format": fmt, "M": M, "N": N, "K": K,
                   "scale_rule": variant["scale_rule"], "rotation": variant["rotation"],
                   "step": ("quantize(A) + gemm" if quantize_a else "gemm") + ", bf16 out",
                   "weights": "pre-quantized" + (", K-panel layout" if panel else ""),
                   "activation_layout": "K-panel" if panel else "rows",
                   "activation_copies_rotated": len(acts),
                   "weight_copies_rotated": len(weights)},
        "timing": {"ms_per_step": "HIP-graph replay of the timed steps",
                   "clock_ramp": f"{ramp_replays} untimed replays of the {args.steps} steps "
                                 f"({ramp_s * 1e3:.0f} ms) after the {args.warmup} warm-up steps",
                   "replays_ms_per_step": spread(replay_ms),
                   "eager_ms_per_step": eager_ms_per_step,
                   "kernel_ms": "HIP events around each launch in an eager pass of the same steps, enqueued behind graph replays so that they run back to back",
                   "graph_output_matches_eager": graph_matches_eager},
        "roofline": roof,
        "gemm": {"TFLOP/s": gemm_tflops, "ms": g_avg,
                 "frac_of_" + MFMA_NAME[fmt] + "_mfma": gemm_tflops / PEAK_MFMA[fmt],
                 "frac_of_" + FORMAT_NAME[fmt] + "_format_peak": gemm_tflops / PEAK_FORMAT[fmt]},
    }
    if quantize_a:
        # The activation quantizer alone: a graph of quantize-only steps over
        # the same activation copies (no event brackets inside the timing).
        q_ms, q_all, _, _, _ = graph_ms_per_step(torch, quant, args.steps, stream, args.ramp_s)
        q_bytes = M * K * (2 + ELEM_BYTES[fmt]) + (4 if fmt == "nvfp4" else 0)
        q_gbps = q_bytes / (q_ms * 1e-3) / 1e9
        line["quantize"] = {"GB/s": q_gbps, "ms": q_ms, "frac_of_hbm": q_gbps / PEAK_HBM_GBPS,
                            "algorithmic_bytes": q_bytes,
                            "timing": "HIP-graph replay of quantize-only steps",
                            "replays_ms": spread(q_all), "ms_events_in_step": q_ms_events}
    if not args.no_cpu_baseline:
        line["cpu_baseline"], line["parity"] = cpu_step_baseline(
            name, fmt, A_bits, B_bits, qb, out, A, M, N, K, args.cpu_rows, variant, panel, mx, torch, np)
    return line


def measured_traffic(workload):
    """HBM bytes per dispatch of the dominant kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary (scaled by the copy calibration),
    or None when there is none for this workload or the kernel source changed
    since it was taken: the record's hash covers its source file followed by
    the headers it lists (shared kernel code such as the epilogue)."""
    import glob
    import hashlib
    import re
    for path in glob.glob(os.path.join(ROOT, "profiles", "*.md")):
        text = open(path).read()
        for block in re.findall(r"```json\n(.*?)\n```", text, re.S):
            try:
                rec = json.loads(block)
            except ValueError:
                continue
            if rec.get("workload") != workload or "traffic_bytes" not in rec:
                continue
            paths = [os.path.join(ROOT, f) for f in [rec["source"], *rec.get("headers", [])]]
            if not all(os.path.exists(f) for f in paths):
                return None
            sha = hashlib.sha256(b"".join(open(f, "rb").read() for f in paths)).hexdigest()[:16]
            return rec["traffic_bytes"] if sha == rec["source_sha256_16"] else None
    return None


ORC_FMT_NAMES = {"mxfp4": "FMT_MXFP4", "mxfp8": "FMT_MXFP8", "nvfp4": "FMT_NVFP4",
                 "w4a16": "FMT_BF16", "mxfp8_e5m2": "FMT_MXFP8_E5M2",
                 "mxfp6_e3m2": "FMT_MXFP6_E3M2", "mxfp4_mbs": "FMT_MXFP4_MBS",
                 "mxfp4_mbs16": "FMT_MXFP4_MBS16"}


def _oracle_quant(orc, ofmt, bits, variant):
    """Oracle codes and scales of a bf16 operand with the step's variant."""
    if variant["scale_rule"] != "ceil" or variant["rotation"]:
        c, s = orc.quantize_ex(ofmt, bits, orc.RULE_OAS if variant["scale_rule"] == "oas" else orc.RULE_CEIL,
                               orc.ROT_WHT32 if variant["rotation"] == "wht32" else orc.ROT_NONE)
        return c, s, 1.0
    return orc.quantize(ofmt, bits)


def cpu_step_baseline(name, fmt, A_bits, B_bits, qb, out, A_dev, M, N, K, rows, variant, panel,
                      mx, torch, np):
    """The oracle on the first `rows` activation rows of the step: quantize
    those rows (one thread), then their exact GEMM against all N weight rows
    (double accumulation, OpenMP over the host cores). Timed and scaled to
    TFLOP/s of 2 rows N K. The same sample is the parity check: the weights'
    and the sample rows' GPU codes and scales against the oracle's (bit for
    bit; the activations quantized again on the GPU in the step's own launch
    configuration), and the step's bf16 outputs of those rows against the
    oracle's exact GEMM within 2^-18 sum|ab| (1 + 2^-8) + 2^-8 |C|."""
    import oracle as orc
    ofmt = getattr(orc, ORC_FMT_NAMES[fmt])
    if rows <= 0:
        rows = int(max(1, min(M, CPU_BUDGET_MACS // (N * K))))
    rows = min(rows, M)
    wvar = dict(scale_rule="ceil", rotation=variant["rotation"])
    bfmt = orc.FMT_MXFP4 if fmt == "w4a16" else ofmt
    bc, bs, bts = _oracle_quant(orc, bfmt, B_bits, wvar)
    b_exact = bool(np.array_equal(qb.codes.cpu().numpy(), bc) and
                   np.array_equal(qb.scales.cpu().numpy().reshape(-1), np.asarray(bs).reshape(-1)))
    a = np.ascontiguousarray(A_bits[:rows])
    threads = orc.num_threads()
    # NVFP4's tensor scale comes from all M rows, so the oracle quantizes the
    # whole activation tensor and the GEMM takes the sample rows of it.
    qrows = M if fmt == "nvfp4" else rows
    t0 = time.perf_counter()
    if fmt == "w4a16":
        ac, asc, ats = a, None, 1.0
    elif fmt == "nvfp4":
        fc, fs, ats = orc.quantize(ofmt, A_bits)
        ac, asc = fc[:rows], fs[:rows]
    else:
        ac, asc, ats = _oracle_quant(orc, ofmt, a, variant)
    C, S = orc.gemm(ofmt, bfmt, rows, N, K, ac, asc, ats, bc, bs, bts)
    dt = time.perf_counter() - t0
    baseline = {"value": 2.0 * rows * N * K / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
                "kind": "oracle", "seconds": dt,
                "sample": f"oracle quantize of {qrows} of {M} activation rows (one thread) + exact "
                          f"GEMM of the first {rows} rows against all {N} weight rows, K={K} "
                          f"(OpenMP, {threads} threads)"}
    parity = {"weights_codes_scales_bitexact": b_exact}
    if fmt != "w4a16":
        q = mx.quantize(A_dev, fmt, layout="kpanel" if panel else "rows", **variant)
        gc, gs = q.codes.cpu().numpy(), q.scales.cpu().numpy()
        if panel:
            W, wb, sb = PANEL_GEOMETRY[fmt]
            P = K // W
            gc = gc.reshape(P, M, wb)[:, :rows].transpose(1, 0, 2).reshape(rows, P * wb)
            gs = gs.reshape(P, M, sb)[:, :rows].transpose(1, 0, 2).reshape(rows, P * sb)
        elif fmt in ("mxfp4_mbs", "mxfp4_mbs16"):
            blk = 16 if fmt == "mxfp4_mbs16" else 32
            e8, mac = orc.mbs_planes(gs, M, K, blk)
            gs = np.concatenate([e8[:rows].reshape(-1), mac[:rows].reshape(-1)])
            gc = gc[:rows]
        else:
            gc, gs = gc[:rows], gs[:rows]
        a_exact = bool(np.array_equal(gc, ac) and np.array_equal(np.asarray(gs).reshape(-1),
                                                                  np.asarray(asc).reshape(-1)))
        if fmt == "nvfp4":
            a_exact = a_exact and float(q.tensor_scale.cpu().numpy()[0]) == ats
        parity["sample_codes_scales_bitexact"] = a_exact
    got = out[:rows].float().cpu().numpy().astype(np.float64)
    tol = 2.0**-18 * S * (1 + 2.0**-8) + 2.0**-8 * np.abs(C)
    ratio = np.abs(got - C) / np.maximum(tol, 1e-300)
    parity.update({"outputs_checked": int(rows * N), "max_err_over_bound": float(np.max(ratio)),
                   "bound": "2^-18 sum|ab| (1 + 2^-8) + 2^-8 |C| (bf16 output)",
                   "pass": bool(np.all(ratio <= 1.0)) and b_exact and
                   parity.get("sample_codes_scales_bitexact") is not False})
    return baseline, parity


def cpu_quantize_baseline(fmt, A_bits, x, mx, torch, np):
    """The oracle quantizer (one thread) on the leading rows of the tensor, up
    to 2^27 elements (about 10 s); its GB/s uses the same algorithmic bytes. Parity: the
    GPU's codes and scales of those rows against the oracle's, bit for bit."""
    import oracle as orc
    ofmt = getattr(orc, ORC_FMT_NAMES[fmt])
    M, K = A_bits.shape
    rows = max(1, min(M, (1 << 27) // K))
    t0 = time.perf_counter()
    oc, os_, _ = orc.quantize(ofmt, np.ascontiguousarray(A_bits[:rows]))
    dt = time.perf_counter() - t0
    q = mx.quantize(x, fmt)
    exact = bool(np.array_equal(q.codes[:rows].cpu().numpy(), oc) and
                 np.array_equal(q.scales[:rows].cpu().numpy(), os_))
    nbytes = rows * K * (2 + ELEM_BYTES[fmt])
    return ({"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle", "seconds": dt,
             "sample": f"first {rows} of {M} rows, one thread"},
            {"sample_codes_scales_bitexact": exact, "rows_checked": rows, "pass": exact})


if __name__ == "__main__":
    main()
