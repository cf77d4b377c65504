"""Benchmark of the microscaling hot path on one MI355X.

Default workload: the MXFP4 W4A4 DiT MLP-down layer, M=4608 tokens, K=12288,
N=3072, activations Laplace(0,1) with 0.5% outlier channels x100, weights
N(0,0.02) quantized beforehand. One step = quantize the bf16 activations to
MXFP4 (codes + E8M0 scales) and run the block-scaled GEMM against the
pre-quantized weights, bf16 output (MXFP4 operands in the K-panel layout:
weights re-laid once by mx_pack, activations quantized straight into it).
Everything in the timed region runs in
libmx's HIP kernels; inputs are resident in HBM before timing starts. After
the warm-up steps the same steps are replayed, untimed, for RAMP_S seconds:
the GPU raises its clocks only after tens of milliseconds of continuous load,
and the timed steps should see the clocks a sustained workload runs at.

Prints one JSON line. `value` is whole-step throughput, 2MNK / step time, in
TFLOP/s. The `roofline` object is for the dominant kernel (the GEMM), timed
with HIP events on its own stream; `quantize` reports the activation
quantizer's algorithmic GB/s; `cpu_baseline` times the oracle on a bounded
sample of the same step on the host.

Other workloads (--workload c1..c5) are for profiling; the default is the one
the headline metric is quoted on.
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
# Dense MFMA peaks the GEMM is measured against: the element format's own
# matrix rate where a native path exists or would exist (MXFP4 on the FP4
# scaled MFMA; MXFP8 against FP8 even though the exact path runs on bf16),
# otherwise the 16-bit MFMA the exact path runs on (NVFP4: fp16 operands,
# W4A16: bf16; MXFP6 against the FP6/FP4 rate, as MXFP8 against FP8).
PEAK_TFLOPS = {"mxfp4": 10100.0, "mxfp8": 5000.0, "nvfp4": 2500.0, "w4a16": 2500.0,
               "mxfp8_e5m2": 5000.0, "mxfp6_e3m2": 10100.0, "mxfp4_mbs": 10100.0}
# fp32 vector lane-operations per second (one mul or one fma per lane per
# cycle, no packed math): 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz. The MBS GEMM
# is bound by its per-macro-block rescale on the vector ALU (2 operations per
# output element per 128 K), so it is measured against this.
PEAK_VALU_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
ROTATE_BYTES = 1 << 30  # activation copies cycled per step: > 256 MB MALL
RAMP_S = 0.2  # seconds of untimed replays before timing (GPU clock ramp)
WEIGHT_ROTATE_BYTES = 512 << 20  # weight copies cycled per step: > 256 MB MALL, so
                                 # every step streams its weights from HBM, as the
                                 # layers of a model would


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="c4")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--ramp-s", type=float, default=RAMP_S,
                   help="seconds of untimed replays between the warm-up and the timed steps")
    p.add_argument("--cpu-rows", type=int, default=640,
                   help="activation rows in the oracle's CPU sample")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain device-to-device copy of 1 GiB, 5 times (reference "
                        "for scaling the HBM byte counters)")
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


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
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
    fmt, M, N, K = w["fmt"], w["M"], w["N"], w["K"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t0 = time.time()
    A_bits, B_bits = synth.workload(name)
    gen_s = time.time() - t0

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    A = to_dev(A_bits)
    Bx = to_dev(B_bits)
    wfmt = "mxfp4" if fmt == "w4a16" else fmt
    variant = dict(scale_rule=w.get("scale_rule", "ceil"), rotation=w.get("rotation"))
    # weights: pre-quantized, outside the timed step (rotated like A when the
    # step rotates, so that the product is unchanged; OAS is an activation-side
    # choice and W keeps the standard rule)
    qb = mx.quantize(Bx, wfmt, rotation=variant["rotation"])
    del Bx
    # MXFP4 operands go to the GEMM in the K-panel layout: the weights re-laid
    # once with their quantization (mx_pack), the activations quantized
    # straight into it in the step, so each GEMM step reads one contiguous
    # range per operand tile; qb keeps the row layout for the CPU baseline.
    panel = fmt == "mxfp4" and K % 256 == 0
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
    stream = torch.cuda.current_stream(dev)

    def step(i, ev=None):
        a = acts[i % len(acts)]
        if ev is not None:
            ev[0].record(stream)
        if quantize_a:
            qa = mx.quantize(a, fmt, layout="kpanel" if panel else "rows", **variant)
        else:
            qa = a
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
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(args.steps):
            step(i)
    graph.replay()
    torch.cuda.synchronize()
    graph_out = out.clone()
    # Clock ramp: the GPU raises its clocks only after tens of milliseconds of
    # continuous load (measured: the c4 step takes ~122 us right after a short
    # warm-up, ~107 us in steady state, and ~125 us again after 2 s idle), so
    # replay the same steps, untimed, for at least RAMP_S before timing.
    t_ramp = time.perf_counter()
    ramp_replays = 0
    while time.perf_counter() - t_ramp < args.ramp_s:
        graph.replay()
        ramp_replays += 1
        torch.cuda.synchronize()
    ramp_s = time.perf_counter() - t_ramp
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    graph.replay()
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    # Spread: four more timed replays of the same steps (reported beside the
    # single timed pass that `value` comes from).
    replay_ms = [ms_per_step]
    for _ in range(4):
        start.record(stream)
        graph.replay()
        end.record(stream)
        torch.cuda.synchronize()
        replay_ms.append(start.elapsed_time(end) / args.steps)

    # Per-kernel times: the same K steps run eagerly, each launch bracketed by
    # HIP events on the stream it runs on. Graph replays queued first keep the
    # GPU busy for at least 20 ms while the host enqueues those launches, so
    # the GPU runs them back to back and no host gap lands inside a bracket.
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
    q_ms = [e[0].elapsed_time(e[1]) for e in evs]
    g_ms = [e[1].elapsed_time(e[2]) for e in evs]
    q_avg = sum(q_ms) / len(q_ms)
    g_avg = sum(g_ms) / len(g_ms)

    flops = 2.0 * M * N * K
    value = flops / (ms_per_step * 1e-3) / 1e12
    gemm_tflops = flops / (g_avg * 1e-3) / 1e12
    peak = PEAK_TFLOPS[fmt]
    # Algorithmic bytes of the quantizer: read bf16 once, write codes + scales.
    elem_bytes = {"mxfp4": 0.5 + 1 / 32, "mxfp8": 1 + 1 / 32, "nvfp4": 0.5 + 1 / 16,
                  "mxfp8_e5m2": 1 + 1 / 32, "mxfp6_e3m2": 0.75 + 1 / 32,
                  "mxfp4_mbs": 0.5 + 1 / 32 + 1 / 128}
    q_bytes = M * K * (2 + elem_bytes.get(fmt, 0)) + (4 if fmt == "nvfp4" else 0)

    if fmt == "w4a16":
        # Decode GEMM is HBM-bound: algorithmic bytes = weights + scales +
        # activations + output.
        g_bytes = N * K / 2 + N * K / 32 + M * K * 2 + M * N * 2
        roof = {"bound": "hbm", "achieved": g_bytes / (g_avg * 1e-3) / 1e9, "peak": PEAK_HBM_GBPS,
                "unit": "GB/s"}
    elif fmt == "mxfp4_mbs":
        # 2 vector operations (factor product, fma into the accumulator) per
        # output element per 128-element macro block.
        valu_ops = 2.0 * M * N * (K // 128)
        roof = {"bound": "alu", "achieved": valu_ops / (g_avg * 1e-3) / 1e12, "peak": PEAK_VALU_TOPS,
                "unit": "Top/s (fp32 vector lane operations)"}
    else:
        roof = {"bound": "mfma", "achieved": gemm_tflops, "peak": peak, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(name)
    roof["kernel_ms"] = g_avg

    line = {
        "metric": "block-scaled GEMM TFLOP/s + quantize GB/s, % of MXFP4/FP8 MFMA & HBM peak",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"mxfp4": "e2m1+e8m0 (fp32 accumulate)", "mxfp8": "e4m3+e8m0 via bf16 (fp32 accumulate)",
                  "nvfp4": "e2m1+e4m3 via fp16 (fp32 accumulate)",
                  "w4a16": "bf16 x e2m1+e8m0 (fp32 accumulate)",
                  "mxfp8_e5m2": "e5m2+e8m0 via bf16 (fp32 accumulate)",
                  "mxfp6_e3m2": "e3m2+e8m0 via bf16 (fp32 accumulate)",
                  "mxfp4_mbs": "e2m1+e8m0, macro factor 1+m/256 (fp32 accumulate)"}[fmt],
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
                   "replays_ms_per_step": {"min": min(replay_ms),
                                           "median": sorted(replay_ms)[len(replay_ms) // 2],
                                           "max": max(replay_ms), "n": len(replay_ms)},
                   "eager_ms_per_step": eager_ms_per_step,
                   "kernel_ms": "HIP events around each launch in an eager pass of the same steps, enqueued behind graph replays so that they run back to back",
                   "graph_output_matches_eager": graph_matches_eager},
        "roofline": roof,
        "gemm": {"TFLOP/s": gemm_tflops, "ms": g_avg, "frac_of_peak": gemm_tflops / peak},
    }
    if quantize_a:
        q_gbps = q_bytes / (q_avg * 1e-3) / 1e9
        line["quantize"] = {"GB/s": q_gbps, "ms": q_avg, "frac_of_hbm": q_gbps / PEAK_HBM_GBPS,
                            "algorithmic_bytes": q_bytes}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(name, fmt, A_bits, qb, M, N, K, args.cpu_rows, variant)
    line["input_gen_s"] = round(gen_s, 2)
    print(json.dumps(line), flush=True)


def measured_traffic(workload):
    """HBM bytes per GEMM dispatch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary (scaled by the copy calibration), or None when there is
    none for this workload or the kernel source changed since it was taken."""
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
            src = os.path.join(ROOT, rec["source"])
            if not os.path.exists(src):
                return None
            sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
            return rec["traffic_bytes"] if sha == rec["source_sha256_16"] else None
    return None


def cpu_baseline(name, fmt, A_bits, qb, M, N, K, rows, variant):
    """The oracle (single-threaded C) on the first `rows` activation rows of the
    same step: quantize those rows, then their GEMM against all N weight rows
    (exact operands, double accumulation). Scaled to TFLOP/s of 2*rows*N*K."""
    import numpy as np

    import oracle as orc
    ofmt = {"mxfp4": orc.FMT_MXFP4, "mxfp8": orc.FMT_MXFP8, "nvfp4": orc.FMT_NVFP4,
            "w4a16": orc.FMT_BF16, "mxfp8_e5m2": orc.FMT_MXFP8_E5M2,
            "mxfp6_e3m2": orc.FMT_MXFP6_E3M2, "mxfp4_mbs": orc.FMT_MXFP4_MBS}[fmt]
    bcodes = qb.codes.cpu().numpy()
    bscales = qb.scales.cpu().numpy()
    bts = float(qb.tensor_scale.cpu().numpy()[0]) if qb.tensor_scale is not None else 1.0
    rows = min(rows, M)
    a = np.ascontiguousarray(A_bits[:rows])
    t0 = time.perf_counter()
    if ofmt == orc.FMT_BF16:
        ac, asc, ats = a, None, 1.0
        fb = orc.FMT_MXFP4
    elif variant["scale_rule"] != "ceil" or variant["rotation"]:
        ac, asc = orc.quantize_ex(ofmt, a, orc.RULE_OAS if variant["scale_rule"] == "oas" else orc.RULE_CEIL,
                                  orc.ROT_WHT32 if variant["rotation"] == "wht32" else orc.ROT_NONE)
        ats, fb = 1.0, ofmt
    else:
        ac, asc, ats = orc.quantize(ofmt, a)
        fb = ofmt
    orc.gemm(ofmt, fb, rows, N, K, ac, asc, ats, bcodes, bscales, bts)
    dt = time.perf_counter() - t0
    return {"value": 2.0 * rows * N * K / dt / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "seconds": dt,
            "sample": f"first {rows} of {M} activation rows: oracle quantize + exact GEMM against "
                      f"all {N} weight rows, K={K}, one thread"}


if __name__ == "__main__":
    main()
