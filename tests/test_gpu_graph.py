"""The library's calls under HIP-graph capture. Every step here is captured
once (quantize A, then the GEMM against pre-quantized weights, each with the
workspace it needs) and replayed with a new input in the captured input
buffer. Between replays the same calls run eagerly on other inputs, with
other torch work and synchronisations. Every replay's codes, scales, tensor
scale and GEMM output must equal, bit for bit, the eager result for its input.
Covered: the NVFP4 two-kernel quantize with its partials workspace, the fp32
GEMM output accumulated over several launches, the W4A16 split-K partials and
reduce, and the no-allocation GEMM entry point, which exists for callers that
capture graphs."""
import ctypes

import pytest
import torch

import microscaling_precision_quantization_amd as mx
import synth
from gpu_helpers import dev_bf16, require_gpu

pytestmark = pytest.mark.gpu

F32, BF16 = torch.float32, torch.bfloat16

# (id, format of both operands or "w4a16", A layout, output dtype, scale rule,
#  rotation, M, N, K)
CASES = [
    ("mxfp4-rows-bf16", "mxfp4", "rows", BF16, "ceil", None, 512, 512, 1024),
    ("mxfp4-kpanel-f32-segments", "mxfp4", "kpanel", F32, "ceil", None, 300, 520, 4096),
    ("mxfp4-oas-wht32", "mxfp4", "rows", BF16, "oas", "wht32", 256, 256, 768),
    ("mxfp8-kpanel-bf16", "mxfp8", "kpanel", BF16, "ceil", None, 300, 520, 1024),
    ("mxfp8-rows-f32-segments", "mxfp8", "rows", F32, "ceil", None, 257, 255, 1600),
    ("nvfp4-kpanel-f32", "nvfp4", "kpanel", F32, "ceil", None, 300, 256, 1024),
    ("nvfp4-rows-bf16", "nvfp4", "rows", BF16, "ceil", None, 256, 300, 512),
    ("e5m2-kpanel-bf16", "mxfp8_e5m2", "kpanel", BF16, "ceil", None, 256, 256, 512),
    ("e3m2-kpanel-bf16", "mxfp6_e3m2", "kpanel", BF16, "ceil", None, 300, 256, 1024),
    ("mbs-bf16", "mxfp4_mbs", "rows", BF16, "ceil", None, 256, 256, 1024),
    ("mbs16-f32", "mxfp4_mbs16", "rows", F32, "ceil", None, 256, 256, 512),
    ("w4a16-bf16", "w4a16", None, BF16, "ceil", None, 16, 2048, 8192),
    ("w4a16-f32", "w4a16", None, F32, "ceil", None, 5, 3000, 6144),
]


def _bits(t):
    """The tensor's bytes, so that equal NaNs compare equal."""
    return t.contiguous().view(torch.uint8)


def _weights(fmt, layout, N, K, seed):
    wfmt = "mxfp4" if fmt == "w4a16" else fmt
    qw = mx.quantize(dev_bf16(synth.normal((N, K), 0.02, seed)), wfmt)
    return mx.pack(qw) if layout == "kpanel" else qw


def _step(case, x, qw):
    """The captured work: quantize(x) and the GEMM; returns every output."""
    _, fmt, layout, out_dtype, rule, rot, *_ = case
    if fmt == "w4a16":
        return [mx.gemm(x, qw, out_dtype)]
    if rule != "ceil" or rot is not None:
        q = mx.quantize(x, fmt, scale_rule=rule, rotation=rot, layout=layout)
    else:
        q = mx.quantize(x, fmt, layout=layout)
    c = mx.gemm(q, qw, out_dtype)
    outs = [q.codes, q.scales, c]
    if q.tensor_scale is not None:
        outs.append(q.tensor_scale)
    return outs


def _capture(fn):
    """fn() captured as a graph after one warm-up run on a side stream;
    returns the graph and fn's outputs in the graph's memory."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = fn()
    torch.cuda.synchronize()
    return graph, outs


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_equal_eager(case):
    require_gpu()
    name, fmt, layout, out_dtype, rule, rot, M, N, K = case
    print(f"graph {name} {M}x{N}x{K}", flush=True)
    qw = _weights(fmt, layout, N, K, 9100)
    # Outlier channels make blocks of very different scales.
    inputs = [dev_bf16(synth.laplace_outlier_channels((M, K), seed=9110 + i, channel_seed=9120 + i,
                                                      frac=0.02, factor=40.0)) for i in range(3)]
    refs = [[t.clone() for t in _step(case, x, qw)] for x in inputs]
    torch.cuda.synchronize()

    x_static = torch.empty_like(inputs[0])
    x_static.copy_(inputs[0])
    graph, outs = _capture(lambda: _step(case, x_static, qw))
    # Input order 1, 2, 0, 0: each replay recomputes, and a replay with an
    # unchanged input gives the same bits again.
    for rep, i in enumerate((1, 2, 0, 0)):
        other = _step(case, inputs[(i + 1) % 3], qw)            # eager library calls
        junk = (other[-1].float().abs() + 1.0).log().sum()       # other torch work
        torch.cuda.synchronize()
        x_static.copy_(inputs[i])
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for k, (got, want) in enumerate(zip(outs, refs[i])):
            assert torch.equal(_bits(got), _bits(want)), f"{name}: replay {rep}, output {k} differs"


@pytest.mark.parametrize("out_dtype", [BF16, F32])
def test_graph_of_noalloc_gemm(out_dtype):
    """mx_gemm_noalloc captured in a graph: every replay equals mx_gemm with
    a caller-allocated workspace on the same input (the library's scratch is
    written in full by each call before it is read)."""
    require_gpu()
    M, N, K = 16, 2048, 8192
    print(f"graph noalloc W4A16 {M}x{N}x{K} {out_dtype}", flush=True)
    qb = mx.quantize(dev_bf16(synth.normal((N, K), 0.02, 9200)), "mxfp4")
    inputs = [dev_bf16(synth.normal((M, K), 1.0, 9210 + i)) for i in range(3)]
    refs = [mx.gemm(x, qb, out_dtype).clone() for x in inputs]
    od = mx.MX_OUT_F32 if out_dtype == F32 else mx.MX_OUT_BF16
    x_static = inputs[0].clone()
    c_static = torch.empty((M, N), dtype=out_dtype, device="cuda")
    P = ctypes.c_void_p

    def call():
        stream = P(torch.cuda.current_stream().cuda_stream)
        st = mx.mx_gemm_noalloc(mx.MX_FMT_BF16, mx.MX_FMT_MXFP4, 32, mx.MX_ROUND_RNE, M, N, K,
                                P(x_static.data_ptr()), None, None, P(qb.codes.data_ptr()),
                                P(qb.scales.data_ptr()), None, od, P(c_static.data_ptr()), N, stream)
        assert st == mx.MX_OK, mx.mx_status_string(st)
        return [c_static]

    graph, _ = _capture(call)
    for rep, i in enumerate((1, 2, 0, 0)):
        mx.gemm(inputs[(i + 2) % 3], qb, out_dtype)   # eager library work in between
        torch.cuda.synchronize()
        x_static.copy_(inputs[i])
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(c_static), _bits(refs[i])), f"noalloc replay {rep} differs"
