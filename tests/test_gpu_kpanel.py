"""GPU parity for the K-panel layout of the formats on the 16-bit MFMAs
(MXFP8, MXFP8-E5M2, MXFP6-E3M2, NVFP4; 64-element panels): the quantizer's
K-panel output and mx_pack against the oracle's codes and scales re-laid by
the layout's definition, bit for bit; the GEMM on K-panel operands bit for
bit equal to the row-layout GEMM and within the oracle's bound; and the step
bench.py times on these workloads, at full size, every code, scale and
output checked."""
import numpy as np
import pytest
import torch

import microscaling_precision_quantization_amd as mx
import oracle as orc
import synth
from gpu_helpers import (ORC_FMT, check_gemm, dev_bf16, dev_u8, host, oracle_gemm_cached,
                         oracle_quant, qtensor_from_host, require_gpu, workload)

pytestmark = pytest.mark.gpu

FMTS = ["mxfp8", "mxfp8_e5m2", "mxfp6_e3m2", "nvfp4"]


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _oracle_panels(fmt, codes, scales, rows, cols):
    return orc.pack_kpanel(codes, scales, rows, cols, ORC_FMT[fmt])


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rows,cols", [(1, 64), (3, 192), (129, 320), (255, 1024), (300, 4096)])
def test_kpanel_quantize_is_the_packed_row_output(fmt, rows, cols):
    """mx_quantize_layout's K-panel output: the oracle's codes and scales in
    K-panel order, bit for bit, and the same NVFP4 tensor scale. Row counts
    that are not whole 128-row groups (odd ones included: for MXFP8 a 16-lane
    scale group then holds one row past the end) and single panels."""
    bits = synth.laplace_outlier_channels((rows, cols), seed=901 + rows, channel_seed=902,
                                          frac=0.01, factor=100.0)
    q = mx.quantize(dev_bf16(bits), fmt, layout="kpanel")
    assert q.layout == mx.MX_LAYOUT_KPANEL
    oc, os_, ts = orc.quantize(ORC_FMT[fmt], bits)
    pc, ps = _oracle_panels(fmt, oc, os_, rows, cols)
    assert np.array_equal(host(q.codes).reshape(-1), pc)
    assert np.array_equal(host(q.scales).reshape(-1), ps)
    if fmt == "nvfp4":
        assert float(host(q.tensor_scale)[0]) == ts


@pytest.mark.parametrize("fmt", FMTS)
def test_kpanel_quantize_specials(fmt):
    """Zero, -0, subnormal, Inf and NaN blocks, and a row of the largest
    finite bf16, in the K-panel output."""
    g = np.random.Generator(np.random.PCG64(911))
    bits = synth.bf16_bits(g.normal(0, 1, (9, 256)))
    bits[0, :32] = 0
    bits[1, 32:64] = 0x8000
    bits[2, 64:96] = g.integers(1, 0x80, 32).astype(np.uint16)
    bits[3, 130] = 0x7F80
    bits[4, 250] = 0xFFC0
    bits[5, :] = 0x7F7F
    q = mx.quantize(dev_bf16(bits), fmt, layout="kpanel")
    oc, os_, ts = orc.quantize(ORC_FMT[fmt], bits)
    pc, ps = _oracle_panels(fmt, oc, os_, 9, 256)
    assert np.array_equal(host(q.codes).reshape(-1), pc)
    assert np.array_equal(host(q.scales).reshape(-1), ps)
    if fmt == "nvfp4":
        got = float(host(q.tensor_scale)[0])
        assert got == ts or (np.isnan(got) and np.isnan(ts))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rows,cols", [(1, 64), (37, 192), (256, 1024), (513, 3072)])
def test_pack_is_the_kpanel_permutation(fmt, rows, cols):
    g = np.random.Generator(np.random.PCG64(921 + rows))
    f = ORC_FMT[fmt]
    codes = g.integers(0, 256, (rows, mx.code_cols(mx.FORMATS[fmt], cols)), dtype=np.uint8)
    scales = g.integers(0, 256, (rows, cols // orc.BLOCK[f]), dtype=np.uint8)
    ts = torch.ones(1, dtype=torch.float32, device="cuda") if fmt == "nvfp4" else None
    q = mx.QTensor(mx.FORMATS[fmt], rows, cols, dev_u8(codes), dev_u8(scales), ts)
    p = mx.pack(q)
    torch.cuda.synchronize()
    pc, ps = _oracle_panels(fmt, codes, scales, rows, cols)
    assert np.array_equal(host(p.codes).reshape(-1), pc)
    assert np.array_equal(host(p.scales).reshape(-1), ps)


def _gemm(qa, qb, out):
    c = mx.gemm(qa, qb, torch.float32 if out == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    return host(c.float())


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(256, 256, 64), (300, 520, 320), (257, 255, 1024),
                                   (37, 1000, 3072), (600, 300, 1600)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemm_kpanel_both(fmt, shape, out):
    """Both operands in K panels: bit for bit the row-layout GEMM on the same
    codes (rows past M and N in the last tiles, the 224- and 256-row tile
    heights, fp32 output over several K segments at K = 1024, 1600 and 3072),
    and within the oracle's bound."""
    M, N, K = shape
    A = synth.laplace_outlier_channels((M, K), seed=931 + M, channel_seed=932, frac=0.01, factor=50.0)
    B = synth.normal((N, K), 0.02, 933 + N)
    f = ORC_FMT[fmt]
    a = orc.quantize(f, A)
    b = orc.quantize(f, B)
    ts = fmt == "nvfp4"
    qa = qtensor_from_host(fmt, a[0], a[1], a[2] if ts else None, M, K)
    qb = qtensor_from_host(fmt, b[0], b[1], b[2] if ts else None, N, K)
    ref = _gemm(qa, qb, out)
    got = _gemm(mx.pack(qa), mx.pack(qb), out)
    assert np.array_equal(ref.view(np.uint32), got.view(np.uint32))
    C, S = orc.gemm(f, f, M, N, K, *a, *b)
    check_gemm(got, C, S, out, f"{fmt} kpanel {shape} {out}")


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_kpanel_one_operand_unsupported(fmt):
    """A single K-panel operand is refused for these formats (the kernel reads
    both operands in one layout)."""
    M, N, K = 64, 64, 128
    q = mx.quantize(dev_bf16(synth.normal((M, K), 1.0, 941)), fmt)
    with pytest.raises(RuntimeError):
        mx.gemm(mx.pack(q), q, torch.float32)


@pytest.mark.parametrize("wl,fmt", [("c2", "mxfp8"), ("c3", "nvfp4"), ("f2a", "mxfp8_e5m2"),
                                    ("f2b", "mxfp6_e3m2")])
def test_bench_step_configuration_every_element(wl, fmt):
    """The step bench.py times on this workload, at its full size and in its
    launch configuration: the activations quantized on the GPU straight into
    K panels, the weights quantized on the GPU and packed, bf16 output. Every
    code and scale of both operands (and the NVFP4 tensor scales) equals the
    oracle's in K-panel order, and every output is within the bound."""
    A, B = workload(wl)
    M, K = A.shape
    N = B.shape[0]
    qa = mx.quantize(dev_bf16(A), fmt, layout="kpanel")
    qb = mx.pack(mx.quantize(dev_bf16(B), fmt))
    got = _gemm(qa, qb, "bf16")
    a = oracle_quant(wl, "A", fmt)
    b = oracle_quant(wl, "B", fmt)
    for q, (codes, scales, ts), rows, what in ((qa, a, M, "A"), (qb, b, N, "B")):
        pc, ps = _oracle_panels(fmt, codes, scales, rows, K)
        assert np.array_equal(host(q.codes).reshape(-1), pc), f"{wl}: {what} codes differ"
        assert np.array_equal(host(q.scales).reshape(-1), ps), f"{wl}: {what} scales differ"
        if fmt == "nvfp4":
            assert float(host(q.tensor_scale)[0]) == ts, f"{wl}: {what} tensor scale differs"
    f = ORC_FMT[fmt]
    C, S = oracle_gemm_cached((wl, fmt, "ceil", None), f, f, M, N, K, *a, *b)
    check_gemm(got, C, S, "bf16", f"{wl} bench step")
