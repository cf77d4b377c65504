"""GPU parity for MXFP8 with E5M2 elements and MXFP6 with E3M2 elements:
quantize bit for bit against the oracle (every bf16 value at every exponent,
ragged shapes, specials), dequantize of every code at every scale bit for bit,
and the GEMM within the oracle's bound."""
import numpy as np
import pytest
import torch

import microscaling_precision_quantization_amd as mx
import oracle as orc
import synth
from gpu_helpers import (ORC_FMT, check_gemm, dev_bf16, gpu_quantize, host, qtensor_from_host,
                         require_gpu)
from test_gpu_quantize import _dequant_compare, _exhaustive_blocks

pytestmark = pytest.mark.gpu

FMTS = ["mxfp8_e5m2", "mxfp6_e3m2"]
EMAX = {"mxfp8_e5m2": (57344.0, 239), "mxfp6_e3m2": (28.0, 250)}


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _assert_quant_equal(bits, fmt):
    c, s, _ = gpu_quantize(bits, fmt)
    oc, os_, _ = orc.quantize(ORC_FMT[fmt], bits)
    bad_s = np.nonzero(s != os_)
    assert bad_s[0].size == 0, f"{fmt}: {bad_s[0].size} scales differ, first at {bad_s[0][0]},{bad_s[1][0]}: gpu {s[bad_s][0]} oracle {os_[bad_s][0]}"
    bad_c = np.nonzero(c != oc)
    assert bad_c[0].size == 0, f"{fmt}: {bad_c[0].size} code bytes differ, first at {bad_c[0][0]},{bad_c[1][0]}: gpu {c[bad_c][0]:#x} oracle {oc[bad_c][0]:#x}"
    return c, s


@pytest.mark.parametrize("fmt", FMTS)
def test_exhaustive_elements_and_exponents(fmt):
    emax, e_hi = EMAX[fmt]
    x = _exhaustive_blocks(emax, e_hi)
    _, s = _assert_quant_equal(x, fmt)
    assert s.min() == 0 and s.max() == e_hi


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(1, 32), (3, 96), (257, 1056), (64, 4096), (1000, 160)])
def test_ragged_shapes(fmt, shape):
    x = synth.normal_outliers(shape, 1.0, 17 + shape[0], 0.01, 80.0)
    _assert_quant_equal(x, fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_special_blocks(fmt):
    g = np.random.Generator(np.random.PCG64(12))
    x = synth.bf16_bits(g.normal(0, 1, (8, 128)))
    x[0, :32] = 0
    x[1, :32] = 0x8000
    x[2, :32] = g.integers(1, 0x80, 32).astype(np.uint16)
    x[3, 5] = 0x7F80
    x[4, 40] = 0xFFC0
    x[5, 64:96] = 0x0001
    x[6, :] = 0x7F7F  # the largest finite bf16 in every block
    _assert_quant_equal(x, fmt)


def _all_codes_table(fmt):
    if fmt == "mxfp8_e5m2":
        codes = np.tile(np.arange(256, dtype=np.uint8), (256, 1))
        scales = np.repeat(np.arange(256, dtype=np.uint8).reshape(256, 1), 8, axis=1)
        return codes, scales, 256, 256
    # 64 six-bit codes 0..63 in two blocks per row, packed little-endian
    bits = np.zeros(64 * 6, np.uint8)
    for i in range(64):
        for b in range(6):
            bits[6 * i + b] = (i >> b) & 1
    row = np.packbits(bits, bitorder="little")
    codes = np.tile(row, (256, 1))
    scales = np.repeat(np.arange(256, dtype=np.uint8).reshape(256, 1), 2, axis=1)
    return codes, scales, 256, 64


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_dequantize_all_codes_all_scales(fmt, out):
    codes, scales, rows, cols = _all_codes_table(fmt)
    _dequant_compare(fmt, out, codes, scales, None, rows, cols)


def _gemm_check(fmt, A, B, out, what):
    M, K = A.shape
    N = B.shape[0]
    f = ORC_FMT[fmt]
    a = orc.quantize(f, A)
    b = orc.quantize(f, B)
    qa = qtensor_from_host(fmt, a[0], a[1], None, M, K)
    qb = qtensor_from_host(fmt, b[0], b[1], None, N, K)
    C, S = orc.gemm(f, f, M, N, K, a[0], a[1], 1.0, b[0], b[1], 1.0)
    got = host(mx.gemm(qa, qb, torch.float32 if out == "f32" else torch.bfloat16).float())
    return check_gemm(got, C, S, out, what)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(200, 72, 416), (1, 1, 32), (300, 520, 768), (257, 255, 512),
                                   (513, 40, 2560)])
def test_gemm_ragged(fmt, shape):
    M, N, K = shape
    A = synth.normal_outliers((M, K), 1.0, 31 + M, 0.01, 50.0)
    B = synth.normal((N, K), 0.02, 32 + N)
    _gemm_check(fmt, A, B, "f32", f"{fmt} {shape}")


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_all_positive_long_k(fmt):
    M, N, K = 48, 80, 12288
    A = synth.uniform_positive((M, K), 0.5, 6.0, 21)
    B = synth.uniform_positive((N, K), 0.01, 1.0, 22)
    rel = _gemm_check(fmt, A, B, "f32", f"{fmt} all-positive")
    print(f"{fmt}: max |err| / sum|ab| = {rel:.3g}")


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_then_gemm_bf16_out(fmt):
    """GPU quantize feeding the GPU GEMM, bf16 output, a 2-tile-by-3 shape."""
    M, N, K = 512, 768, 1024
    A = synth.normal((M, K), 1.0, 61)
    B = synth.normal((N, K), 0.02, 62)
    qa = mx.quantize(dev_bf16(A), fmt)
    qb = mx.quantize(dev_bf16(B), fmt)
    got = host(mx.gemm(qa, qb, torch.bfloat16).float())
    f = ORC_FMT[fmt]
    C, S = orc.gemm(f, f, M, N, K, host(qa.codes), host(qa.scales), 1.0, host(qb.codes), host(qb.scales), 1.0)
    check_gemm(got, C, S, "bf16", f"{fmt} quantize+gemm")


@pytest.mark.parametrize("wl,fmt", [("f2a", "mxfp8_e5m2"), ("f2b", "mxfp6_e3m2")])
def test_bench_step_configuration_every_element(wl, fmt):
    """The step bench.py times, at its full size (4608 x 9216 x 3072): both
    operands quantized on the GPU, every code and scale equal to the
    oracle's, then the GEMM with bf16 output, every output within the
    bound."""
    A, B = synth.workload(wl)
    M, K = A.shape
    N = B.shape[0]
    qa = mx.quantize(dev_bf16(A), fmt)
    qb = mx.quantize(dev_bf16(B), fmt)
    got = host(mx.gemm(qa, qb, torch.bfloat16).float())
    f = ORC_FMT[fmt]
    oa = orc.quantize(f, A)
    ob = orc.quantize(f, B)
    for q, o, what in ((qa, oa, "A"), (qb, ob, "B")):
        assert np.array_equal(host(q.codes), o[0]), f"{wl}: {what} codes differ"
        assert np.array_equal(host(q.scales), o[1]), f"{wl}: {what} scales differ"
    C, S = orc.gemm(f, f, M, N, K, oa[0], oa[1], 1.0, ob[0], ob[1], 1.0)
    check_gemm(got, C, S, "bf16", f"{wl} bench step")
