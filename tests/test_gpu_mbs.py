"""GPU parity for MXFP4 with static macro-block scaling (MBS), over 32-element
base blocks (MXFP4-MBS) and over the 16-element base blocks the gist.science
summary prints (MXFP4-MBS16): quantize bit for bit against the oracle (every
bf16 value as a macro maximum; every reachable macro factor with every element
value near the top of its block; ragged and special inputs), dequantize bit
for bit, and both GEMM kernels (the 256 x 256-tile kernel and the 128 x 128
one for K % 256 = 128 or ragged shapes) within the oracle's bound, up to the
full MLP-down shape with every output checked."""
import numpy as np
import pytest
import torch

import microscaling_precision_quantization_amd as mx
import oracle as orc
import synth
from gpu_helpers import check_gemm, dev_bf16, dev_u8, host, require_gpu

pytestmark = pytest.mark.gpu

class V:
    """One MBS variant: names and base block."""

    def __init__(self, name, ofmt, mfmt, base):
        self.name, self.F, self.mfmt, self.base = name, ofmt, mfmt, base


VARIANTS = [V("mxfp4_mbs", orc.FMT_MXFP4_MBS, mx.MX_FMT_MXFP4_MBS, 32),
            V("mxfp4_mbs16", orc.FMT_MXFP4_MBS16, mx.MX_FMT_MXFP4_MBS16, 16)]


@pytest.fixture(params=VARIANTS, ids=["base32", "base16"])
def v(request):
    return request.param


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _gpu_mbs(bits, v):
    q = mx.quantize(dev_bf16(bits), v.name)
    torch.cuda.synchronize()
    return host(q.codes), host(q.scales)


def _assert_equal(bits, v, what=""):
    rows, cols = bits.shape
    c, s = _gpu_mbs(bits, v)
    oc, os_, _ = orc.quantize(v.F, bits)
    ge, gm = orc.mbs_planes(s, rows, cols, v.base)
    oe, om = orc.mbs_planes(os_, rows, cols, v.base)
    bad = np.argwhere(gm != om)
    assert bad.size == 0, f"{what}: {len(bad)} macro bytes differ, first {bad[0]}: gpu {gm[tuple(bad[0])]} oracle {om[tuple(bad[0])]}"
    bad = np.argwhere(ge != oe)
    assert bad.size == 0, f"{what}: {len(bad)} scales differ, first {bad[0]}: gpu {ge[tuple(bad[0])]} oracle {oe[tuple(bad[0])]}"
    bad = np.argwhere(c != oc)
    assert bad.size == 0, f"{what}: {len(bad)} code bytes differ, first {bad[0]}: gpu {c[tuple(bad[0])]:#x} oracle {oc[tuple(bad[0])]:#x}"
    return c, s


def test_every_bf16_as_macro_maximum(v):
    """Each finite nonzero bf16 value (both signs) heads a macro block whose
    other 127 elements are seeded values below it in magnitude."""
    allbits = np.arange(1, 0x7F80, dtype=np.uint16)
    alpha = np.concatenate([allbits, allbits | 0x8000])
    a = synth.bf16_to_f32(alpha).astype(np.float64)
    rng = np.random.default_rng(901)
    fill = np.abs(a)[:, None] * rng.uniform(-1, 1, (alpha.size, 127)) * rng.choice(
        [1.0, 0.5, 0.125, 2.0**-6], (alpha.size, 127))
    x = np.concatenate([alpha[:, None], synth.bf16_bits(fill)], axis=1)
    # the maximum's position varies over the 4 blocks
    shift = rng.integers(0, 128, alpha.size)
    x = np.stack([np.roll(row, s) for row, s in zip(x, shift)])
    _assert_equal(x, v, "macro maxima")


def _factor_grid_rows():
    """For every significand S in 128..255 of the macro maximum alpha (which
    fixes the factor) and a spread of exponents: blocks [alpha, x_1..x_31]
    whose x run over every bf16 magnitude from alpha down 12 binades, both
    signs, so each block's scale is the maximum's and every element decision
    near the top of the E2M1 grid (ties included) is exercised."""
    rows = []
    for e in (-133, -126, -120, -3, 0, 7, 60, 120, 126):
        for S in range(128, 256):
            a = S * 2.0 ** (e - 7)
            if a > 3.3e38:
                continue
            ab = synth.bf16_bits(np.array([a]))[0]
            av = float(synth.bf16_to_f32(np.array([ab]))[0])
            if av == 0:
                continue
            lo = av * 2.0**-12
            allv = synth.bf16_to_f32(np.arange(0, 0x7F80, dtype=np.uint16)).astype(np.float64)
            sel = np.arange(0, 0x7F80, dtype=np.uint16)[(allv <= av) & (allv >= lo)]
            sel = np.concatenate([sel, sel | 0x8000, [0, 0x8000]]).astype(np.uint16)
            pad = (-len(sel)) % 124
            sel = np.concatenate([sel, np.zeros(pad, np.uint16)]).reshape(-1, 4, 31)
            blk = np.concatenate([np.full((sel.shape[0], 4, 1), ab, np.uint16), sel], axis=2)
            rows.append(blk.reshape(-1, 128))
    return np.concatenate(rows)


def test_every_factor_every_element_near_the_top(v):
    x = _factor_grid_rows()
    _, s = _assert_equal(x, v, "factor grid")
    _, m = orc.mbs_planes(s, x.shape[0], 128, v.base)
    assert len(np.unique(m)) >= 120  # the reachable factors


@pytest.mark.parametrize("shape", [(1, 128), (3, 384), (257, 1152), (64, 4096), (1000, 256)])
def test_ragged_shapes(shape, v):
    x = synth.laplace_outlier_channels(shape, seed=911 + shape[0], channel_seed=912, frac=0.01,
                                       factor=100.0)
    _assert_equal(x, v, f"laplace {shape}")


def test_special_blocks(v):
    g = np.random.Generator(np.random.PCG64(913))
    x = synth.bf16_bits(g.normal(0, 1, (10, 256)))
    x[0, :128] = 0                       # all-zero macro block
    x[1, :128] = 0x8000                  # -0
    x[2, :128] = g.integers(1, 0x80, 128).astype(np.uint16)  # subnormals only
    x[3, 5] = 0x7F80                     # Inf: m = 0, that block NaN-scaled
    x[4, 200] = 0xFFC0                   # NaN in the second macro block
    x[5, 64:96] = 0x0001
    x[6, :] = 0x7F7F                     # largest finite bf16 everywhere
    x[7, :] = 0xFF7F
    x[8, 0] = 0x4040                     # 3.0 heads its macro block (factor 1)
    x[9, 130] = 0x4140                   # 12.0
    _assert_equal(x, v, "specials")


def test_workload_rows(v):
    """256 rows of the MXFP4 MLP-down activations (Laplace with outlier
    channels), all 12288 columns."""
    A, _ = synth.workload("mxfp4_dit_mlp_down_4608x12288x3072", rows_a=256, rows_b=8)
    _assert_equal(A, v, "workload rows")


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_dequantize_codes_scales_factors(out, v):
    rng = np.random.default_rng(921)
    rows, cols = 256, 512
    codes = np.tile(np.arange(256, dtype=np.uint8), (rows, 1))
    e8 = np.repeat(np.arange(256, dtype=np.uint8).reshape(256, 1), cols // v.base, axis=1)
    mac = rng.integers(0, 256, (rows, cols // 128), dtype=np.uint8)
    mac[:, 0] = 0
    mac[:, 1] = 255
    scales = np.concatenate([e8.reshape(-1), mac.reshape(-1)])
    q = mx.QTensor(v.mfmt, rows, cols, dev_u8(codes), dev_u8(scales), None)
    y = mx.dequantize(q, torch.float32 if out == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    od = orc.OUT_F32 if out == "f32" else orc.OUT_BF16
    ref = orc.dequantize(v.F, codes, scales, 1.0, rows, cols, od)
    if out == "f32":
        got = host(y)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got.view(np.uint32)[~nan], ref.view(np.uint32)[~nan])
    else:
        got = host(y.view(torch.int16)).view(np.uint16)
        nan = ((ref & 0x7F80) == 0x7F80) & ((ref & 0x7F) != 0)
        gnan = ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0)
        assert np.array_equal(gnan, nan)
        assert np.array_equal(got[~nan], ref[~nan])


def _qt(v, codes, scales, rows, cols):
    return mx.QTensor(v.mfmt, rows, cols, dev_u8(codes), dev_u8(scales), None)


def _gemm_check(A, B, out, v, what):
    M, K = A.shape
    N = B.shape[0]
    ca, sa, _ = orc.quantize(v.F, A)
    cb, sb, _ = orc.quantize(v.F, B)
    C, S = orc.gemm(v.F, v.F, M, N, K, ca, sa, 1.0, cb, sb, 1.0)
    got = host(mx.gemm(_qt(v, ca, sa, M, K), _qt(v, cb, sb, N, K),
                       torch.float32 if out == "f32" else torch.bfloat16).float())
    return check_gemm(got, C, S, out, what)


# K % 256 = 0 takes the 256 x 256-tile kernel; K % 256 = 128 takes the
# 128 x 128 one. Both see ragged M and N.
@pytest.mark.parametrize("shape", [(256, 128, 256), (200, 72, 512), (1, 1, 128), (300, 520, 768),
                                   (257, 255, 384), (513, 40, 2560), (520, 300, 1152)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemm_shapes(shape, out, v):
    M, N, K = shape
    A = synth.laplace_outlier_channels((M, K), seed=931 + M, channel_seed=932, frac=0.01, factor=50.0)
    B = synth.normal((N, K), 0.02, 933 + N)
    _gemm_check(A, B, out, v, f"{v.name} {shape} {out}")


@pytest.mark.parametrize("K", [12288, 12288 + 128])
def test_gemm_all_positive_long_k(K, v):
    M, N = 48, 80
    A = synth.uniform_positive((M, K), 0.5, 6.0, 941)
    B = synth.uniform_positive((N, K), 0.01, 1.0, 942)
    rel = _gemm_check(A, B, "f32", v, f"{v.name} all-positive")
    print(f"{v.name} K={K}: max |err| / sum|ab| = {rel:.3g}")


def test_quantize_then_gemm_bf16_out(v):
    """GPU quantize feeding the GPU GEMM, bf16 output, several tiles."""
    M, N, K = 512, 384, 1024
    A = synth.laplace_outlier_channels((M, K), seed=951, channel_seed=952, frac=0.01, factor=100.0)
    B = synth.normal((N, K), 0.02, 953)
    qa = mx.quantize(dev_bf16(A), v.name)
    qb = mx.quantize(dev_bf16(B), v.name)
    got = host(mx.gemm(qa, qb, torch.bfloat16).float())
    C, S = orc.gemm(v.F, v.F, M, N, K, host(qa.codes), host(qa.scales), 1.0, host(qb.codes),
                    host(qb.scales), 1.0)
    check_gemm(got, C, S, "bf16", f"{v.name} quantize+gemm")


def test_full_size_every_element(v):
    """The MLP-down shape (4608 x 12288 activations, 3072 x 12288 weights) in
    the benchmark's launch configuration: GPU quantize of both operands, the
    GEMM with bf16 output, every output against the oracle (which
    re-quantizes the same inputs itself)."""
    A, B = synth.workload("mxfp4_dit_mlp_down_4608x12288x3072")
    M, K = A.shape
    N = B.shape[0]
    qa = mx.quantize(dev_bf16(A), v.name)
    qb = mx.quantize(dev_bf16(B), v.name)
    c = mx.gemm(qa, qb, torch.bfloat16)
    torch.cuda.synchronize()
    ca, sa, _ = orc.quantize(v.F, A)
    cb, sb, _ = orc.quantize(v.F, B)
    assert np.array_equal(host(qa.codes), ca) and np.array_equal(host(qa.scales), sa)
    assert np.array_equal(host(qb.codes), cb) and np.array_equal(host(qb.scales), sb)
    C, S = orc.gemm(v.F, v.F, M, N, K, ca, sa, 1.0, cb, sb, 1.0)
    check_gemm(host(c.float()), C, S, "bf16", f"{v.name} full size")
