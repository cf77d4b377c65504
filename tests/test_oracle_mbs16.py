"""Pins for the oracle's MXFP4-MBS16: macro-block scaling (static variant) as
the gist.science summary of "Unveiling the Potential of Quantization with
MXFP4", section 2.B, prints it -- a factor with an 8-bit mantissa per 1 x 128
macro block, the main quantization in 1 x 16 blocks (E2M1 codes, one E8M0
scale per 16 elements). Checked against brute force over exact rationals,
against the pinned MXFP4 path (16-element blocks padded to 32 with zeros),
closed forms and invariants, not against the oracle's own formulas.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as orc
import synth

F = orc.FMT_MXFP4_MBS16
E2M1 = [Fraction(v) for v in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]


def _mbs16(x_bits):
    rows, cols = x_bits.shape
    codes, scales, _ = orc.quantize(F, x_bits)
    e8, mac = orc.mbs_planes(scales, rows, cols, block=16)
    return codes, e8, mac


def _nibbles(codes):
    return np.stack([codes & 0xF, codes >> 4], -1).reshape(codes.shape[0], -1)


def _frac_bf16(bits):
    return Fraction(float(synth.bf16_to_f32(np.array([bits], np.uint16))[0]))


def test_storage_bits():
    """4 bits per code, 8 per 16-element E8M0 scale, 8 per 128-element macro
    mantissa: 4.5625 bits per element."""
    assert orc.storage_bytes(F, 4, 1024) * 8 / (4 * 1024) == 4 + 8 / 16 + 8 / 128


def _brute_macro_mantissa(alpha):
    """j of the smallest 6 (1 + j/256) 2^k >= alpha, by search."""
    if alpha == 0:
        return 0
    k = -140
    while Fraction(6) * (Fraction(2) ** k) * Fraction(511, 256) < alpha:
        k += 1
    for j in range(256):
        if Fraction(6) * (1 + Fraction(j, 256)) * Fraction(2) ** k >= alpha:
            return j
    raise AssertionError("unreachable")


def _brute_block(xs, f):
    """Scale byte and codes of one base block of x / f by brute force: the
    smallest n with amax <= 6 f 2^n, then the nearest of all 8 magnitudes."""
    amax = max(abs(v) for v in xs)
    if amax == 0:
        E = 0
    else:
        n = -200
        while amax > 6 * f * Fraction(2) ** n:
            n += 1
        E = min(max(n + 127, 0), 254)
    D = f * Fraction(2) ** (E - 127)
    out = []
    for v in xs:
        a = abs(v)
        best = None
        for c in range(8):
            d = abs(a - E2M1[c] * D)
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                best = (d, c)
        out.append(best[1])
    return E, out


def test_brute_force_small():
    """Seeded Laplace rows with outliers, zeros, -0 and subnormals: macro
    mantissas, 16-block scales and codes equal a brute-force search over
    exact rationals (nearest of all 8 magnitudes, ties to the even code)."""
    rows, cols = 4, 256
    x = synth.laplace_outlier_channels((rows, cols), seed=1811, channel_seed=1812, frac=0.02,
                                       factor=100.0).copy()
    x[3, :128] = 0
    x[3, 5] = 0x8000          # -0
    x[3, 7] = 0x0003          # subnormal
    x[3, 40] = 0x8001
    x[2, 130:135] = synth.bf16_bits(np.array([5.0, -3.0, 0.75, 1e-3, 2.5]))
    codes, e8, mac = _mbs16(x)
    nib = _nibbles(codes)
    for r in range(rows):
        for q in range(cols // 128):
            xs = [_frac_bf16(b) for b in x[r, 128 * q:128 * (q + 1)]]
            m = _brute_macro_mantissa(max(abs(v) for v in xs))
            assert mac[r, q] == m, (r, q)
            f = 1 + Fraction(m, 256)
            for b in range(8):
                E, cs = _brute_block(xs[16 * b:16 * (b + 1)], f)
                assert e8[r, 8 * q + b] == E, (r, q, b)
                lo = 128 * q + 16 * b
                got = nib[r, lo:lo + 16]
                sign = (x[r, lo:lo + 16] >> 15).astype(np.uint8)
                assert np.array_equal(got, np.array(cs, np.uint8) | (sign << 3)), (r, q, b)


def _pad16(x):
    """Each 16-element block followed by 16 zeros: MXFP4's 32-block scale of
    the padded row is the 16-block's own MX scale."""
    rows, cols = x.shape
    y = np.zeros((rows, cols // 16, 32), np.uint16)
    y[:, :, :16] = x.reshape(rows, cols // 16, 16)
    return y.reshape(rows, 2 * cols)


def test_reduces_to_16_element_mx_when_mantissa_is_zero():
    """m = 0 means f = 1: every 16-block then quantizes by the plain MX rule,
    which the pinned MXFP4 path computes on the row padded to 32-blocks.
    (a) every macro maximum is 3 * 2^k, whose factor is 1; (b) random rows:
    every macro block that got m = 0 matches."""
    rng = np.random.default_rng(1821)
    v = rng.uniform(-1, 1, (8, 512))
    v[:, ::128] = 3.0 * np.exp2(rng.integers(1, 6, (8, 4)))
    for x, check_all in ((synth.bf16_bits(v), True), (synth.normal((64, 512), 1.0, seed=1822), False)):
        codes, e8, mac = _mbs16(x)
        c4, s4, _ = orc.quantize(orc.FMT_MXFP4, _pad16(x))
        n4 = _nibbles(c4).reshape(x.shape[0], -1, 32)[:, :, :16].reshape(x.shape[0], -1)
        nm = _nibbles(codes)
        if check_all:
            assert np.all(mac == 0)
        zero = np.argwhere(mac == 0)
        assert len(zero) > 0
        for r, q in zero:
            assert np.array_equal(nm[r, 128 * q:128 * (q + 1)], n4[r, 128 * q:128 * (q + 1)])
            assert np.array_equal(e8[r, 8 * q:8 * (q + 1)], s4[r, 8 * q:8 * (q + 1)])


def test_macro_max_rounds_up_onto_grid_exhaustive():
    """Every positive finite bf16 value as the only nonzero element of a macro
    block: it encodes as E2M1 6 and dequantizes to the smallest
    6 (1 + j/256) 2^k >= it (E > 0); the other 16-blocks are zero."""
    amax = np.arange(1, 0x7F80, dtype=np.uint16)
    x = np.zeros((amax.size, 128), np.uint16)
    x[:, 37] = amax  # block 2 of the macro
    codes, e8, mac = _mbs16(x)
    a = synth.bf16_to_f32(amax).astype(np.float64)
    E = e8[:, 2].astype(np.int64)
    m = mac[:, 0].astype(np.int64)
    code = _nibbles(codes)[:, 37]
    deq = 6.0 * np.exp2(E - 127.0) * (1.0 + m / 256.0)
    assert np.all(deq >= a)
    inner = E > 0
    assert np.all(code[inner] == 7)
    below = np.where(m > 0, 6.0 * np.exp2(E - 127.0) * (1.0 + (m - 1) / 256.0),
                     6.0 * np.exp2(E - 128.0) * (1.0 + 255 / 256.0))
    assert np.all(below[inner] < a[inner])
    for b in (0, 1, 3, 4, 5, 6, 7):
        assert np.all(e8[:, b] == 0)
    assert np.all(np.delete(_nibbles(codes), 37, axis=1) == 0)


def test_nonfinite():
    """A macro block holding Inf gets m = 0; the 16-block with Inf gets the
    E8M0 NaN byte and zero codes, its neighbours are 16-element MX blocks;
    the next macro block is unaffected."""
    x = synth.normal((1, 256), 1.0, seed=1831).copy()
    x[0, 70] = 0x7F80
    codes, e8, mac = _mbs16(x)
    assert mac[0, 0] == 0
    assert e8[0, 4] == 255 and np.all(_nibbles(codes)[0, 64:80] == 0)
    c4, s4, _ = orc.quantize(orc.FMT_MXFP4, _pad16(x))
    assert np.array_equal(e8[0, :4], s4[0, :4])
    assert mac[0, 1] == _brute_macro_mantissa(max(abs(_frac_bf16(b)) for b in x[0, 128:]))


def test_dequant_is_exact():
    """Random codes, exponents and macro mantissas: the fp32 output is exactly
    e * 2^(E-127) * (1 + m/256) with E per 16 elements, and the bf16 output is
    torch's nearest-even rounding of it."""
    rng = np.random.default_rng(1841)
    rows, cols = 8, 512
    codes = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    e8 = rng.integers(1, 254, (rows, cols // 16), dtype=np.uint8)
    mac = rng.integers(0, 256, (rows, cols // 128), dtype=np.uint8)
    scales = np.concatenate([e8.reshape(-1), mac.reshape(-1)])
    y = orc.dequantize(F, codes, scales, 1.0, rows, cols)
    yb = orc.dequantize(F, codes, scales, 1.0, rows, cols, orc.OUT_BF16)
    nib = _nibbles(codes)
    mag = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    e = np.where(nib & 8, -1.0, 1.0) * mag[nib & 7]
    want = (e * np.exp2(np.repeat(e8.astype(np.float64), 16, 1) - 127)
            * (1 + np.repeat(mac.astype(np.float64), 128, 1) / 256))
    with np.errstate(over="ignore"):
        w32 = want.astype(np.float32)
    exact = np.isfinite(w32) & (w32.astype(np.float64) == want)
    assert exact.mean() > 0.99
    assert np.array_equal(y[exact], w32[exact])
    assert np.all(np.isinf(y[~exact]))
    tb = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(yb, tb)


def test_gemm_matches_float64_matmul():
    M, N, K = 24, 40, 512
    a = synth.laplace_outlier_channels((M, K), seed=1851, channel_seed=1852, frac=0.01, factor=50.0)
    b = synth.normal((N, K), 0.02, seed=1853)
    ca, sa, _ = orc.quantize(F, a)
    cb, sb, _ = orc.quantize(F, b)
    C, S = orc.gemm(F, F, M, N, K, ca, sa, 1.0, cb, sb, 1.0)
    da = orc.dequantize(F, ca, sa, 1.0, M, K).astype(np.float64)
    db = orc.dequantize(F, cb, sb, 1.0, N, K).astype(np.float64)
    assert np.all(np.abs(C - da @ db.T) <= K * 2.0**-50 * S)
    assert np.allclose(S, np.abs(da) @ np.abs(db).T, rtol=2.0**-40, atol=0)


def _qsnr(x, y):
    return 10 * np.log10(np.sum(x * x) / np.sum((x - y) ** 2))


def test_lowers_error_on_outlier_data():
    """The direction the summary reports, on outlier-channel data: MBS with
    16-element blocks reproduces the tensor better than MBS over 32-element
    blocks, which beats plain MXFP4."""
    rows, cols = 64, 1024
    x = synth.laplace_outlier_channels((rows, cols), seed=1861, channel_seed=1862, frac=0.005,
                                       factor=100.0)
    xf = synth.bf16_to_f32(x).astype(np.float64)
    q = {}
    for name, fmt in (("mxfp4", orc.FMT_MXFP4), ("mbs32", orc.FMT_MXFP4_MBS), ("mbs16", F)):
        c, s, _ = orc.quantize(fmt, x)
        q[name] = _qsnr(xf, orc.dequantize(fmt, c, s, 1.0, rows, cols))
    assert q["mbs16"] > q["mbs32"] > q["mxfp4"] + 0.5, q


def test_argument_checks():
    x = synth.normal((2, 96), 1.0, seed=1871)
    with pytest.raises(ValueError):
        orc.quantize(F, x)  # 96 is not a multiple of 128
