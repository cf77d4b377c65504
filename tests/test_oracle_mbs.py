"""Pins for the oracle's MXFP4-MBS (macro-block scaling, static variant; the
gist.science summary of "Unveiling the Potential of Quantization with MXFP4",
section 2.B), checked against brute force with exact rationals, closed forms
and the pinned MXFP4 path, not against the oracle's own formulas.

The reading pinned here: a 1 x 128 macro block carries one factor
f = 1 + m/256 (8-bit mantissa m) chosen from the macro maximum alone, such that
the maximum, divided by f, sits at the top of the E2M1 grid; the four
32-element MXFP4 blocks inside then quantize x / f with the standard rule, and
an element's value is e * 2^(E-127) * f.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as orc
import synth

E2M1 = [Fraction(v) for v in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]


def _mbs(x_bits):
    rows, cols = x_bits.shape
    codes, scales, _ = orc.quantize(orc.FMT_MXFP4_MBS, x_bits)
    e8, mac = orc.mbs_planes(scales, rows, cols)
    return codes, e8, mac


def _nibbles(codes):
    return np.stack([codes & 0xF, codes >> 4], -1).reshape(codes.shape[0], -1)


def _frac_bf16(bits):
    v = float(synth.bf16_to_f32(np.array([bits], np.uint16))[0])
    return Fraction(v)


def test_mbs_storage_bits():
    """4 bits per code, 8 per 32-block scale, 8 per 128-element macro
    mantissa: 4.3125 bits per element."""
    assert orc.storage_bytes(orc.FMT_MXFP4_MBS, 4, 1024) * 8 / (4 * 1024) == 4 + 8 / 32 + 8 / 128


def test_mbs_macro_max_rounds_up_onto_grid_exhaustive():
    """Every positive finite bf16 value as the only nonzero element of a macro
    block: it encodes as E2M1 6 and its dequantized value is the smallest
    number of the form 6 (1 + j/256) 2^k (j = 0..255) that is >= it -- the
    outlier is reproduced to within 2^-8, never saturated (E > 0 cases; with E
    clamped at 0 only the no-saturation half holds)."""
    amax = np.arange(1, 0x7F80, dtype=np.uint16)
    x = np.zeros((amax.size, 128), np.uint16)
    x[:, 37] = amax  # block 1 of the macro
    codes, e8, mac = _mbs(x)
    a = synth.bf16_to_f32(amax).astype(np.float64)
    E = e8[:, 1].astype(np.int64)
    m = mac[:, 0].astype(np.int64)
    code = _nibbles(codes)[:, 37]
    deq = 6.0 * np.exp2(E - 127.0) * (1.0 + m / 256.0)  # exact in double
    assert np.all(deq >= a)
    inner = E > 0
    assert np.all(code[inner] == 7)
    # the grid point just below deq is < amax
    below = np.where(m > 0, 6.0 * np.exp2(E - 127.0) * (1.0 + (m - 1) / 256.0),
                     6.0 * np.exp2(E - 128.0) * (1.0 + 255 / 256.0))
    assert np.all(below[inner] < a[inner])
    assert np.all((deq[inner] - a[inner]) <= a[inner] / 255)
    # the other three blocks are zero
    for b in (0, 2, 3):
        assert np.all(e8[:, b] == 0)
    assert np.all(np.delete(_nibbles(codes), 37, axis=1) == 0)


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
    """Scale byte and codes of one 32-block of x / f by brute force."""
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


def test_mbs_brute_force_small():
    """Seeded Laplace rows with outliers, zeros, -0 and subnormals: macro
    mantissas, scales and codes equal a brute-force search over exact
    rationals (nearest of all 8 magnitudes, ties to the even code)."""
    rows, cols = 4, 256
    x = synth.laplace_outlier_channels((rows, cols), seed=811, channel_seed=812, frac=0.02, factor=100.0)
    x = x.copy()
    x[3, :128] = 0
    x[3, 5] = 0x8000          # -0
    x[3, 7] = 0x0003          # subnormal
    x[3, 40] = 0x8001
    x[2, 130:135] = synth.bf16_bits(np.array([5.0, -3.0, 0.75, 1e-3, 2.5]))
    codes, e8, mac = _mbs(x)
    nib = _nibbles(codes)
    for r in range(rows):
        for q in range(cols // 128):
            xs = [_frac_bf16(b) for b in x[r, 128 * q:128 * (q + 1)]]
            m = _brute_macro_mantissa(max(abs(v) for v in xs))
            assert mac[r, q] == m, (r, q)
            f = 1 + Fraction(m, 256)
            for b in range(4):
                E, cs = _brute_block(xs[32 * b:32 * (b + 1)], f)
                assert e8[r, 4 * q + b] == E, (r, q, b)
                got = nib[r, 128 * q + 32 * b:128 * q + 32 * (b + 1)]
                sign = (x[r, 128 * q + 32 * b:128 * q + 32 * (b + 1)] >> 15).astype(np.uint8)
                assert np.array_equal(got, np.array(cs, np.uint8) | (sign << 3)), (r, q, b)


def test_mbs_reduces_to_mxfp4_when_mantissa_is_zero():
    """m = 0 means f = 1: the codes and E8M0 scales are MXFP4's. (a) every
    macro maximum is 3 * 2^k, whose factor is 1; (b) random rows: every macro
    block that got m = 0 matches MXFP4 on its 128 elements."""
    rng = np.random.default_rng(821)
    v = rng.uniform(-1, 1, (8, 512))
    v[:, ::128] = 3.0 * np.exp2(rng.integers(1, 6, (8, 4)))  # above every |v| <= 1
    x = synth.bf16_bits(v)
    c_m, e8, mac = _mbs(x)
    c_4, s_4, _ = orc.quantize(orc.FMT_MXFP4, x)
    assert np.all(mac == 0)
    assert np.array_equal(c_m, c_4) and np.array_equal(e8, s_4)

    x = synth.normal((64, 512), 1.0, seed=822)
    c_m, e8, mac = _mbs(x)
    c_4, s_4, _ = orc.quantize(orc.FMT_MXFP4, x)
    zero = np.argwhere(mac == 0)
    assert len(zero) > 0
    for r, q in zero:
        assert np.array_equal(c_m[r, 64 * q:64 * (q + 1)], c_4[r, 64 * q:64 * (q + 1)])
        assert np.array_equal(e8[r, 4 * q:4 * (q + 1)], s_4[r, 4 * q:4 * (q + 1)])


def test_mbs_nonfinite_macro():
    """A macro block holding Inf gets m = 0; the 32-block with Inf gets the
    E8M0 NaN byte and zero codes, the other blocks are MXFP4's; the next macro
    block is unaffected."""
    x = synth.normal((1, 256), 1.0, seed=831).copy()
    x[0, 70] = 0x7F80
    c_m, e8, mac = _mbs(x)
    c_4, s_4, _ = orc.quantize(orc.FMT_MXFP4, x)
    assert mac[0, 0] == 0
    assert e8[0, 2] == 255 and np.all(c_m[0, 32:48] == 0)
    assert np.array_equal(e8[0, :4], s_4[0, :4])
    assert np.array_equal(c_m[0, :64], c_4[0, :64])
    assert mac[0, 1] == _brute_macro_mantissa(max(abs(_frac_bf16(b)) for b in x[0, 128:]))


def test_mbs_dequant_is_exact():
    """Random codes, exponents and macro mantissas: the fp32 output is exactly
    e * 2^(E-127) * (1 + m/256) and the bf16 output is torch's nearest-even
    rounding of it."""
    rng = np.random.default_rng(841)
    rows, cols = 8, 512
    codes = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    e8 = rng.integers(1, 254, (rows, cols // 32), dtype=np.uint8)
    e8[0, 0] = 0
    mac = rng.integers(0, 256, (rows, cols // 128), dtype=np.uint8)
    scales = np.concatenate([e8.reshape(-1), mac.reshape(-1)])
    y = orc.dequantize(orc.FMT_MXFP4_MBS, codes, scales, 1.0, rows, cols)
    yb = orc.dequantize(orc.FMT_MXFP4_MBS, codes, scales, 1.0, rows, cols, orc.OUT_BF16)
    nib = _nibbles(codes)
    mag = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    e = np.where(nib & 8, -1.0, 1.0) * mag[nib & 7]
    want = (e * np.exp2(np.repeat(e8.astype(np.float64), 32, 1) - 127)
            * (1 + np.repeat(mac.astype(np.float64), 128, 1) / 256))
    with np.errstate(over="ignore"):
        w32 = want.astype(np.float32)
    exact = np.isfinite(w32) & (w32.astype(np.float64) == want)
    assert exact.mean() > 0.99  # the rest overflow fp32
    assert np.array_equal(y[exact], w32[exact])
    assert np.all(np.isinf(y[~exact]))
    tb = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(yb, tb)


def test_mbs_gemm_matches_float64_matmul():
    """The exact-operand GEMM over MBS operands agrees with numpy's float64
    matmul of the dequantized operands within K 2^-50 S, and with all macro
    mantissas 0 it equals the MXFP4 GEMM of the same codes."""
    M, N, K = 24, 40, 512
    a = synth.laplace_outlier_channels((M, K), seed=851, channel_seed=852, frac=0.01, factor=50.0)
    b = synth.normal((N, K), 0.02, seed=853)
    ca, sa, _ = orc.quantize(orc.FMT_MXFP4_MBS, a)
    cb, sb, _ = orc.quantize(orc.FMT_MXFP4_MBS, b)
    C, S = orc.gemm(orc.FMT_MXFP4_MBS, orc.FMT_MXFP4_MBS, M, N, K, ca, sa, 1.0, cb, sb, 1.0)
    da = orc.dequantize(orc.FMT_MXFP4_MBS, ca, sa, 1.0, M, K).astype(np.float64)
    db = orc.dequantize(orc.FMT_MXFP4_MBS, cb, sb, 1.0, N, K).astype(np.float64)
    ref = da @ db.T
    assert np.all(np.abs(C - ref) <= K * 2.0**-50 * S)
    assert np.allclose(S, np.abs(da) @ np.abs(db).T, rtol=2.0**-40, atol=0)

    ea, ma = orc.mbs_planes(sa, M, K)
    eb, mb = orc.mbs_planes(sb, N, K)
    z_a = np.concatenate([ea.reshape(-1), np.zeros(ma.size, np.uint8)])
    z_b = np.concatenate([eb.reshape(-1), np.zeros(mb.size, np.uint8)])
    C0, _ = orc.gemm(orc.FMT_MXFP4_MBS, orc.FMT_MXFP4_MBS, M, N, K, ca, z_a, 1.0, cb, z_b, 1.0)
    C4, _ = orc.gemm(orc.FMT_MXFP4, orc.FMT_MXFP4, M, N, K, ca, ea, 1.0, cb, eb, 1.0)
    assert np.array_equal(C0, C4)


def _qsnr(x, y):
    return 10 * np.log10(np.sum(x * x) / np.sum((x - y) ** 2))


def test_mbs_lowers_error_on_outlier_data():
    """The direction the summary reports: with outlier channels, MBS
    reproduces the tensor with a higher signal-to-noise ratio than MXFP4."""
    rows, cols = 64, 1024
    x = synth.laplace_outlier_channels((rows, cols), seed=861, channel_seed=862, frac=0.005, factor=100.0)
    xf = synth.bf16_to_f32(x).astype(np.float64)
    c4, s4, _ = orc.quantize(orc.FMT_MXFP4, x)
    cm, sm, _ = orc.quantize(orc.FMT_MXFP4_MBS, x)
    q4 = _qsnr(xf, orc.dequantize(orc.FMT_MXFP4, c4, s4, 1.0, rows, cols))
    qm = _qsnr(xf, orc.dequantize(orc.FMT_MXFP4_MBS, cm, sm, 1.0, rows, cols))
    assert qm > q4 + 0.5, (q4, qm)


def test_mbs_argument_checks():
    x = synth.normal((2, 96), 1.0, seed=871)
    with pytest.raises(ValueError):
        orc.quantize(orc.FMT_MXFP4_MBS, x)  # 96 is not a multiple of 128
