"""Pins for the oracle's quantize and dequantize.

Brute force over every E2M1 code and every E8M0 exponent on tiny tensors, the
printed storage figures (4.25 bits per element, the KV-cache example), the
nearest-value property on random blocks (checked against the printed value
set), and invariants for the NVFP4 sequence.
"""
import math

import numpy as np
import pytest

import synth

FP4_VALUES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _bits(vals):
    """Exact float -> bf16 bits (asserting exactness)."""
    f = np.asarray(vals, dtype=np.float64)
    b = synth.bf16_bits(f)
    assert np.array_equal(synth.bf16_to_f32(b).astype(np.float64), f), "not exact in bf16"
    return b


def _is_bf16_exact(v):
    f = np.float64(v)
    return float(synth.bf16_to_f32(synth.bf16_bits(np.array([f])))[0]) == f


def _unpack_fp4(codes):
    codes = np.asarray(codes, np.uint8)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = codes & 0xF
    out[..., 1::2] = codes >> 4
    return out


def test_mxfp4_brute_force_all_codes_all_exponents(orc, pages):
    """Every E2M1 code c with every reachable exponent E: a block holding the
    anchor 6 * 2^(E-127) and c's value times 2^(E-127) quantizes to scale E and
    codes (7, c); the page's decode x = 2^(E-127) * x_elem returns the input."""
    vals = pages["e2m1_values"]["values"]
    rows = []
    expect = []
    for E in range(0, 253):
        s = 2.0 ** (E - 127)
        for c in range(16):
            v = (-1 if c & 8 else 1) * vals[c & 7] * s
            row = np.zeros(32)
            row[0] = 6.0 * s
            row[1] = v
            row[2:] = 0.0
            rows.append(row)
            expect.append((E, c))
    x = _bits(np.array(rows))
    codes, scales, _ = orc.quantize(orc.FMT_MXFP4, x)
    c = _unpack_fp4(codes)
    for r, (E, code) in enumerate(expect):
        assert scales[r, 0] == E
        assert c[r, 0] == 7 and c[r, 1] == code, (E, code, c[r, :2])
        assert np.all(c[r, 2:] == 0)
    y = orc.dequantize(orc.FMT_MXFP4, codes, scales, 1.0, len(rows), 32)
    assert np.array_equal(y.astype(np.float64), synth.bf16_to_f32(x).astype(np.float64))


def test_mxfp4_top_exponent(orc):
    # The largest finite bf16 gives E = 253 (never 254, never the NaN code).
    x = np.zeros((1, 32), np.uint16)
    x[0, 0] = 0x7F7F
    x[0, 1] = _bits([3.0 * 2.0**126])[0]
    codes, scales, _ = orc.quantize(orc.FMT_MXFP4, x)
    assert scales[0, 0] == 253
    c = _unpack_fp4(codes)[0]
    assert c[0] == 6 and c[1] == 5  # 3.98 -> 4 (code 6); 3.0 -> code 5


def test_dequantize_all_codes_all_exponents(orc, pages):
    """All 16 codes x all 256 E8M0 bytes through dequantize (fp32 and bf16 out)."""
    vals = pages["e2m1_values"]["values"]
    codes = np.zeros((256, 16), np.uint8)
    for c in range(16):
        codes[:, c // 2] |= np.uint8(c << (4 * (c % 2)))
    codes = codes[:, :8].copy()
    codes = np.concatenate([codes, np.zeros((256, 8), np.uint8)], axis=1)  # 32 elements
    scales = np.arange(256, dtype=np.uint8).reshape(256, 1)
    y = orc.dequantize(orc.FMT_MXFP4, codes, scales, 1.0, 256, 32)
    yb = orc.dequantize(orc.FMT_MXFP4, codes, scales, 1.0, 256, 32, out=orc.OUT_BF16)
    for E in range(256):
        for c in range(16):
            got = float(y[E, c])
            if E == 255:
                assert math.isnan(got)
                continue
            want = (-1 if c & 8 else 1) * vals[c & 7] * 2.0 ** (E - 127)
            want32 = float(np.float64(want).astype(np.float32))  # overflow -> inf
            assert got == want32 and math.copysign(1, got) == math.copysign(1, want32), (E, c)
            gb = float(synth.bf16_to_f32(np.array([yb[E, c]], np.uint16))[0])
            if math.isinf(want32) or abs(want32) > 3.3895e38:
                assert math.isinf(gb)
            else:
                assert gb == want32


def test_mxfp8_brute_force(orc):
    """Every finite E4M3 code at every exponent where it is exact in bf16."""
    rows, expect = [], []
    for E in range(0, 247, 3):
        s = 2.0 ** (E - 127)
        for code in range(256):
            v = orc.e4m3_value(code)
            if math.isnan(v) or not _is_bf16_exact(v * s) or not _is_bf16_exact(448 * s):
                continue
            row = np.zeros(32)
            row[0] = 448.0 * s
            row[1] = v * s
            rows.append(row)
            expect.append((E, code))
    x = _bits(np.array(rows))
    codes, scales, _ = orc.quantize(orc.FMT_MXFP8, x)
    for r, (E, code) in enumerate(expect):
        assert scales[r, 0] == E and codes[r, 0] == 0x7E and codes[r, 1] == code, (E, code)
    y = orc.dequantize(orc.FMT_MXFP8, codes, scales, 1.0, len(rows), 32)
    assert np.array_equal(y.astype(np.float64), synth.bf16_to_f32(x).astype(np.float64))


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_mx_quantize_is_nearest_on_random_blocks(orc, pages, fmt):
    """Random outlier-heavy blocks: every code is a nearest grid value at the
    block's scale, and the scale obeys the (3, 6] / (224, 448] range."""
    f = orc.FMT_MXFP4 if fmt == "mxfp4" else orc.FMT_MXFP8
    x = synth.normal_outliers((64, 256), 1.0, 5, 0.02, 50.0)
    x[3, :32] = 0  # an all-zero block
    x[5, 32:64] = synth.bf16_bits(np.full(32, 1e-39))  # subnormal bf16 block
    codes, scales, _ = orc.quantize(f, x)
    if fmt == "mxfp4":
        grid = np.array(FP4_VALUES)
        c = _unpack_fp4(codes)
        mag = grid[c & 7]
        sign = np.where(c & 8, -1.0, 1.0)
        emax, lo = 6.0, 3.0
    else:
        grid = np.array([orc.e4m3_value(k) for k in range(0x7F)])
        mag = grid[codes & 0x7F]
        sign = np.where(codes & 0x80, -1.0, 1.0)
        emax, lo = 448.0, 224.0
    xf = synth.bf16_to_f32(x).astype(np.float64)
    s = 2.0 ** (scales.astype(np.float64) - 127)
    s_el = np.repeat(s, 32, axis=1)
    v = np.abs(xf) / s_el
    err = np.abs(v - mag)
    best = np.min(np.abs(v[..., None] - grid[None, None, :]), axis=-1)
    assert np.all(err == best)
    assert np.all(np.signbit(sign) == np.signbit(xf))
    amax = np.abs(xf).reshape(64, -1, 32).max(axis=-1)
    scaled = amax / s
    assert np.all(scaled <= emax)
    assert np.all((scaled > lo) | (scales == 0))
    assert scales[3, 0] == 0 and np.all(mag[3, :32] == 0)


def test_storage_matches_printed_figures(orc, pages):
    kv = pages["kv_cache_example"]
    n = 2 * kv["layers"] * kv["kv_heads"] * kv["head_dim"]
    assert n * 2 == kv["bytes_per_token"]["bf16"]
    assert n * 1 == kv["bytes_per_token"]["fp8"]
    assert orc.storage_bytes(orc.FMT_MXFP4, 1, n) == kv["bytes_per_token"]["mxfp4"]
    assert orc.storage_bytes(orc.FMT_MXFP4, 1, n) / n == kv["mxfp4_bytes_per_element"]
    assert round(100 * (1 - kv["mxfp4_bytes_per_element"] / 2), 1) == kv["reduction_vs_bf16_percent"]
    bits = pages["format_table"]["effective_bits"]
    R, C = 64, 4096
    assert orc.storage_bytes(orc.FMT_MXFP4, R, C) * 8 / (R * C) == bits["mxfp4"]
    nv = (orc.storage_bytes(orc.FMT_NVFP4, R, C) - 4) * 8 / (R * C)
    assert bits["nvfp4_min"] <= nv <= bits["nvfp4_max"]
    assert orc.storage_bytes(orc.FMT_MXFP8, R, C) * 8 / (R * C) == 8.25
    # The quantizer's outputs have exactly these sizes.
    x = synth.normal((R, C), 1.0, 9)
    codes, scales, _ = orc.quantize(orc.FMT_MXFP4, x)
    assert codes.nbytes + scales.nbytes == orc.storage_bytes(orc.FMT_MXFP4, R, C)


def test_fp4_packing_even_element_low_nibble(orc):
    x = np.zeros((1, 32), np.uint16)
    x[0, 0] = _bits([6.0])[0]
    x[0, 3] = _bits([-1.0])[0]
    codes, scales, _ = orc.quantize(orc.FMT_MXFP4, x)
    assert scales[0, 0] == 127
    assert codes[0, 0] == 0x07 and codes[0, 1] == 0xA0


def test_non_finite_blocks(orc):
    x = synth.normal((2, 64), 1.0, 1)
    x[0, 5] = 0x7FC0  # NaN in block 0 of row 0
    x[1, 40] = 0xFF80  # -Inf in block 1 of row 1
    for f in (orc.FMT_MXFP4, orc.FMT_MXFP8):
        codes, scales, _ = orc.quantize(f, x)
        assert scales[0, 0] == 255 and scales[1, 1] == 255
        assert scales[0, 1] != 255 and scales[1, 0] != 255
        per = 16 if f == orc.FMT_MXFP4 else 32
        assert np.all(codes[0, :per] == 0) and np.all(codes[1, per:] == 0)
    codes, scales, ts = orc.quantize(orc.FMT_NVFP4, x)
    assert math.isnan(ts) and np.all(scales == 0x7F) and np.all(codes == 0)


def test_nvfp4_tensor_scale_and_anchor_block(orc):
    x = synth.student_t((32, 256), 4.0, 12)
    codes, scales, ts = orc.quantize(orc.FMT_NVFP4, x)
    xf = synth.bf16_to_f32(x)
    T = float(np.abs(xf).max())
    assert ts == float(np.float32(T) / np.float32(2688.0))
    i = int(np.argmax(np.abs(xf)))
    r, col = divmod(i, 256)
    assert scales[r, col // 16] == 0x7E  # 448
    c = _unpack_fp4(codes)
    assert c[r, col] & 7 == 7  # the tensor amax encodes as 6
    # Every block scale is a finite, non-negative E4M3 code.
    assert np.all(scales <= 0x7E)


def test_nvfp4_grid_values_round_trip(orc):
    """With T = 2688 the tensor scale is exactly 1; blocks built from E4M3
    scale values times E2M1 values come back unchanged."""
    g = np.random.Generator(np.random.PCG64(4))
    sb_codes = g.integers(8, 0x7E, 64)  # normal E4M3 scales
    rows = []
    for k, sc in enumerate(sb_codes):
        s = orc.e4m3_value(int(sc))
        e = g.integers(0, 16, 16)
        blk = np.array([(-1 if v & 8 else 1) * FP4_VALUES[v & 7] for v in e]) * s
        blk[g.integers(0, 16)] = 6.0 * s  # anchor
        rows.append(blk)
    x = np.concatenate(rows).reshape(4, 256)
    x[0, 0] = 2688.0 / 448.0 * 448.0  # keep T = 2688 in the tensor
    x[0, 1:16] = 0.0
    xb = _bits(x)
    codes, scales, ts = orc.quantize(orc.FMT_NVFP4, xb)
    assert ts == 1.0
    y = orc.dequantize(orc.FMT_NVFP4, codes, scales, ts, 4, 256)
    assert np.array_equal(y, synth.bf16_to_f32(xb))


def test_nvfp4_zero_tensor_and_signed_zero(orc):
    x = np.zeros((2, 32), np.uint16)
    x[1, 3] = 0x8000  # -0
    codes, scales, ts = orc.quantize(orc.FMT_NVFP4, x)
    assert ts == 1.0 and np.all(scales == 0)
    c = _unpack_fp4(codes)
    assert c[1, 3] == 8 and np.count_nonzero(c) == 1


def test_nvfp4_reciprocal_form_rarely_differs(orc):
    """The cheaper fp32 form fl(x * fl(1 / fl(s_b s_t))) decides a handful of
    codes differently from the exact quotient; the scales are the same."""
    x = synth.student_t((128, 512), 4.0, 13)
    c1, s1, t1 = orc.quantize(orc.FMT_NVFP4, x)
    c2, s2, t2 = orc.quantize_nvfp4_reciprocal(x)
    assert t1 == t2 and np.array_equal(s1, s2)
    diff = np.count_nonzero(_unpack_fp4(c1) != _unpack_fp4(c2))
    assert diff <= 0.001 * x.size


def _nvfp4_pin_tensors():
    """Student-t rows, an outlier row, a block that s_b rounds to zero, and
    whole tensors at the bottom and top of the bf16 range (where fl(s_b s_t)
    underflows or 1 / fl(s_b s_t) overflows in fp32)."""
    base = synth.student_t((6, 128), 4.0, 31)
    base[1, 5] = synth.bf16_bits(np.array([300.0]))[0]
    base[2, 16:32] = synth.bf16_bits(np.full(16, 1e-6))
    base[3, 32:48] = 0x8000
    f = synth.bf16_to_f32(synth.student_t((4, 128), 4.0, 32)).astype(np.float64)
    out = [base]
    for scale in (2.0**-100, 2.0**-126, 2.0**-131, 1e37):
        out.append(synth.bf16_bits(f * scale))
    return out


def test_nvfp4_codes_nearest_to_exact_quotient(orc):
    """Each NVFP4 code is the E2M1 value nearest the exact rational
    x / (s_b s_t), ties to the even code, saturating at 6, sign copied; a
    zero block scale gives sign-only zeros. Brute force with Fractions over
    every magnitude, for the oracle's own s_b and s_t."""
    from fractions import Fraction
    for x in _nvfp4_pin_tensors():
        codes, scales, ts = orc.quantize(orc.FMT_NVFP4, x)
        c = _unpack_fp4(codes)
        xf = synth.bf16_to_f32(x).astype(np.float64)
        st = Fraction(float(ts))
        for r in range(x.shape[0]):
            for j in range(x.shape[1]):
                v = float(xf[r, j])
                sign = 8 if math.copysign(1.0, v) < 0 else 0
                sb = Fraction(orc.e4m3_value(int(scales[r, j // 16])))
                if v == 0.0 or sb == 0:
                    assert c[r, j] == sign, (r, j)
                    continue
                q = abs(Fraction(v)) / (sb * st)
                best = min(range(8), key=lambda k: (abs(q - Fraction(FP4_VALUES[k])), k & 1))
                assert c[r, j] == sign | best, (r, j, v, float(q), c[r, j], best)


def test_nvfp4_block_scales_match_torch_e4m3(orc):
    """s_b is torch's float8_e4m3fn rounding (nearest-even) of the fp32 value
    amax_b / (6 s_t), clamped at 448 first; s_t = T / 2688 in fp32."""
    import torch
    for x in _nvfp4_pin_tensors():
        codes, scales, ts = orc.quantize(orc.FMT_NVFP4, x)
        xf = synth.bf16_to_f32(x)
        T = np.float32(np.abs(xf).max())
        assert np.float32(ts) == (np.float32(1.0) if T == 0 else T / np.float32(2688.0))
        bamax = np.abs(xf).reshape(x.shape[0], -1, 16).max(axis=2).astype(np.float32)
        r = np.minimum(bamax / (np.float32(6.0) * np.float32(ts)), np.float32(448.0))
        want = torch.from_numpy(r).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(scales, want)
