"""Pins for the oracle's MXFP8-E5M2 and MXFP6-E3M2 formats (zubnet.ai summary:
MXFP8 is E4M3/E5M2 in 32-blocks; produtoramaxvision format table: MXFP6 is
E3M2 with an E8M0 scale per 32, 6.25 bits per element). E5M2 against torch's
float8_e5m2; E3M2 against the fixed points of its bit-field definition; the
6-bit packing against a hand-packed byte string; the scale rule's ranges."""
import math

import numpy as np
import pytest
import torch

import oracle as orc
import synth


def test_e5m2_decode_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e5m2).to(torch.float64).numpy()
    got = np.array([orc.e5m2_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert orc.e5m2_value(0x7B) == 57344.0 and orc.e5m2_value(0x7C) == math.inf


def test_e5m2_encode_matches_torch_in_range():
    """Every finite E5M2 value, every midpoint between neighbours, and random
    values within +-57344: nearest-even encode equals torch's conversion."""
    vals = np.array([orc.e5m2_value(c) for c in range(0x7C)])
    mids = (vals[:-1] + vals[1:]) / 2
    g = np.random.Generator(np.random.PCG64(8))
    rnd = g.uniform(-57344, 57344, 2000) * np.exp2(-g.integers(0, 30, 2000))
    v = np.concatenate([vals, -vals, mids, -mids, rnd])
    ref = torch.from_numpy(v).to(torch.float8_e5m2).view(torch.uint8).numpy()
    got = np.array([orc.encode_e5m2(x) for x in v], np.uint8)
    assert np.array_equal(got, ref)


def test_e3m2_fixed_points():
    """Bias 3, 2 mantissa bits, no Inf/NaN: max 28, min normal 0.25, the three
    subnormals 1/16, 2/16, 3/16, and 32 increasing non-negative values."""
    v = [orc.e3m2_value(c) for c in range(32)]
    assert v[31] == 28.0 and v[4] == 0.25 and v[1:4] == [0.0625, 0.125, 0.1875] and v[0] == 0.0
    assert all(a < b for a, b in zip(v, v[1:]))
    assert [orc.e3m2_value(32 + c) for c in range(32)] == [-x for x in v]
    # nearest-even with saturation: ties go to the even code
    assert orc.encode_e3m2(30.0) == 31 and orc.encode_e3m2(1e9) == 31
    assert orc.encode_e3m2((v[5] + v[6]) / 2) == 6  # tie between codes 5 and 6
    assert orc.encode_e3m2(-(v[6] + v[7]) / 2) == 32 + 6


@pytest.mark.parametrize("fmt,emax,lo", [(orc.FMT_MXFP8_E5M2, 57344.0, 28672.0),
                                         (orc.FMT_MXFP6_E3M2, 28.0, 14.0)])
def test_scale_rule_ranges(fmt, emax, lo):
    """Every positive finite bf16 amax maps into (emax/2, emax] (E > 0)."""
    amax = np.arange(1, 0x7F80, dtype=np.uint16)
    x = np.zeros((amax.size, 32), np.uint16)
    x[:, 7] = amax
    _, s, _ = orc.quantize(fmt, x)
    E = s[:, 0].astype(np.int64)
    a = synth.bf16_to_f32(amax).astype(np.float64)
    sc = a * np.exp2(127.0 - E)
    assert np.all(sc[E > 0] > lo) and np.all(sc[E > 0] <= emax)
    assert np.all(a[E == 0] * 2.0**127 <= emax)


def test_fp6_packing_by_hand():
    """Codes 1, 2, 3, 4 then 28 more: element i in bits 6i .. 6i+5,
    little-endian: 000001 000010 000011 000100 -> 0x81 0x30 0x10."""
    vals = np.zeros(32)
    vals[:4] = [orc.e3m2_value(c) for c in (1, 2, 3, 4)]
    x = synth.bf16_bits(vals * 2.0**-4).reshape(1, 32)  # any scale: pick E so codes stay
    c, s, _ = orc.quantize(orc.FMT_MXFP6_E3M2, x)
    # amax = 0.25 * 2^-4 = 2^-6 -> E = ceil(log2(2^-6 / 28)) + 127 = -10 + 127
    assert s[0, 0] == 117
    y = orc.dequantize(orc.FMT_MXFP6_E3M2, c, s, 1.0, 1, 32)
    assert np.array_equal(y[0], (vals * 2.0**-4).astype(np.float32))
    x2 = synth.bf16_bits(np.concatenate([[orc.e3m2_value(c) for c in (1, 2, 3, 4)], np.zeros(27), [28.0]])).reshape(1, 32)
    c2, s2, _ = orc.quantize(orc.FMT_MXFP6_E3M2, x2)
    assert s2[0, 0] == 127 and c2.shape == (1, 24)
    assert list(c2[0, :3]) == [0x81, 0x30, 0x10]
    assert c2[0, 23] == (31 << 2) & 0xFF  # element 31 = code 31 in bits 186..191


def test_storage_bits():
    """6.25 bits per element for MXFP6 (the page's table), 8.25 for MXFP8."""
    n = 32 * 1000
    assert orc.storage_bytes(orc.FMT_MXFP6_E3M2, 1000, 32) * 8 / n == 6.25
    assert orc.storage_bytes(orc.FMT_MXFP8_E5M2, 1000, 32) * 8 / n == 8.25


@pytest.mark.parametrize("fmt", [orc.FMT_MXFP8_E5M2, orc.FMT_MXFP6_E3M2])
def test_brute_force_codes_and_exponents(fmt):
    """Every non-negative code at every reachable exponent, anchored by the
    largest code: quantize returns exactly that code and exponent, and
    dequantize returns code value * 2^(E-127)."""
    n = 124 if fmt == orc.FMT_MXFP8_E5M2 else 32
    val = orc.e5m2_value if fmt == orc.FMT_MXFP8_E5M2 else orc.e3m2_value
    top = val(n - 1)
    rows = []
    for E in range(40, 215, 7):
        blk = [val(c) * 2.0 ** (E - 127) for c in range(n)]
        blk = [top * 2.0 ** (E - 127)] + blk[: 31]
        rows.append(blk)
    x = synth.bf16_bits(np.array(rows))
    c, s, _ = orc.quantize(fmt, x)
    y = orc.dequantize(fmt, c, s, 1.0, *x.shape)
    assert np.array_equal(y.astype(np.float64), synth.bf16_to_f32(x).astype(np.float64))
    assert list(s[:, 0]) == list(range(40, 215, 7))
