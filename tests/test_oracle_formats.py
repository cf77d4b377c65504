"""Pins for the oracle's format decoders and element encoders.

Each check compares the oracle with something other than itself: the value
sets and formulas the pages print (tests/golden/pages_formats.json), torch's
own float8_e4m3fn and bfloat16 conversions, and brute force over the printed
value set.
"""
import math

import numpy as np
import pytest
import torch


def test_e2m1_decodes_to_printed_value_set(orc, pages):
    printed = pages["e2m1_values"]["values"]
    assert [orc.e2m1_value(c) for c in range(8)] == printed
    for c in range(8):
        assert orc.e2m1_value(c | 8) == -printed[c]
    assert math.copysign(1.0, orc.e2m1_value(8)) == -1.0  # code 0x8 is -0


def test_e2m1_bit_layout(orc):
    # 1 sign, 2 exponent bits with bias 1, 1 mantissa bit: field e > 0 is
    # 2^(e-1) * (1 + m/2); code 0b0110 -> e=3, m=0 -> 4.0.
    assert orc.e2m1_value(0b0110) == 4.0
    assert orc.e2m1_value(0b0011) == 1.5
    assert orc.e2m1_value(0b0001) == 0.5  # subnormal


def test_e8m0_is_power_of_two(orc, pages):
    bias = pages["e8m0"]["bias"]
    for E in range(255):
        assert orc.e8m0_value(E) == 2.0 ** (E - bias)
    assert math.isnan(orc.e8m0_value(255))


def test_e4m3_decode_matches_torch(orc, pages):
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).tolist()
    for c in range(256):
        v = orc.e4m3_value(c)
        if math.isnan(ref[c]):
            assert math.isnan(v), c
        else:
            assert v == ref[c] and math.copysign(1, v) == math.copysign(1, ref[c]), c
    assert orc.e4m3_value(0x7E) == pages["format_table"]["fp8_e4m3_max"]


def test_e4m3_encode_matches_torch_in_range(orc):
    # Every float32 in a dense sweep of [-448, 448] plus all midpoints between
    # neighbouring E4M3 values: torch's cast is round-to-nearest-even.
    vals = sorted({orc.e4m3_value(c) for c in range(0x7F)})
    mids = [(a + b) / 2 for a, b in zip(vals, vals[1:])]
    g = np.random.Generator(np.random.PCG64(7))
    sweep = np.concatenate([
        np.array(vals + mids, dtype=np.float64),
        g.uniform(-448, 448, 20000),
        g.uniform(-1, 1, 20000) * 2.0 ** g.integers(-12, 0, 20000),
    ]).astype(np.float32)
    sweep = np.concatenate([sweep, -sweep])
    ref = torch.from_numpy(sweep).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.encode_e4m3(float(v)) for v in sweep], dtype=np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(sweep[i]), int(got[i]), int(ref[i])) for i in bad[:10]]


def test_e4m3_encode_saturates(orc):
    for v in (448.0, 460.0, 464.0, 500.0, 1e30, math.inf):
        assert orc.encode_e4m3(v) == 0x7E
        assert orc.encode_e4m3(-v) == 0xFE
    assert orc.encode_e4m3(-0.0) == 0x80


def test_e2m1_encode_is_nearest_on_printed_set(orc, pages):
    printed = pages["e2m1_values"]["values"]
    g = np.random.Generator(np.random.PCG64(3))
    for v in np.concatenate([g.uniform(0, 7, 5000), np.arange(0, 7.01, 0.125)]):
        c = orc.encode_e2m1(float(v))
        assert c < 8
        d = abs(v - printed[c])
        assert all(d <= abs(v - p) for p in printed), v


def test_e2m1_ties_go_to_even_code(orc):
    # Midpoints between neighbours: round-to-nearest-even picks the code with
    # a clear mantissa bit.
    table = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for v, want in table.items():
        c = orc.encode_e2m1(v)
        assert orc.e2m1_value(c) == want, v
        assert c % 2 == 0
        assert orc.e2m1_value(orc.encode_e2m1(-v)) == -want


def test_e2m1_saturates_and_keeps_sign(orc):
    for v in (6.0, 6.5, 7.0, 100.0, math.inf):
        assert orc.encode_e2m1(v) == 0x7
        assert orc.encode_e2m1(-v) == 0xF
    assert orc.encode_e2m1(-0.0) == 0x8
    assert orc.encode_e2m1(-0.1) == 0x8  # rounds to -0
    assert orc.encode_e2m1(0.0) == 0x0


def test_f32_to_bf16_matches_torch(orc):
    g = np.random.Generator(np.random.PCG64(11))
    bits = g.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32)
    special = np.array([0, 0x80000000, 0x7F7FFFFF, 0xFF7FFFFF, 0x7F800000, 0x00000001,
                        0x00008000, 0x00018000, 0x3F808000, 0x3F818000, 0x7F7F8000],
                       dtype=np.uint32)
    bits = np.concatenate([bits, special])
    f = bits.view(np.float32)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.f32_to_bf16(float(x)) for x in f], dtype=np.uint16)
    nan = np.isnan(f)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7F80) == 0x7F80) and np.all((got[nan] & 0x7F) != 0)
