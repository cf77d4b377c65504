"""Pins for the oracle's MX quantization variants, checked against what the
pages and the mathematics fix, not against the oracle's own formulas:

* overflow-aware scaling (gist.science summary of "Unveiling the Potential of
  Quantization with MXFP4", section 2.A): the scaled block amax lies in
  (3.5, 7] instead of (3, 6], and values in (6, 7] saturate;
* the 32-point Walsh-Hadamard rotation (produtoramaxvision page, section
  "Tecnicas de preservacao de acuracia: QuaRot, SpinQuant e ReSET"): checked
  against the Sylvester matrix H[i][j] = (-1)^popcount(i & j), exact integer
  products, orthogonality and energy preservation.
"""
import numpy as np
import pytest
import torch

import oracle as orc
import synth


def _positive_finite_bf16():
    b = np.arange(1, 0x7F80, dtype=np.uint16)  # +min subnormal .. +max finite
    return b


def test_oas_scale_range_exhaustive():
    """Every positive finite bf16 amax: E8M0 E with amax * 2^(127-E) in
    (3.5, 7] (the OAS range), or E = 0 when even 2^-127 * 7 covers it."""
    amax = _positive_finite_bf16()
    x = np.zeros((amax.size, 32), np.uint16)
    x[:, 5] = amax
    _, scales = orc.quantize_ex(orc.FMT_MXFP4, x, orc.RULE_OAS)
    E = scales[:, 0].astype(np.int64)
    a = synth.bf16_to_f32(amax).astype(np.float64)
    scaled = a * np.exp2(127.0 - E)
    interior = E > 0
    assert np.all(scaled[interior] > 3.5) and np.all(scaled[interior] <= 7.0)
    assert np.all(a[~interior] * 2.0**127 <= 7.0)
    # and the ceil rule keeps (3, 6] on the same inputs
    _, sc = orc.quantize_ex(orc.FMT_MXFP4, x, orc.RULE_CEIL)
    Ec = sc[:, 0].astype(np.int64)
    s2 = a * np.exp2(127.0 - Ec)
    assert np.all(s2[Ec > 0] > 3.0) and np.all(s2[Ec > 0] <= 6.0)
    # OAS takes one binade less exactly when the scaled amax would be in (3, 3.5]
    lower = (Ec > 0) & (E == Ec - 1)
    assert np.array_equal(lower, (Ec > 0) & (s2 <= 3.5))
    assert np.all((E == Ec) | lower)


def test_oas_saturates_six_to_seven():
    """A block whose OAS-scaled values reach (6, 7]: those elements give the
    largest code (6), every other element is the nearest E2M1 value of the
    finer scale."""
    vals = np.array([6.5, 6.25, -7.0, 6.0, 5.0, 3.5, 1.75, -0.25] * 4)
    x = synth.bf16_bits(vals).reshape(1, 32)
    codes, scales = orc.quantize_ex(orc.FMT_MXFP4, x, orc.RULE_OAS)
    assert scales[0, 0] == 127  # 7 * 2^0 covers amax 7
    nib = np.stack([codes[0] & 0xF, codes[0] >> 4], 1).reshape(-1)
    mag = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    got = np.where(nib & 8, -1, 1) * mag[nib & 7]
    want = np.array([6, 6, -6, 6, 4, 4, 2, -0] * 4, float)  # 5 -> 4 (tie to even code), 3.5 -> 4, 1.75 -> 2
    assert np.array_equal(got, want)


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_wht32_columns_are_sylvester():
    """Rotating the unit vector e_j gives column j of H / sqrt(32):
    (-1)^popcount(i & j) * bf16(fl32(1/sqrt(32)))."""
    c = np.float32(1.0 / np.sqrt(32.0))
    for j in range(32):
        x = np.zeros((1, 64), np.uint16)
        x[0, 32 + j] = synth.bf16_bits(np.array([1.0]))[0]
        y = orc.wht32(x)
        assert np.all(y[0, :32] == 0)
        signs = np.array([-1.0 if bin(i & j).count("1") % 2 else 1.0 for i in range(32)], np.float32)
        assert np.array_equal(y[0, 32:], _bf16(signs * c)), j


def test_wht32_integer_vectors_exact():
    """Small integers: the butterfly's fp32 sums are exact, so the result is
    bf16(fl32(H x) * c) with H x from exact integer arithmetic."""
    g = np.random.Generator(np.random.PCG64(77))
    X = g.integers(-100, 101, (64, 32))
    H = np.array([[-1 if bin(i & j).count("1") % 2 else 1 for j in range(32)] for i in range(32)])
    HX = X @ H.T  # exact integers
    c = np.float32(1.0 / np.sqrt(32.0))
    want = _bf16(HX.astype(np.float32) * c)
    got = orc.wht32(synth.bf16_bits(X.astype(np.float64)))
    assert np.array_equal(got, want)


def test_wht32_orthogonal_and_energy():
    """H H^T = 32 I: rotating twice returns the input and the block energy is
    kept, within the two bf16 roundings."""
    x = synth.normal_outliers((64, 256), 1.0, 5, 0.02, 40.0)
    xf = synth.bf16_to_f32(x).astype(np.float64)
    y = orc.wht32(x)
    yf = synth.bf16_to_f32(y).astype(np.float64)
    e_x = (xf.reshape(64, 8, 32) ** 2).sum(-1)
    e_y = (yf.reshape(64, 8, 32) ** 2).sum(-1)
    assert np.allclose(e_y, e_x, rtol=2**-6)
    z = synth.bf16_to_f32(orc.wht32(y)).astype(np.float64)
    err = np.abs(z - xf).reshape(64, 8, 32).max(-1)
    scale = np.abs(xf).reshape(64, 8, 32).max(-1)
    assert np.all(err <= 2**-6 * scale)


@pytest.mark.parametrize("fmt", [orc.FMT_MXFP4, orc.FMT_MXFP8])
def test_rotated_quantize_is_quantize_of_rotation(fmt):
    x = synth.laplace_outlier_channels((40, 512), 3, 4, 0.01, 100.0)
    c1, s1 = orc.quantize_ex(fmt, x, orc.RULE_CEIL, orc.ROT_WHT32)
    c2, s2, _ = orc.quantize(fmt, orc.wht32(x))
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_variant_arguments_rejected():
    x = np.zeros((2, 64), np.uint16)
    with pytest.raises(Exception):
        orc.quantize_ex(orc.FMT_MXFP8, x, orc.RULE_OAS)  # OAS is MXFP4's rule
    with pytest.raises(Exception):
        orc.quantize_ex(orc.FMT_NVFP4, x, orc.RULE_CEIL)


def test_wht32_close_to_exact_rotation_on_outlier_blocks():
    """The oracle's rotation against the exact one on data where fp32 sums
    round (the MLP-down activations: Laplace with x100 outlier channels, plus
    blocks mixing values 2^20 apart): each output y_i must lie within the
    rounding budget of the exact (H x)_i / sqrt(32), computed in rational
    arithmetic with 1/sqrt(32) to 80 bits. Budget, with u = 2^-24: five fp32
    butterfly levels gamma_5 sum|x| (gamma_5 = 5u / (1 - 5u)), the rounded
    constant and the product 2u |H x| / sqrt(32), then the bf16 rounding
    2^-8 |t| of the fp32 value t (or 2^-134 below bf16's normal range). A
    wrong sign, pairing or constant misses this by orders of magnitude."""
    from fractions import Fraction
    import math
    A = synth.laplace_outlier_channels((8, 2048), 401, 403, 0.005, 100.0)
    g = synth.rng(77)
    B = synth.bf16_bits(g.normal(0, 1, (4, 2048)) * np.exp2(g.integers(-10, 11, (4, 2048))))
    X = np.concatenate([A, B], 0)
    Y = orc.wht32(X)
    xv = synth.bf16_to_f32(X).astype(np.float64)
    yv = synth.bf16_to_f32(Y).astype(np.float64)
    H = np.array([[(-1) ** bin(i & j).count("1") for j in range(32)] for i in range(32)])
    inv_sqrt32 = Fraction(math.isqrt(2**160 // 32), 2**80)  # 1/sqrt(32) to 80 bits
    u = 2.0**-24
    gamma5 = 5 * u / (1 - 5 * u)
    worst = 0.0
    for r in range(X.shape[0]):
        for b in range(X.shape[1] // 32):
            x = [Fraction(float(v)) for v in xv[r, 32 * b:32 * b + 32]]
            s_abs = float(sum(abs(v) for v in x))
            for i in range(32):
                z = sum(x[j] if H[i, j] > 0 else -x[j] for j in range(32))
                exact = float(z * inv_sqrt32)
                t_bound = abs(exact) * (1 + 2 * u) + gamma5 * s_abs / math.sqrt(32) * (1 + u)
                budget = (gamma5 * s_abs / math.sqrt(32) * (1 + u) + 2.0 * u * abs(exact)
                          + max(2.0**-8 * t_bound, 2.0**-134))
                err = abs(yv[r, 32 * b + i] - exact)
                assert err <= budget, (r, b, i, yv[r, 32 * b + i], exact, err, budget)
                worst = max(worst, err / budget)
    print(f"wht32: worst error / budget = {worst:.3f}")
