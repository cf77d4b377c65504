"""Pins for the oracle's MX shared-exponent rule, exhaustively over bf16.

The rule (FAQ on the produtoramaxvision page: E = ceil(log2(amax / max_E2M1))
+ 127, so that no scaled element exceeds the element format's ceiling) is
checked against two facts that do not come from the oracle:
  * no scaled amax exceeds the ceiling (6 for E2M1, 448 for E4M3), and
  * the standard MXFP4 scale maps the block amax into (3, 6] (gist.science
    summary, section 2.A), i.e. one exponent lower would overflow. For E4M3
    the same minimality gives (224, 448].
"""
import math

import numpy as np


def _all_positive_finite_bf16():
    bits = np.arange(1, 0x7F80, dtype=np.uint32)  # +0 excluded, up to max finite
    return (bits << 16).view(np.float32).astype(np.float64)


def _check_rule(orc, emax, lo):
    amaxes = _all_positive_finite_bf16()
    at_zero = 0
    for a in amaxes:
        E = orc.mx_scale_exponent(a, emax)
        assert 0 <= E <= 254
        scaled = a * 2.0 ** (127 - E)  # exact: power-of-two scaling in double
        assert scaled <= emax, (a, E)
        if E > 0:
            assert lo < scaled, (a, E)
        else:
            at_zero += 1
    return at_zero


def test_mxfp4_scale_rule_exhaustive(orc, pages):
    rng = pages["standard_scaled_amax_range"]
    assert (rng["open_low"], rng["closed_high"]) == (3.0, 6.0)
    at_zero = _check_rule(orc, 6.0, 3.0)
    # E = 0 exactly for amax <= 6 * 2^-127 (the clamp covers amax <= 3 * 2^-127).
    assert at_zero == sum(1 for a in _all_positive_finite_bf16() if a * 2.0**127 <= 6.0)


def test_mxfp8_scale_rule_exhaustive(orc):
    _check_rule(orc, 448.0, 224.0)


def test_scale_rule_edges(orc):
    assert orc.mx_scale_exponent(0.0, 6.0) == 0
    assert orc.mx_scale_exponent(math.inf, 6.0) == 255
    assert orc.mx_scale_exponent(math.nan, 6.0) == 255
    # Largest finite bf16 never reaches E = 254 or the NaN code 255.
    bmax = float(np.array([0x7F7F0000], np.uint32).view(np.float32)[0])
    assert orc.mx_scale_exponent(bmax, 6.0) == 253
    assert orc.mx_scale_exponent(bmax, 448.0) == 247
    # Block amax exactly at the ceiling keeps scale 2^0.
    assert orc.mx_scale_exponent(6.0, 6.0) == 127
    assert orc.mx_scale_exponent(6.0 * (1 + 2**-7), 6.0) == 128
    assert orc.mx_scale_exponent(448.0, 448.0) == 127
