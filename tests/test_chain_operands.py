"""The one-direction accumulation operands (chain_operands.py) do what they are
built for, checked with the oracle on the CPU: a plain fp32 chain over the
kernel's K groups breaks 2^-18 * sum|ab|, and chains of at most 48 steps
folded into a running total stay within it. These pin the GPU accumulation
tests that use the same operands."""
import numpy as np
import pytest

import chain_operands as co
import oracle as orc

BOUND = 2.0**-18


def _increments(x, y, groups):
    """Exact per-group sums of x * y (float64; every product is a power of two
    times a small integer, so each group sum is exact)."""
    return [float(sum(np.float64(x[k]) * np.float64(y[k]) for k in grp)) for grp in groups]


def _check(fmt, codes, scales, K, groups, ts=1.0, nsteps_expected=None):
    C, S = orc.gemm(fmt, fmt, 1, 1, K, codes[None], scales[None], ts, codes[None], scales[None], ts)
    C, S = float(C[0, 0]), float(S[0, 0])
    x = orc.dequantize(fmt, codes[None], scales[None], ts, 1, K)[0].astype(np.float64)
    inc = _increments(x, x, groups)
    assert np.isclose(sum(inc), C, rtol=0, atol=0)
    if nsteps_expected:
        assert len(groups) == nsteps_expected
    plain = float(co.fp32_chain(inc))
    seg = float(co.fp32_chain(inc, segment=48))
    assert abs(plain - C) > 1.25 * BOUND * S, (plain - C) / S
    assert abs(seg - C) <= BOUND * S, (seg - C) / S
    return abs(plain - C) / (BOUND * S), abs(seg - C) / (BOUND * S)


@pytest.mark.parametrize("K", [12288, 16384])
def test_mxfp4_tile256(K):
    codes, scales, groups = co.mxfp4(K, "tile256")
    elems = [tuple(range(32 * b, 32 * b + 32)) for b in range(K // 32)]
    g_elems = [sum((elems[b] for b in grp), ()) for grp in groups]
    plain, seg = _check(orc.FMT_MXFP4, codes, scales, K, g_elems, nsteps_expected=K // 64)
    print(f"MXFP4 K={K}: plain chain {plain:.2f}x the bound, segmented {seg:.2f}x")


def test_mxfp4_tile128():
    K = 12288 + 128
    codes, scales, groups = co.mxfp4(K, "tile128")
    g_elems = [tuple(range(128 * t, 128 * t + 128)) for t in range(len(groups))]
    _check(orc.FMT_MXFP4, codes, scales, K, g_elems, nsteps_expected=K // 128)


def test_mxfp8_groups_of_16():
    K = 3072
    codes, scales = co.mxfp8(K)
    groups = [tuple(range(16 * g, 16 * g + 16)) for g in range(K // 16)]
    _check(orc.FMT_MXFP8, codes, scales, K, groups)


def test_nvfp4_groups_of_16():
    K = 3072
    codes, scales = co.nvfp4(K)
    groups = [tuple(range(16 * g, 16 * g + 16)) for g in range(K // 16)]
    _check(orc.FMT_NVFP4, codes, scales, K, groups)
