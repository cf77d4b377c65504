"""Pins for the oracle's exact-operand GEMM.

Closed forms (constant operands give K*a*b; one-hot operands give a single
product), exact integer arithmetic on tiny inputs, and numpy's float64 matmul
over the dequantized operands (a library routine; it catches a transposed or
mis-indexed operand).
"""
import numpy as np
import pytest

import synth


def _mx_const(orc, fmt, rows, K, code, E):
    if fmt == orc.FMT_MXFP8:
        codes = np.full((rows, K), code, np.uint8)
        scales = np.full((rows, K // 32), E, np.uint8)
    else:
        codes = np.full((rows, K // 2), code | (code << 4), np.uint8)
        blk = 16 if fmt == orc.FMT_NVFP4 else 32
        scales = np.full((rows, K // blk), E, np.uint8)
    return codes, scales


def test_constant_operands_closed_form(orc):
    M, N, K = 8, 6, 256
    a, sa = _mx_const(orc, orc.FMT_MXFP4, M, K, 0x3, 128)  # 1.5 * 2
    b, sb = _mx_const(orc, orc.FMT_MXFP4, N, K, 0xD, 125)  # -3 * 2^-2
    C, S = orc.gemm(orc.FMT_MXFP4, orc.FMT_MXFP4, M, N, K, a, sa, 1.0, b, sb, 1.0)
    assert np.all(C == K * 3.0 * -0.75) and np.all(S == K * 2.25)
    a, sa = _mx_const(orc, orc.FMT_MXFP8, M, K, 0x3C, 120)  # 1.5 * 2^-7
    b, sb = _mx_const(orc, orc.FMT_MXFP8, N, K, 0x41, 127)  # 2.25
    C, S = orc.gemm(orc.FMT_MXFP8, orc.FMT_MXFP8, M, N, K, a, sa, 1.0, b, sb, 1.0)
    assert np.all(C == K * 1.5 * 2.0**-7 * 2.25)
    # NVFP4: e * s_b * s_t on both sides.
    a, sa = _mx_const(orc, orc.FMT_NVFP4, M, K, 0x7, 0x38)  # 6 * 1.0
    b, sb = _mx_const(orc, orc.FMT_NVFP4, N, K, 0x2, 0x30)  # 1 * 0.5
    C, S = orc.gemm(orc.FMT_NVFP4, orc.FMT_NVFP4, M, N, K, a, sa, 0.25, b, sb, 3.0)
    assert np.all(C == K * (6 * 1.0 * 0.25) * (1 * 0.5 * 3.0))


def test_one_hot_single_product(orc):
    M, N, K = 4, 5, 128
    a = np.zeros((M, K // 2), np.uint8)
    b = np.zeros((N, K // 2), np.uint8)
    sa = np.full((M, K // 32), 127, np.uint8)
    sb = np.full((N, K // 32), 127, np.uint8)
    a[2, 37 // 2] = 0x7 << 4  # A[2][37] = 6 (odd element -> high nibble)
    sa[2, 37 // 32] = 130  # x 2^3
    b[4, 37 // 2] = 0xB << 4  # B[4][37] = -1.5
    C, S = orc.gemm(orc.FMT_MXFP4, orc.FMT_MXFP4, M, N, K, a, sa, 1.0, b, sb, 1.0)
    want = np.zeros((M, N))
    want[2, 4] = 6 * 8 * -1.5
    assert np.array_equal(C, want) and np.array_equal(S, np.abs(want))


def test_integer_operands_exact(orc):
    g = np.random.Generator(np.random.PCG64(21))
    M, N, K = 7, 9, 64
    # E2M1 codes 2 (1.0), 4 (2.0), 5 (3.0), 6 (4.0) and negatives at scale 2^0.
    pool = np.array([0, 2, 4, 5, 6, 10, 12, 13, 14], np.uint8)
    val = {0: 0, 2: 1, 4: 2, 5: 3, 6: 4, 10: -1, 12: -2, 13: -3, 14: -4}
    ea = g.choice(pool, (M, K))
    eb = g.choice(pool, (N, K))
    a = (ea[:, 0::2] | (ea[:, 1::2] << 4)).astype(np.uint8)
    b = (eb[:, 0::2] | (eb[:, 1::2] << 4)).astype(np.uint8)
    sa = np.full((M, 2), 127, np.uint8)
    sb = np.full((N, 2), 127, np.uint8)
    C, S = orc.gemm(orc.FMT_MXFP4, orc.FMT_MXFP4, M, N, K, a, sa, 1.0, b, sb, 1.0)
    for i in range(M):
        for j in range(N):
            exact = sum(val[int(ea[i, k])] * val[int(eb[j, k])] for k in range(K))
            absum = sum(abs(val[int(ea[i, k])] * val[int(eb[j, k])]) for k in range(K))
            assert C[i, j] == exact and S[i, j] == absum


@pytest.mark.parametrize("fmt_name", ["mxfp4", "mxfp8", "nvfp4", "w4a16"])
def test_gemm_matches_numpy_on_dequantized(orc, fmt_name):
    M, N, K = 33, 47, 320
    A = synth.normal_outliers((M, K), 1.0, 31, 0.01, 50.0)
    B = synth.normal((N, K), 0.02, 32)
    if fmt_name == "w4a16":
        fa, fb = orc.FMT_BF16, orc.FMT_MXFP4
        a, sa, ta = A, None, 1.0
        ad = synth.bf16_to_f32(A).astype(np.float64)
    else:
        fa = fb = {"mxfp4": orc.FMT_MXFP4, "mxfp8": orc.FMT_MXFP8, "nvfp4": orc.FMT_NVFP4}[fmt_name]
        a, sa, ta = orc.quantize(fa, A)
    b, sb, tb = orc.quantize(fb, B)
    # Dequantized operands: MX values are exact in fp32; for NVFP4 take e*s_b
    # (tensor scale 1, exact) and apply the tensor scales in double.
    if fmt_name != "w4a16":
        ad = orc.dequantize(fa, a, sa, 1.0, M, K).astype(np.float64) * (ta if fa == orc.FMT_NVFP4 else 1.0)
    bd = orc.dequantize(fb, b, sb, 1.0, N, K).astype(np.float64) * (tb if fb == orc.FMT_NVFP4 else 1.0)
    C, S = orc.gemm(fa, fb, M, N, K, a, sa, ta, b, sb, tb)
    Cn = ad @ bd.T
    Sn = np.abs(ad) @ np.abs(bd).T
    assert np.all(np.abs(C - Cn) <= K * 2.0**-50 * Sn)
    assert np.allclose(S, Sn, rtol=K * 2.0**-50, atol=0)
    # The entries variant computes the same definition.
    ii = np.array([0, 5, M - 1, 17])
    jj = np.array([0, N - 1, 3, 29])
    Ce, Se = orc.gemm_entries(fa, fb, M, N, K, a, sa, ta, b, sb, tb, ii, jj)
    assert np.array_equal(Ce, C[ii, jj]) and np.array_equal(Se, S[ii, jj])


def test_gemm_rejects_bad_arguments(orc):
    a = np.zeros((4, 16), np.uint8)
    s = np.zeros((4, 1), np.uint8)
    with pytest.raises(ValueError):
        orc.gemm(orc.FMT_MXFP4, orc.FMT_MXFP4, 4, 4, 30, a, s, 1.0, a, s, 1.0)
    with pytest.raises(ValueError):
        orc.gemm_entries(orc.FMT_MXFP4, orc.FMT_MXFP4, 4, 4, 32, a, s, 1.0, a, s, 1.0,
                         np.array([4]), np.array([0]))
    # Operands shorter than M, N, K imply are refused before the C code reads
    # past them (here A holds 4 rows of a claimed 8; a bf16 A of 4 rows).
    with pytest.raises(ValueError):
        orc.gemm(orc.FMT_MXFP4, orc.FMT_MXFP4, 8, 4, 32, a, s, 1.0, a, s, 1.0)
    with pytest.raises(ValueError):
        orc.gemm(orc.FMT_BF16, orc.FMT_MXFP4, 8, 4, 32, np.zeros((4, 32), np.uint16), None, 1.0,
                 a, s, 1.0)
    with pytest.raises(ValueError):
        orc.dequantize(orc.FMT_MXFP4, a, s, 1.0, 8, 32)


@pytest.mark.parametrize("fmt,bits,W", [("FMT_MXFP4", 4, 256), ("FMT_MXFP8", 8, 64),
                                         ("FMT_MXFP8_E5M2", 8, 64), ("FMT_MXFP6_E3M2", 6, 64),
                                         ("FMT_NVFP4", 4, 64)])
def test_pack_kpanel_brute_force(orc, fmt, bits, W):
    """The K-panel layout by its definition, byte by byte, panels of W
    elements: code byte (p * rows + r) * wb + j is byte wb p + j of row r
    (wb = W * bits / 8), scale byte (p * rows + r) * sb + j is the scale of
    block sb p + j of row r (sb = W / block)."""
    f = getattr(orc, fmt)
    blk = orc.BLOCK[f]
    rows, cols = 5, 3 * W
    wb, sb = W * bits // 8, W // blk
    g = np.random.Generator(np.random.PCG64(71))
    codes = g.integers(0, 256, (rows, cols * bits // 8), dtype=np.uint8)
    scales = g.integers(0, 256, (rows, cols // blk), dtype=np.uint8)
    pc, ps = orc.pack_kpanel(codes, scales, rows, cols, f)
    assert pc.size == codes.size and ps.size == scales.size
    for p in range(cols // W):
        for r in range(rows):
            for j in range(wb):
                assert pc[(p * rows + r) * wb + j] == codes[r, wb * p + j]
            for j in range(sb):
                assert ps[(p * rows + r) * sb + j] == scales[r, sb * p + j]