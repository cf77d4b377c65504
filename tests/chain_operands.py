"""Operands built to make a long fp32 accumulation chain err in one direction.

Every output C[i][j] of these operands is the same dot product: one large
product ("big") in the first K group a kernel sums with one instruction, then
one small increment d per later group, where d is just over half a unit in
the last place of the running sum. A plain fp32 chain that rounds each group's
exact sum onto the running total to nearest then rounds up by almost half an
ulp at every step, so after n steps it is off by about n/2 ulps: beyond
2^-18 * sum|ab| once n passes ~64 (the accumulation bound the GEMM promises).

The group structure follows each kernel's K order (which K elements one
matrix instruction sums before adding to the accumulator); the values are
code bytes and scale bytes written directly, not quantized from bf16.

Formats (element values from the E2M1 / E4M3 tables):
 * MXFP4: E2M1 code 2 = 1.0, 6 = 4.0, 1 = 0.5; E8M0 byte E is 2^(E-127).
 * MXFP8: E4M3 0x38 = 1.0, 0x20 = 0.125.
 * NVFP4: E2M1 codes with E4M3 block scales 0x78 = 256, 0x20 = 0.125;
   tensor scales 1.
"""
import numpy as np


def _fp4_row(K, vals):
    """Codes [K/2] of one row from {element index: E2M1 code}."""
    codes = np.zeros(K // 2, np.uint8)
    for k, c in vals.items():
        codes[k // 2] |= np.uint8(c << (4 * (k % 2)))
    return codes


def mxfp4(K, layout):
    """MXFP4 operands (codes [K/2], scales [K/32]) for one row, identical for A
    and B. layout "tile256": one K super-step of 256 is 4 instructions, the
    instruction j covering blocks j and 4 + j (32x32x64, scale per lane
    group); "tile128": one instruction per 128 K (16x16x128, blocks 4t..4t+3).
    Returns (codes, scales, groups) with groups the list of block-index
    tuples in chain order."""
    nb = K // 32
    if layout == "tile256":
        assert K % 256 == 0
        groups = [(8 * s + j, 8 * s + 4 + j) for s in range(K // 256) for j in range(4)]
    else:
        assert K % 128 == 0
        groups = [tuple(range(4 * t, 4 * t + 4)) for t in range(K // 128)]
    vals = {}
    scales = np.full(nb, 127, np.uint8)
    for n, grp in enumerate(groups):
        b = grp[0]
        if n == 0:
            vals[32 * b] = 2          # 1.0 at scale 2^0: product 1
        else:
            vals[32 * b] = 6          # 4.0 * 2^-14: product 2^-24
            vals[32 * b + 1] = 1      # 0.5 * 2^-14: product 2^-30
            scales[b] = 127 - 14
    return _fp4_row(K, vals), scales, groups


def mxfp8(K):
    """MXFP8 (E4M3) operands for one row: the 16-bit path sums 16 consecutive
    K elements per instruction. Group 0 holds the product 1; groups 2, 3, ...
    each hold 2^-24 + 2^-30 (group 1 shares block 0's scale 2^0, where the
    small values are not representable, and stays zero)."""
    assert K % 32 == 0
    codes = np.zeros(K, np.uint8)
    scales = np.full(K // 32, 127, np.uint8)
    codes[0] = 0x38                   # 1.0
    for g in range(2, K // 16):
        k = 16 * g
        codes[k] = 0x38               # 1.0 * 2^-12
        codes[k + 1] = 0x20           # 0.125 * 2^-12
        scales[k // 32] = 127 - 12
    return codes, scales


def nvfp4(K):
    """NVFP4 operands for one row (16-blocks = one instruction's K group of the
    16-bit path): block 0 holds 4 * 256 (product 2^20, ulp 2^-3), every later
    block 6 * 0.125 and 0.5 * 0.125 (products 0.5625 + 0.00390625 = 4.53
    ulps, rounded up by 0.47 ulp each)."""
    assert K % 16 == 0
    vals = {0: 6}
    scales = np.full(K // 16, 0x20, np.uint8)
    scales[0] = 0x78
    for b in range(1, K // 16):
        vals[16 * b] = 7
        vals[16 * b + 1] = 1
    return _fp4_row(K, vals), scales


def tile(row, rows):
    """The same row repeated `rows` times."""
    return np.ascontiguousarray(np.broadcast_to(row, (rows,) + row.shape))


def fp32_chain(increments, segment=None):
    """Sum exact float64 increments in fp32, one rounding per step (each
    increment is exact in double and the running fp32 value plus it is exact
    in double, so float32() of the double sum rounds once). With `segment`,
    every `segment` increments start a fresh chain from zero and each
    finished chain is added to the running total (one rounding per fold)."""
    total = None
    acc = np.float32(0.0)
    for n, p in enumerate(increments):
        if segment and n > 0 and n % segment == 0:
            total = acc if total is None else np.float32(np.float64(total) + np.float64(acc))
            acc = np.float32(0.0)
        acc = np.float32(np.float64(acc) + p)
    if total is None:
        return acc
    return np.float32(np.float64(total) + np.float64(acc))
