"""Plain CPU reference ("oracle") for microscaling quantization and the
block-scaled GEMM, wrapped for numpy.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The GPU library never calls it and
shares no code with it; the product path fails when its HIP library is missing
instead of falling back here.

The arithmetic lives in mx_oracle.c (see its header for what each routine
follows and how each is pinned). This module only marshals numpy arrays.
"""
import ctypes
import os

import numpy as np

from . import build as _build

FMT_BF16, FMT_MXFP4, FMT_MXFP8, FMT_NVFP4 = 0, 1, 2, 3
FMT_MXFP8_E5M2, FMT_MXFP6_E3M2, FMT_MXFP4_MBS, FMT_MXFP4_MBS16 = 4, 5, 6, 7
RULE_CEIL, RULE_OAS = 0, 1
ROT_NONE, ROT_WHT32 = 0, 1
OUT_F32, OUT_BF16 = 0, 1
BLOCK = {FMT_MXFP4: 32, FMT_MXFP8: 32, FMT_NVFP4: 16, FMT_MXFP8_E5M2: 32, FMT_MXFP6_E3M2: 32,
         FMT_MXFP4_MBS: 32, FMT_MXFP4_MBS16: 16}

_lib = None


def lib():
    """Load liboracle.so, compiling it first if it is missing or stale.
    MX_ORACLE_LIB, if set, names another build of the same source to load
    instead (the sanitizer build, in the sanitizer test's child process)."""
    global _lib
    if _lib is None:
        path = os.environ.get("MX_ORACLE_LIB") or _build.build(force=False)
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.mxo_bf16_value.restype = ctypes.c_double
        L.mxo_bf16_value.argtypes = [ctypes.c_uint16]
        for n in ("mxo_e2m1_value", "mxo_e4m3_value", "mxo_e8m0_value", "mxo_e5m2_value",
                  "mxo_e3m2_value"):
            getattr(L, n).restype = ctypes.c_double
            getattr(L, n).argtypes = [ctypes.c_uint8]
        for n in ("mxo_encode_e2m1", "mxo_encode_e4m3", "mxo_encode_e5m2", "mxo_encode_e3m2"):
            getattr(L, n).restype = ctypes.c_uint8
            getattr(L, n).argtypes = [ctypes.c_double]
        L.mxo_f32_to_bf16.restype = ctypes.c_uint16
        L.mxo_f32_to_bf16.argtypes = [ctypes.c_float]
        L.mxo_mx_scale_exponent.restype = ctypes.c_int
        L.mxo_mx_scale_exponent.argtypes = [ctypes.c_double, ctypes.c_double]
        L.mxo_mbs_macro_mantissa.restype = ctypes.c_int
        L.mxo_mbs_macro_mantissa.argtypes = [ctypes.c_double]
        L.mxo_storage_bytes.restype = i64
        L.mxo_storage_bytes.argtypes = [ctypes.c_int, i64, i64]
        L.mxo_quantize.restype = ctypes.c_int
        L.mxo_quantize.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, P, P, P, P]
        L.mxo_quantize_nvfp4_reciprocal.restype = ctypes.c_int
        L.mxo_quantize_nvfp4_reciprocal.argtypes = [i64, i64, P, P, P, P]
        L.mxo_quantize_ex.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, i64, i64, P, P, P]
        L.mxo_wht32.argtypes = [i64, i64, P, P]
        L.mxo_dequantize.restype = ctypes.c_int
        L.mxo_dequantize.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, P, P,
                                     ctypes.c_float, ctypes.c_int, P]
        L.mxo_gemm.restype = ctypes.c_int
        L.mxo_gemm.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64,
                               P, P, ctypes.c_float, P, P, ctypes.c_float, P, P]
        L.mxo_gemm_entries.restype = ctypes.c_int
        L.mxo_gemm_entries.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64,
                                       P, P, ctypes.c_float, P, P, ctypes.c_float,
                                       i64, P, P, P, P]
        L.mxo_num_threads.restype = ctypes.c_int
        L.mxo_num_threads.argtypes = []
        _lib = L
    return _lib


def num_threads():
    """Host threads the GEMM routines use (OpenMP's limit)."""
    return int(lib().mxo_num_threads())


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (status {rc})")


# ---- scalar format helpers -------------------------------------------------
def bf16_value(bits):
    return lib().mxo_bf16_value(int(bits))


def e2m1_value(code):
    return lib().mxo_e2m1_value(int(code))


def e4m3_value(code):
    return lib().mxo_e4m3_value(int(code))


def e8m0_value(e):
    return lib().mxo_e8m0_value(int(e))


def encode_e2m1(v):
    return lib().mxo_encode_e2m1(float(v))


def encode_e4m3(v):
    return lib().mxo_encode_e4m3(float(v))


def e5m2_value(code):
    return lib().mxo_e5m2_value(int(code))


def e3m2_value(code):
    return lib().mxo_e3m2_value(int(code))


def encode_e5m2(v):
    return lib().mxo_encode_e5m2(float(v))


def encode_e3m2(v):
    return lib().mxo_encode_e3m2(float(v))


def f32_to_bf16(f):
    return lib().mxo_f32_to_bf16(float(f))


def mx_scale_exponent(amax, emax):
    return lib().mxo_mx_scale_exponent(float(amax), float(emax))


def mbs_macro_mantissa(alpha):
    return lib().mxo_mbs_macro_mantissa(float(alpha))


def storage_bytes(fmt, rows, cols):
    return lib().mxo_storage_bytes(fmt, rows, cols)


# ---- tensor operations -----------------------------------------------------
def code_shape(fmt, rows, cols):
    if fmt in (FMT_MXFP8, FMT_MXFP8_E5M2):
        return (rows, cols)
    if fmt == FMT_MXFP6_E3M2:
        return (rows, cols * 3 // 4)
    return (rows, cols // 2)


def scale_shape(fmt, rows, cols):
    """[rows][cols/block]; MXFP4-MBS / MBS16: one flat buffer holding the E8M0
    plane [rows][cols/block] and then the macro plane [rows][cols/128]."""
    if fmt in (FMT_MXFP4_MBS, FMT_MXFP4_MBS16):
        return (rows * (cols // BLOCK[fmt]) + rows * (cols // 128),)
    return (rows, cols // BLOCK[fmt])


def mbs_planes(scales, rows, cols, block=32):
    """Split an MXFP4-MBS (block 32) or MBS16 (block 16) scale buffer into
    (E8M0 [rows][cols/block], macro mantissas [rows][cols/128])."""
    s = np.asarray(scales).reshape(-1)
    n = rows * (cols // block)
    return s[:n].reshape(rows, cols // block), s[n:].reshape(rows, cols // 128)


# K-panel geometry per format: panel width W in elements, code bytes and
# scale bytes of one row in one panel (W * bits / 8 and W / block).
KPANEL = {FMT_MXFP4: (256, 128, 8), FMT_MXFP8: (64, 64, 2), FMT_MXFP8_E5M2: (64, 64, 2),
          FMT_MXFP6_E3M2: (64, 48, 2), FMT_NVFP4: (64, 32, 4)}


def pack_kpanel(codes, scales, rows, cols, fmt=FMT_MXFP4):
    """The K-panel layout of a quantized tensor (a byte permutation, no
    arithmetic): codes [cols/W][rows][wb], scales [cols/W][rows][sb], from
    the row layout [rows][cols * bits / 8] and [rows][cols / block], with W,
    wb and sb from KPANEL (MXFP4: 256, 128, 8)."""
    W, wb, sb = KPANEL[fmt]
    assert cols % W == 0
    p = cols // W
    c = np.asarray(codes, np.uint8).reshape(rows, p, wb).transpose(1, 0, 2).reshape(-1)
    s = np.asarray(scales, np.uint8).reshape(rows, p, sb).transpose(1, 0, 2).reshape(-1)
    return c.copy(), s.copy()


def quantize(fmt, x_bits):
    """x_bits: uint16 [rows][cols] bf16 bit patterns.
    Returns (codes uint8, scales uint8 (scale_shape), tensor_scale float)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    rows, cols = x.shape
    blk = BLOCK[fmt]
    codes = np.zeros(code_shape(fmt, rows, cols), np.uint8)
    scales = np.zeros(scale_shape(fmt, rows, cols), np.uint8)
    ts = np.zeros(1, np.float32)
    _check(lib().mxo_quantize(fmt, blk, rows, cols, _ptr(x), _ptr(codes),
                              _ptr(scales), _ptr(ts)), "quantize")
    return codes, scales, float(ts[0])


def quantize_ex(fmt, x_bits, rule=RULE_CEIL, rot=ROT_NONE):
    """MX quantization variants (mx_oracle.h: mxo_quantize_ex): overflow-aware
    scaling (MXFP4) and/or the 32-point Walsh-Hadamard rotation first.
    Returns (codes, scales)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    rows, cols = x.shape
    codes = np.zeros(code_shape(fmt, rows, cols), np.uint8)
    scales = np.zeros((rows, cols // 32), np.uint8)
    _check(lib().mxo_quantize_ex(fmt, 32, rule, rot, rows, cols, _ptr(x), _ptr(codes), _ptr(scales)),
           "quantize_ex")
    return codes, scales


def wht32(x_bits):
    """bf16 bits [rows][cols] -> the rotated bf16 bits (mx_oracle.h: mxo_wht32)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    y = np.zeros_like(x)
    _check(lib().mxo_wht32(x.shape[0], x.shape[1], _ptr(x), _ptr(y)), "wht32")
    return y


def quantize_nvfp4_reciprocal(x_bits):
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    rows, cols = x.shape
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // 16), np.uint8)
    ts = np.zeros(1, np.float32)
    _check(lib().mxo_quantize_nvfp4_reciprocal(rows, cols, _ptr(x), _ptr(codes),
                                               _ptr(scales), _ptr(ts)), "quantize")
    return codes, scales, float(ts[0])


def dequantize(fmt, codes, scales, tensor_scale, rows, cols, out=OUT_F32):
    """Returns float32 [rows][cols] (OUT_F32) or uint16 bf16 bits (OUT_BF16)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    if cols % BLOCK[fmt] == 0:
        _need(codes, int(np.prod(code_shape(fmt, rows, cols))), "codes")
        _need(scales, int(np.prod(scale_shape(fmt, rows, cols))), "scales")
    y = np.zeros((rows, cols), np.float32 if out == OUT_F32 else np.uint16)
    _check(lib().mxo_dequantize(fmt, BLOCK[fmt], rows, cols, _ptr(codes), _ptr(scales),
                                float(tensor_scale), out, _ptr(y)), "dequantize")
    return y


def _need(arr, n, what):
    """The C routines read exactly n elements: refuse any other size."""
    if arr.size != n:
        raise ValueError(f"oracle: {what} holds {arr.size} elements, the shape needs {n}")


def _gemm_operands(fmt, data, scales, rows, K):
    if fmt == FMT_BF16:
        data = np.ascontiguousarray(data, dtype=np.uint16)
        _need(data, rows * K, "bf16 operand")
        return data, None
    if K % BLOCK[fmt] != 0:
        raise ValueError(f"oracle: K = {K} is not a multiple of the block size {BLOCK[fmt]}")
    data = np.ascontiguousarray(data, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    _need(data, int(np.prod(code_shape(fmt, rows, K))), "code operand")
    _need(scales, int(np.prod(scale_shape(fmt, rows, K))), "scale operand")
    return data, scales


def gemm(fmt_a, fmt_b, M, N, K, a, a_scales, a_ts, b, b_scales, b_ts):
    """Exact-operand GEMM in double. Returns (C, S), each float64 [M][N], with
    S = sum_k |a_ik * b_jk|. B is stored N x K."""
    a, a_scales = _gemm_operands(fmt_a, a, a_scales, M, K)
    b, b_scales = _gemm_operands(fmt_b, b, b_scales, N, K)
    C = np.zeros((M, N), np.float64)
    S = np.zeros((M, N), np.float64)
    _check(lib().mxo_gemm(fmt_a, fmt_b, M, N, K, _ptr(a), _ptr(a_scales), float(a_ts),
                          _ptr(b), _ptr(b_scales), float(b_ts), _ptr(C), _ptr(S)), "gemm")
    return C, S


def gemm_entries(fmt_a, fmt_b, M, N, K, a, a_scales, a_ts, b, b_scales, b_ts, ii, jj):
    """As gemm(), only for output entries (ii[t], jj[t]). Returns (C, S) 1-D."""
    a, a_scales = _gemm_operands(fmt_a, a, a_scales, M, K)
    b, b_scales = _gemm_operands(fmt_b, b, b_scales, N, K)
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    C = np.zeros(len(ii), np.float64)
    S = np.zeros(len(ii), np.float64)
    _check(lib().mxo_gemm_entries(fmt_a, fmt_b, M, N, K, _ptr(a), _ptr(a_scales),
                                  float(a_ts), _ptr(b), _ptr(b_scales), float(b_ts),
                                  len(ii), _ptr(ii), _ptr(jj), _ptr(C), _ptr(S)),
           "gemm_entries")
    return C, S
