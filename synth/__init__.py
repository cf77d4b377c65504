"""Seeded synthetic inputs for the quantizer and the block-scaled GEMM.

Shared by the tests, the benchmark and the smoke check. Holds none of the
method's arithmetic: it only draws random tensors and rounds them to bf16, the
input dtype. Every tensor is a uint16 numpy array of bf16 bit patterns.

Generator: numpy's PCG64 bit generator (numpy.random.Generator), seeded per
tensor. Values are drawn in float64, rounded to float32 (nearest-even, numpy's
cast) and then to bf16 (nearest-even on the bit pattern). The pages run on
diffusion and LLM checkpoints that are not available here; these tensors stand
in for their Linear-layer inputs and weights, with the shapes and distributions
listed in WORKLOADS.
"""
import hashlib

import numpy as np


def f32_to_bf16_bits(x32):
    """float32 array -> uint16 bf16 bit patterns, nearest-even; NaN stays NaN."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    r = np.where(nan, (u >> np.uint32(16)) | np.uint32(0x40), r)
    return r.astype(np.uint16)


def bf16_bits(x):
    """float64 (or float32) array -> bf16 bits via float32."""
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float64).astype(np.float32))


def bf16_to_f32(bits):
    """uint16 bf16 bit patterns -> float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def normal(shape, sigma, seed):
    return bf16_bits(rng(seed).normal(0.0, sigma, size=shape))


def normal_outliers(shape, sigma, seed, frac, factor):
    """N(0, sigma) with each entry independently multiplied by `factor` with
    probability `frac` (Bernoulli per entry, applied before bf16 rounding)."""
    g = rng(seed)
    x = g.normal(0.0, sigma, size=shape)
    mask = g.random(size=shape) < frac
    x[mask] *= factor
    return bf16_bits(x)


def student_t(shape, nu, seed):
    return bf16_bits(rng(seed).standard_t(nu, size=shape))


def laplace_outlier_channels(shape, seed, channel_seed, frac, factor):
    """Laplace(0, 1) with round(frac * cols) whole columns (channels, the K
    axis) multiplied by `factor`, chosen without replacement."""
    x = rng(seed).laplace(0.0, 1.0, size=shape)
    cols = shape[1]
    n = int(round(frac * cols))
    chans = rng(channel_seed).choice(cols, size=n, replace=False)
    x[:, chans] *= factor
    return bf16_bits(x)


def uniform_positive(shape, lo, hi, seed):
    """All-positive operands: the GEMM's |C| equals sum |a*b| (worst case for
    accumulation error)."""
    return bf16_bits(rng(seed).uniform(lo, hi, size=shape))


# Workloads. A is M x K (tokens x hidden); B is stored N x K (the Linear
# weight layout, K contiguous); blocks run along K.
WORKLOADS = {
    "mxfp4_roundtrip_256x512x256": dict(
        fmt="mxfp4", M=256, N=256, K=512,
        a=("normal_outliers", 1.0, 101, 0.01, 50.0),
        b=("normal_outliers", 1.0, 102, 0.01, 50.0)),
    "mxfp8_dit_qkv_4608x3072x9216": dict(
        fmt="mxfp8", M=4608, N=9216, K=3072,
        a=("normal", 1.0, 201), b=("normal", 0.02, 202)),
    "nvfp4_dit_mlp_up_4608x3072x12288": dict(
        fmt="nvfp4", M=4608, N=12288, K=3072,
        a=("student_t", 4.0, 301), b=("normal", 0.02, 302)),
    "mxfp4_dit_mlp_down_4608x12288x3072": dict(
        fmt="mxfp4", M=4608, N=3072, K=12288,
        a=("laplace_outlier_channels", 401, 403, 0.005, 100.0),
        b=("normal", 0.02, 402)),
    "w4a16_decode_16x8192x28672": dict(
        fmt="w4a16", M=16, N=28672, K=8192,
        a=("normal", 1.0, 501), b=("normal", 0.02, 502)),
    # Format and quantizer variants on the shapes and data of the rows above.
    "mxfp8e5m2_dit_qkv_4608x3072x9216": dict(
        fmt="mxfp8_e5m2", M=4608, N=9216, K=3072,
        a=("normal", 1.0, 201), b=("normal", 0.02, 202)),
    "mxfp6e3m2_dit_qkv_4608x3072x9216": dict(
        fmt="mxfp6_e3m2", M=4608, N=9216, K=3072,
        a=("normal", 1.0, 201), b=("normal", 0.02, 202)),
    "mxfp4oas_dit_mlp_down_4608x12288x3072": dict(
        fmt="mxfp4", M=4608, N=3072, K=12288, scale_rule="oas",
        a=("laplace_outlier_channels", 401, 403, 0.005, 100.0),
        b=("normal", 0.02, 402)),
    "mxfp4wht32_dit_mlp_down_4608x12288x3072": dict(
        fmt="mxfp4", M=4608, N=3072, K=12288, rotation="wht32",
        a=("laplace_outlier_channels", 401, 403, 0.005, 100.0),
        b=("normal", 0.02, 402)),
    "mxfp4mbs_dit_mlp_down_4608x12288x3072": dict(
        fmt="mxfp4_mbs", M=4608, N=3072, K=12288,
        a=("laplace_outlier_channels", 401, 403, 0.005, 100.0),
        b=("normal", 0.02, 402)),
    "mxfp4mbs16_dit_mlp_down_4608x12288x3072": dict(
        fmt="mxfp4_mbs16", M=4608, N=3072, K=12288,
        a=("laplace_outlier_channels", 401, 403, 0.005, 100.0),
        b=("normal", 0.02, 402)),
    # The decode weights alone (28672 x 8192 bf16, 470 MB, beyond the
    # last-level cache): their MXFP4 quantization is the largest HBM-bound
    # quantize of the workloads.
    "mxfp4_quantize_decode_weights_28672x8192": dict(
        fmt="mxfp4", M=28672, N=0, K=8192, step="quantize",
        a=("normal", 0.02, 502), b=None),
}

# Short names used on the command line and in tests.
ALIASES = {
    "c1": "mxfp4_roundtrip_256x512x256",
    "c2": "mxfp8_dit_qkv_4608x3072x9216",
    "c3": "nvfp4_dit_mlp_up_4608x3072x12288",
    "c4": "mxfp4_dit_mlp_down_4608x12288x3072",
    "c5": "w4a16_decode_16x8192x28672",
    "f1": "mxfp4oas_dit_mlp_down_4608x12288x3072",
    "f2a": "mxfp8e5m2_dit_qkv_4608x3072x9216",
    "f2b": "mxfp6e3m2_dit_qkv_4608x3072x9216",
    "f3": "mxfp4mbs_dit_mlp_down_4608x12288x3072",
    "f4": "mxfp4wht32_dit_mlp_down_4608x12288x3072",
    "f3b": "mxfp4mbs16_dit_mlp_down_4608x12288x3072",
    "c5w": "mxfp4_quantize_decode_weights_28672x8192",
}


def _draw(spec, shape):
    kind = spec[0]
    if kind == "normal":
        return normal(shape, spec[1], spec[2])
    if kind == "normal_outliers":
        return normal_outliers(shape, spec[1], spec[2], spec[3], spec[4])
    if kind == "student_t":
        return student_t(shape, spec[1], spec[2])
    if kind == "laplace_outlier_channels":
        return laplace_outlier_channels(shape, spec[1], spec[2], spec[3], spec[4])
    raise ValueError(kind)


def workload(name, rows_a=None, rows_b=None):
    """Draw (A [M][K], B [N][K]) bf16 bits for a named workload. rows_a/rows_b
    draw only that many leading rows (same values as the full draw's rows only
    for per-row-independent recipes; used for bounded CPU samples)."""
    name = ALIASES.get(name, name)
    w = WORKLOADS[name]
    M = w["M"] if rows_a is None else rows_a
    N = w["N"] if rows_b is None else rows_b
    A = _draw(w["a"], (M, w["K"]))
    B = _draw(w["b"], (N, w["K"])) if w["b"] is not None else None
    return A, B


def digest(bits):
    """Short content hash of an input tensor, logged next to results."""
    return hashlib.blake2b(np.ascontiguousarray(bits).tobytes(), digest_size=8).hexdigest()
