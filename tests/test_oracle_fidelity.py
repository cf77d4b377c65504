"""Quantizer fidelity on workload-like data: the directions the pages report,
checked on the oracle as diagnostics (QSNR of the dequantized tensor, in dB),
not as parity.
 - NVFP4's finer scales (16 elements, E4M3 with a mantissa) reproduce a tensor
   better than MXFP4's (gist.science summary of "Unveiling the Potential of
   Quantization with MXFP4", section 1; produtoramaxvision page, format table),
   and 8-bit elements better still.
 - The overflow-aware scale rule lowers MXFP4's error (the same summary,
   section 2.A).
 - A Walsh-Hadamard rotation spreads an outlier's energy over its block
   (produtoramaxvision page, QuaRot / SpinQuant section), so MXFP4 on outlier
   channels gains.
Data: the activation recipe of the MXFP4 MLP-down workload (Laplace with 0.5%
of channels x100) on 128 rows, and the Student-t(4) recipe of the NVFP4 MLP-up
workload."""
import numpy as np

import oracle as orc
import synth


def _qsnr(x, y):
    return 10 * np.log10(np.sum(x * x) / np.sum((x - y) ** 2))


def _outlier_rows():
    return synth.laplace_outlier_channels((128, 12288), seed=1901, channel_seed=1902, frac=0.005,
                                          factor=100.0)


def test_format_order_on_outlier_activations():
    x = _outlier_rows()
    xf = synth.bf16_to_f32(x).astype(np.float64)
    q = {}
    for name, fmt in (("mxfp4", orc.FMT_MXFP4), ("nvfp4", orc.FMT_NVFP4), ("mxfp8", orc.FMT_MXFP8)):
        c, s, t = orc.quantize(fmt, x)
        q[name] = _qsnr(xf, orc.dequantize(fmt, c, s, t, *x.shape))
    assert q["mxfp8"] > q["nvfp4"] + 2.0 and q["nvfp4"] > q["mxfp4"] + 5.0, q


def test_nvfp4_beats_mxfp4_on_heavy_tails():
    x = synth.student_t((128, 3072), 4.0, 1903)
    xf = synth.bf16_to_f32(x).astype(np.float64)
    q = {}
    for name, fmt in (("mxfp4", orc.FMT_MXFP4), ("nvfp4", orc.FMT_NVFP4)):
        c, s, t = orc.quantize(fmt, x)
        q[name] = _qsnr(xf, orc.dequantize(fmt, c, s, t, *x.shape))
    assert q["nvfp4"] > q["mxfp4"] + 2.0, q


def test_oas_and_rotation_lower_mxfp4_error_on_outlier_channels():
    """OAS against the standard rule on the same data; the rotation against
    the standard rule on the rotated data (the rotation is orthonormal, so the
    error it leaves after rotating back is the same)."""
    x = _outlier_rows()
    xf = synth.bf16_to_f32(x).astype(np.float64)
    c, s, _ = orc.quantize(orc.FMT_MXFP4, x)
    base = _qsnr(xf, orc.dequantize(orc.FMT_MXFP4, c, s, 1.0, *x.shape))
    c, s = orc.quantize_ex(orc.FMT_MXFP4, x, orc.RULE_OAS, orc.ROT_NONE)
    oas = _qsnr(xf, orc.dequantize(orc.FMT_MXFP4, c, s, 1.0, *x.shape))
    xr = orc.wht32(x)
    c, s = orc.quantize_ex(orc.FMT_MXFP4, x, orc.RULE_CEIL, orc.ROT_WHT32)
    rot = _qsnr(synth.bf16_to_f32(xr).astype(np.float64), orc.dequantize(orc.FMT_MXFP4, c, s, 1.0, *x.shape))
    assert oas > base, (oas, base)
    assert rot > base + 0.3, (rot, base)
