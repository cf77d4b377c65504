"""The C ABI without a GPU: the library loads, exports every symbol that
include/mx.h declares, and rejects bad arguments with the documented status
before launching anything (these calls never reach HIP)."""
import ctypes
import os
import re

import pytest

import microscaling_precision_quantization_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "mx.h")).read()
    return set(re.findall(r"^\s*(?:mx_status|size_t|int|const char\*)\s+(mx_\w+)\s*\(", src, re.M))


def test_exports_every_declared_symbol():
    declared = _declared()
    assert declared == set(mx.EXPORTS)
    L = mx.lib()
    for name in declared:
        assert hasattr(L, name), name


def test_status_strings():
    assert mx.mx_status_string(mx.MX_OK) == "MX_OK"
    assert mx.mx_status_string(mx.MX_ERR_INVALID_ARG) == "MX_ERR_INVALID_ARG"
    assert mx.mx_status_string(mx.MX_ERR_UNSUPPORTED) == "MX_ERR_UNSUPPORTED"
    assert mx.mx_status_string(mx.MX_ERR_HIP) == "MX_ERR_HIP"


# Fake, 16-byte aligned "device" addresses: validation never dereferences them
# because every case below fails a check first.
P = ctypes.c_void_p(0x100000)
P2 = ctypes.c_void_p(0x200000)
MIS = ctypes.c_void_p(0x100004)


def q(fmt=mx.MX_FMT_MXFP4, block=32, rnd=0, rows=4, cols=64, x=P, codes=P, scales=P, ts=None,
      ws=None, wsb=0):
    return mx.mx_quantize(fmt, block, rnd, rows, cols, x, codes, scales, ts, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), mx.MX_ERR_INVALID_ARG),
    (dict(codes=None), mx.MX_ERR_INVALID_ARG),
    (dict(scales=None), mx.MX_ERR_INVALID_ARG),
    (dict(rows=0), mx.MX_ERR_INVALID_ARG),
    (dict(cols=-32), mx.MX_ERR_INVALID_ARG),
    (dict(cols=48), mx.MX_ERR_INVALID_ARG),               # not a multiple of 32
    (dict(x=MIS), mx.MX_ERR_INVALID_ARG),                 # misaligned
    (dict(ts=P), mx.MX_ERR_INVALID_ARG),                  # tensor scale is NVFP4 only
    (dict(block=16), mx.MX_ERR_UNSUPPORTED),              # MX needs 32
    (dict(rnd=1), mx.MX_ERR_UNSUPPORTED),                 # only RNE
    (dict(fmt=mx.MX_FMT_BF16), mx.MX_ERR_UNSUPPORTED),
    (dict(fmt=9), mx.MX_ERR_UNSUPPORTED),
    (dict(fmt=mx.MX_FMT_NVFP4, block=32), mx.MX_ERR_UNSUPPORTED),
    (dict(fmt=mx.MX_FMT_NVFP4, block=16), mx.MX_ERR_INVALID_ARG),  # no tensor scale
    (dict(fmt=mx.MX_FMT_NVFP4, block=16, ts=P), mx.MX_ERR_INVALID_ARG),  # no workspace
    (dict(fmt=mx.MX_FMT_NVFP4, block=16, ts=P, ws=P2, wsb=16), mx.MX_ERR_INVALID_ARG),  # too small
    (dict(fmt=mx.MX_FMT_NVFP4, block=16, cols=40, ts=P, ws=P2, wsb=1 << 20), mx.MX_ERR_INVALID_ARG),
    (dict(fmt=mx.MX_FMT_MXFP4_MBS, cols=64), mx.MX_ERR_INVALID_ARG),    # macro blocks of 128
    (dict(fmt=mx.MX_FMT_MXFP4_MBS, cols=128, ts=P), mx.MX_ERR_INVALID_ARG),
    (dict(fmt=mx.MX_FMT_MXFP4_MBS, cols=128, block=16), mx.MX_ERR_UNSUPPORTED),
    (dict(fmt=mx.MX_FMT_MXFP4_MBS16, cols=128, block=32), mx.MX_ERR_UNSUPPORTED),  # base 16
    (dict(fmt=mx.MX_FMT_MXFP4_MBS16, cols=64, block=16), mx.MX_ERR_INVALID_ARG),
    (dict(fmt=mx.MX_FMT_MXFP4_MBS16, cols=128, block=16, ts=P), mx.MX_ERR_INVALID_ARG),
])
def test_quantize_rejects(kw, status):
    assert q(**kw) == status


def qx(fmt=mx.MX_FMT_MXFP4, block=32, rnd=0, rule=0, rot=0, rows=4, cols=64, x=P, codes=P, scales=P,
       layout=mx.MX_LAYOUT_ROWS):
    return mx.mx_quantize_ex(fmt, block, rnd, rule, rot, rows, cols, x, codes, scales, None, layout)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), mx.MX_ERR_INVALID_ARG),
    (dict(scales=MIS), mx.MX_ERR_INVALID_ARG),
    (dict(cols=48), mx.MX_ERR_INVALID_ARG),
    (dict(fmt=mx.MX_FMT_MXFP8, rule=mx.MX_SCALE_OAS), mx.MX_ERR_UNSUPPORTED),  # OAS is MXFP4's
    (dict(fmt=mx.MX_FMT_NVFP4, block=16), mx.MX_ERR_UNSUPPORTED),
    (dict(fmt=mx.MX_FMT_NVFP4, block=16, rot=mx.MX_ROTATE_WHT32), mx.MX_ERR_UNSUPPORTED),
    (dict(rule=2), mx.MX_ERR_UNSUPPORTED),
    (dict(rot=2), mx.MX_ERR_UNSUPPORTED),
    (dict(rnd=1), mx.MX_ERR_UNSUPPORTED),
    (dict(fmt=mx.MX_FMT_MXFP4_MBS, cols=128), mx.MX_ERR_UNSUPPORTED),  # MBS is its own format
    (dict(fmt=mx.MX_FMT_MXFP4_MBS16, block=16, cols=128), mx.MX_ERR_UNSUPPORTED),
    (dict(layout=5), mx.MX_ERR_UNSUPPORTED),
    (dict(layout=mx.MX_LAYOUT_KPANEL, fmt=mx.MX_FMT_MXFP8_E5M2, cols=256), mx.MX_ERR_UNSUPPORTED),
    (dict(layout=mx.MX_LAYOUT_KPANEL, fmt=mx.MX_FMT_MXFP8, cols=96), mx.MX_ERR_INVALID_ARG),  # cols % 64
    (dict(layout=mx.MX_LAYOUT_KPANEL, cols=128), mx.MX_ERR_INVALID_ARG),          # cols % 256
    (dict(layout=mx.MX_LAYOUT_KPANEL, cols=256 * 65536), mx.MX_ERR_INVALID_ARG),  # > 65535 panels
    (dict(layout=mx.MX_LAYOUT_KPANEL, rows=1 << 23, cols=512), mx.MX_ERR_INVALID_ARG),  # 2^31 bytes
])
def test_quantize_ex_rejects(kw, status):
    assert qx(**kw) == status


def ql(fmt=mx.MX_FMT_MXFP8, block=32, rnd=0, rows=4, cols=256, x=P, codes=P, scales=P, ts=None,
       ws=None, wsb=0, layout=mx.MX_LAYOUT_KPANEL):
    return mx.mx_quantize_layout(fmt, block, rnd, rows, cols, x, codes, scales, ts, ws, wsb, None,
                                 layout)


@pytest.mark.parametrize("kw,status", [
    (dict(layout=5), mx.MX_ERR_UNSUPPORTED),
    (dict(fmt=mx.MX_FMT_MXFP4_MBS, cols=256), mx.MX_ERR_UNSUPPORTED),             # no K panels
    (dict(fmt=mx.MX_FMT_MXFP4_MBS16, block=16, cols=256), mx.MX_ERR_UNSUPPORTED),
    (dict(fmt=mx.MX_FMT_MXFP8, block=16), mx.MX_ERR_UNSUPPORTED),
    (dict(cols=96), mx.MX_ERR_INVALID_ARG),                                         # cols % 64
    (dict(fmt=mx.MX_FMT_MXFP4, cols=192), mx.MX_ERR_INVALID_ARG),                   # cols % 256
    (dict(fmt=mx.MX_FMT_MXFP6_E3M2, cols=64 * 65536), mx.MX_ERR_INVALID_ARG),       # > 65535 panels
    (dict(rows=1 << 24, cols=128), mx.MX_ERR_INVALID_ARG),                          # 2^31 code bytes
    (dict(fmt=mx.MX_FMT_NVFP4, block=16), mx.MX_ERR_INVALID_ARG),                   # no tensor scale
    (dict(fmt=mx.MX_FMT_NVFP4, block=16, ts=P2), mx.MX_ERR_INVALID_ARG),            # no workspace
    (dict(ts=P2), mx.MX_ERR_INVALID_ARG),                                           # MX takes none
    (dict(x=None), mx.MX_ERR_INVALID_ARG),
    (dict(scales=MIS), mx.MX_ERR_INVALID_ARG),
])
def test_quantize_layout_rejects(kw, status):
    assert ql(**kw) == status


def test_dequantize_rejects():
    d = mx.mx_dequantize
    assert d(1, 32, 0, 4, 64, P, P, None, 0, None, None) == mx.MX_ERR_INVALID_ARG  # y null
    assert d(1, 32, 0, 4, 64, P, P, None, 7, P2, None) == mx.MX_ERR_UNSUPPORTED  # out dtype
    assert d(3, 16, 0, 4, 64, P, P, None, 0, P2, None) == mx.MX_ERR_INVALID_ARG  # NVFP4 needs ts
    assert d(2, 32, 0, 4, 64, P, P, P, 0, P2, None) == mx.MX_ERR_INVALID_ARG  # MX takes no ts
    assert d(2, 32, 0, 4, 64, P, MIS, None, 0, P2, None) == mx.MX_ERR_INVALID_ARG
    assert d(2, 16, 0, 4, 64, P, P, None, 0, P2, None) == mx.MX_ERR_UNSUPPORTED
    assert d(6, 32, 0, 4, 96, P, P, None, 0, P2, None) == mx.MX_ERR_INVALID_ARG  # MBS: cols % 128
    assert d(6, 32, 0, 4, 128, P, P, P, 0, P2, None) == mx.MX_ERR_INVALID_ARG  # MBS takes no ts
    assert d(7, 32, 0, 4, 128, P, P, None, 0, P2, None) == mx.MX_ERR_UNSUPPORTED  # MBS16: block 16
    assert d(7, 16, 0, 4, 112, P, P, None, 0, P2, None) == mx.MX_ERR_INVALID_ARG  # cols % 128


def g(fa=1, fb=1, block=32, rnd=0, M=64, N=64, K=128, a=P, sa=P, ta=None, b=P, sb=P, tb=None,
      od=0, c=P2, ldc=64, ws=None, wsb=0):
    return mx.mx_gemm(fa, fb, block, rnd, M, N, K, a, sa, ta, b, sb, tb, od, c, ldc, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(fa=1, fb=2), mx.MX_ERR_UNSUPPORTED),                  # mixed formats
    (dict(fa=0, fb=2), mx.MX_ERR_UNSUPPORTED),                  # bf16 only with MXFP4 weights
    (dict(fa=3, fb=3, block=32), mx.MX_ERR_UNSUPPORTED),
    (dict(block=16), mx.MX_ERR_UNSUPPORTED),
    (dict(rnd=2), mx.MX_ERR_UNSUPPORTED),
    (dict(od=5), mx.MX_ERR_UNSUPPORTED),
    (dict(M=0), mx.MX_ERR_INVALID_ARG),
    (dict(K=96 + 16), mx.MX_ERR_INVALID_ARG),                   # K % 32
    (dict(ldc=32), mx.MX_ERR_INVALID_ARG),                      # ldc < N
    (dict(a=None), mx.MX_ERR_INVALID_ARG),
    (dict(sa=None), mx.MX_ERR_INVALID_ARG),
    (dict(sb=None), mx.MX_ERR_INVALID_ARG),
    (dict(c=MIS), mx.MX_ERR_INVALID_ARG),
    (dict(ta=P), mx.MX_ERR_INVALID_ARG),                        # MX takes no tensor scales
    (dict(fa=3, fb=3, block=16), mx.MX_ERR_INVALID_ARG),        # NVFP4 needs tensor scales
    (dict(fa=0, fb=1, sa=P), mx.MX_ERR_INVALID_ARG),            # bf16 A has no scales
    (dict(fa=0, fb=1, sa=None, M=16, N=28672, K=8192), mx.MX_ERR_INVALID_ARG),  # no workspace
    (dict(fa=0, fb=1, sa=None, M=16, N=64, K=65536 + 32, ws=P2, wsb=1 << 40), mx.MX_ERR_INVALID_ARG),  # W4A16 K limit
    (dict(fa=6, fb=6, K=160), mx.MX_ERR_INVALID_ARG),           # MBS: K % 128
    (dict(fa=6, fb=1), mx.MX_ERR_UNSUPPORTED),                  # MBS pairs with MBS only
    (dict(fa=6, fb=6, block=16), mx.MX_ERR_UNSUPPORTED),
    (dict(fa=6, fb=6, ta=P), mx.MX_ERR_INVALID_ARG),
    (dict(fa=7, fb=7, block=32), mx.MX_ERR_UNSUPPORTED),        # MBS16 has block 16
    (dict(fa=7, fb=6, block=16), mx.MX_ERR_UNSUPPORTED),        # base blocks differ
    (dict(fa=7, fb=7, block=16, K=160), mx.MX_ERR_INVALID_ARG), # K % 128
])
def test_gemm_rejects(kw, status):
    assert g(**kw) == status


def test_workspace_sizes():
    assert mx.mx_quantize_workspace_bytes(mx.MX_FMT_MXFP4, 100, 64) == 0
    assert mx.mx_quantize_workspace_bytes(mx.MX_FMT_NVFP4, 100, 64) > 0
    assert mx.mx_gemm_workspace_bytes(1, 1, 4608, 3072, 12288) == 0
    w = mx.mx_gemm_workspace_bytes(0, 1, 16, 28672, 8192)
    assert w > 0 and w % (16 * 28672 * 4) == 0


def gx(layout=mx.MX_LAYOUT_KPANEL, fa=1, fb=1, block=32, rnd=0, M=64, N=64, K=256, a=P, sa=P,
       ta=None, b=P, sb=P, tb=None, od=0, c=P2, ldc=64, ws=None, wsb=0, a_layout=mx.MX_LAYOUT_ROWS):
    return mx.mx_gemm_ex(fa, fb, block, rnd, M, N, K, a, sa, ta, b, sb, tb, od, c, ldc, ws, wsb,
                         None, a_layout, layout)


@pytest.mark.parametrize("kw,status", [
    (dict(layout=7), mx.MX_ERR_UNSUPPORTED),                    # unknown layout
    (dict(fa=2, fb=2), mx.MX_ERR_UNSUPPORTED),                  # MXFP8: both K-panel or neither
    (dict(fa=3, fb=3, block=16, ta=P2, tb=P2), mx.MX_ERR_UNSUPPORTED),  # NVFP4 likewise
    (dict(fa=2, fb=2, a_layout=mx.MX_LAYOUT_KPANEL, K=96), mx.MX_ERR_INVALID_ARG),  # K % 64
    (dict(fa=0, fb=1, sa=None, M=16), mx.MX_ERR_UNSUPPORTED),   # not for W4A16
    (dict(fa=6, fb=6), mx.MX_ERR_UNSUPPORTED),                  # not for MBS
    (dict(K=128 + 32), mx.MX_ERR_INVALID_ARG),                  # K % 256
    (dict(K=128), mx.MX_ERR_INVALID_ARG),
    (dict(N=1 << 20, ldc=1 << 20, K=1 << 12), mx.MX_ERR_INVALID_ARG),  # N * K / 2 >= 2^31
    (dict(b=None), mx.MX_ERR_INVALID_ARG),
    (dict(sb=MIS), mx.MX_ERR_INVALID_ARG),
    (dict(layout=mx.MX_LAYOUT_ROWS, fa=1, fb=2), mx.MX_ERR_UNSUPPORTED),  # ROWS is mx_gemm
    (dict(layout=mx.MX_LAYOUT_ROWS, a_layout=9), mx.MX_ERR_UNSUPPORTED),  # unknown A layout
    (dict(layout=mx.MX_LAYOUT_ROWS, a_layout=mx.MX_LAYOUT_KPANEL, fa=2, fb=2), mx.MX_ERR_UNSUPPORTED),
    (dict(layout=mx.MX_LAYOUT_ROWS, a_layout=mx.MX_LAYOUT_KPANEL, K=128), mx.MX_ERR_INVALID_ARG),
    (dict(a_layout=mx.MX_LAYOUT_KPANEL, M=1 << 20, K=1 << 12), mx.MX_ERR_INVALID_ARG),  # M K / 2 >= 2^31
])
def test_gemm_ex_rejects(kw, status):
    assert gx(**kw) == status


def pk(fmt=mx.MX_FMT_MXFP4, block=32, rows=4, cols=256, codes=P, scales=ctypes.c_void_p(0x110000),
       pc=P2, ps=ctypes.c_void_p(0x210000)):
    return mx.mx_pack(fmt, block, rows, cols, codes, scales, pc, ps, None)


@pytest.mark.parametrize("kw,status", [
    (dict(fmt=mx.MX_FMT_MXFP4_MBS), mx.MX_ERR_UNSUPPORTED),     # no K panels
    (dict(fmt=mx.MX_FMT_NVFP4, block=32), mx.MX_ERR_UNSUPPORTED),
    (dict(block=16), mx.MX_ERR_UNSUPPORTED),
    (dict(fmt=mx.MX_FMT_MXFP8, cols=96), mx.MX_ERR_INVALID_ARG),   # cols % 64
    (dict(rows=0), mx.MX_ERR_INVALID_ARG),
    (dict(cols=128), mx.MX_ERR_INVALID_ARG),                    # cols % 256
    (dict(rows=1 << 23, cols=1 << 9), mx.MX_ERR_INVALID_ARG),    # rows * cols / 2 >= 2^31
    (dict(codes=None), mx.MX_ERR_INVALID_ARG),
    (dict(ps=MIS), mx.MX_ERR_INVALID_ARG),
    (dict(pc=ctypes.c_void_p(0x100100)), mx.MX_ERR_INVALID_ARG),  # output overlaps the codes
    (dict(ps=ctypes.c_void_p(0x110000)), mx.MX_ERR_INVALID_ARG),  # output overlaps the scales
])
def test_pack_rejects(kw, status):
    assert pk(**kw) == status


def _visible_gpus():
    """(status, count) of hipGetDeviceCount from the HIP runtime libmx links."""
    hip = ctypes.CDLL("libamdhip64.so")
    n = ctypes.c_int(0)
    rc = hip.hipGetDeviceCount(ctypes.byref(n))
    return rc, n.value


def test_launch_failure_reports_hip_error():
    """Valid arguments with no GPU visible: the argument checks pass, the
    kernel launch itself fails, and the call returns MX_ERR_HIP with that
    launch's hipError_t saved for mx_last_hip_error (per thread). Only runs
    where no GPU is visible, so the fake pointers never reach a kernel."""
    rc, count = _visible_gpus()
    if rc == 0 and count > 0:
        pytest.skip("a GPU is visible: the launch would not fail")
    for call in (lambda: q(),
                 lambda: mx.mx_quantize_ex(mx.MX_FMT_MXFP4, 32, 0, mx.MX_SCALE_OAS, mx.MX_ROTATE_WHT32,
                                           4, 256, P, P, P, None, mx.MX_LAYOUT_KPANEL),
                 lambda: mx.mx_dequantize(mx.MX_FMT_MXFP8, 32, 0, 4, 64, P, P, None, mx.MX_OUT_BF16,
                                          P2, None),
                 lambda: mx.mx_gemm(mx.MX_FMT_MXFP4, mx.MX_FMT_MXFP4, 32, 0, 64, 64, 256, P, P, None,
                                    P2, P2, None, mx.MX_OUT_F32, P, 64, None, 0, None),
                 # (needs the library's scratch: the device lookup itself fails)
                 lambda: mx.mx_gemm_noalloc(mx.MX_FMT_BF16, mx.MX_FMT_MXFP4, 32, 0, 16, 4096, 8192,
                                            P, None, None, P2, P2, None, mx.MX_OUT_BF16, P, 4096,
                                            None)):
        assert call() == mx.MX_ERR_HIP
        err = mx.mx_last_hip_error()
        assert err != 0
        # hipErrorNoDevice (100) or another "no usable device" code, as
        # hipGetDeviceCount itself reported
        assert err == rc or rc == 0, (err, rc)


def test_gemm_noalloc_rejects():
    """mx_gemm_noalloc checks like mx_gemm, and refuses a W4A16 shape whose
    split-K partials (4 M N ceil(K / 2048) bytes) exceed its 8 MiB scratch
    before touching HIP."""
    n = mx.mx_gemm_noalloc
    assert n(1, 2, 32, 0, 64, 64, 128, P, P, None, P2, P2, None, 0, P, 64, None) == mx.MX_ERR_UNSUPPORTED
    assert n(1, 1, 32, 0, 0, 64, 128, P, P, None, P2, P2, None, 0, P, 64, None) == mx.MX_ERR_INVALID_ARG
    assert n(0, 1, 32, 0, 64, 28672, 8192, P, None, None, P2, P2, None, 1, P, 28672, None) == \
        mx.MX_ERR_INVALID_ARG  # 29 MB of partials
    assert n(0, 1, 32, 0, 16, 64, 65536 + 32, P, None, None, P2, P2, None, 1, P, 64, None) == \
        mx.MX_ERR_INVALID_ARG  # W4A16 K limit


def test_calib_library_exports_and_rejects():
    """libmx_calib.so (include/mx_calib.h) loads, exports what its header
    declares, and refuses bad arguments before any HIP call."""
    src = open(os.path.join(ROOT, "include", "mx_calib.h")).read()
    declared = set(re.findall(r"^\s*int\s+(mx_\w+)\s*\(", src, re.M))
    assert declared == {"mx_calib_mfma", "mx_calib_stream"}
    L = ctypes.CDLL(os.path.join(ROOT, "microscaling_precision_quantization_amd", "libmx_calib.so"))
    f = L.mx_calib_mfma
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double)]
    ms, fl = ctypes.c_float(), ctypes.c_double()
    assert f(3, 1, 1, 1, ctypes.byref(ms), ctypes.byref(fl)) == -1
    assert f(0, 0, 1, 1, ctypes.byref(ms), ctypes.byref(fl)) == -1
    assert f(0, 1, 1, 1, None, ctypes.byref(fl)) == -1
    g = L.mx_calib_stream
    g.restype = ctypes.c_int
    g.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double)]
    ok = (0, 1 << 20, 64, 4, 0, 2)
    for bad in ((4, 1 << 20, 64, 4, 0, 2), (-1, 1 << 20, 64, 4, 0, 2), (0, 4000, 64, 4, 0, 2),
                (0, (1 << 20) + 16, 64, 4, 0, 2), (0, (1 << 36) + 64, 64, 4, 0, 2),
                (0, 1 << 20, -1, 4, 0, 2), (0, 1 << 20, 65536, 4, 0, 2), (0, 1 << 20, 64, 3, 0, 2),
                (0, 1 << 20, 64, 16, 0, 2), (0, 1 << 20, 64, 4, 2, 2), (0, 1 << 20, 64, 4, 0, 0)):
        assert g(*bad, ctypes.byref(ms), ctypes.byref(fl)) == -1, bad
    assert g(*ok, None, ctypes.byref(fl)) == -1
    assert g(*ok, ctypes.byref(ms), None) == -1
