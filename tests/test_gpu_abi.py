"""The C ABI on a GPU: a HIP error that an earlier call of the caller left
pending on the thread is not reported as a failure of a libmx launch; the
roofline calibration library runs."""
import ctypes

import numpy as np
import pytest
import torch

import microscaling_precision_quantization_amd as mx
import oracle as orc
import synth
from gpu_helpers import dev_bf16, host, require_gpu

pytestmark = pytest.mark.gpu


def test_pending_error_is_not_charged_to_libmx():
    require_gpu()
    hip = ctypes.CDLL("libamdhip64.so")
    A = synth.normal((64, 256), 1.0, 71)
    x = dev_bf16(A)
    codes = torch.empty((64, 128), dtype=torch.uint8, device="cuda")
    scales = torch.empty((64, 8), dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    # An invalid device ordinal: the call fails and leaves its error pending
    # on this thread, without changing the current device.
    assert hip.hipSetDevice(9999) != 0
    st = mx.mx_quantize(mx.MX_FMT_MXFP4, 32, 0, 64, 256, ctypes.c_void_p(x.data_ptr()),
                        ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
                        None, None, 0, stream)
    hip.hipGetLastError()  # clear whatever is left before torch runs again
    assert st == mx.MX_OK, mx.mx_status_string(st)
    torch.cuda.synchronize()
    oc, os_, _ = orc.quantize(orc.FMT_MXFP4, A)
    assert np.array_equal(host(codes), oc) and np.array_equal(host(scales), os_)


def test_mfma_ceiling_calibration_runs():
    """libmx_calib.so (include/mx_calib.h) on the GPU: each kind launches,
    reports its FLOP count exactly, and a rate below the published peak."""
    require_gpu()
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    L = ctypes.CDLL(os.path.join(root, "microscaling_precision_quantization_amd", "libmx_calib.so"))
    f = L.mx_calib_mfma
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double)]
    for kind, threads, per_wave, peak in ((0, 256, 16 * 131072, 10.1e15), (1, 512, 8 * 32768, 2.5e15),
                                          (2, 512, 8 * 32768, 2.5e15)):
        ms, fl = ctypes.c_float(), ctypes.c_double()
        assert f(kind, 64, 200, 4, ctypes.byref(ms), ctypes.byref(fl)) == 0
        assert fl.value == 64 * (threads // 64) * 200 * per_wave
        assert ms.value > 0 and fl.value / (ms.value * 1e-3) < peak


def test_hbm_stream_calibration_runs():
    """mx_calib_stream on the GPU: each kind launches and reports exactly the
    bytes it moves per launch and a plausible rate."""
    require_gpu()
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    L = ctypes.CDLL(os.path.join(root, "microscaling_precision_quantization_amd", "libmx_calib.so"))
    g = L.mx_calib_stream
    g.restype = ctypes.c_int
    g.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double)]
    nbytes = (64 << 20) + 64     # not a whole number of 256-thread blocks
    for kind, moved in ((0, nbytes), (1, nbytes), (2, 2 * nbytes), (3, nbytes + nbytes // 4)):
        # one pass and grid-stride grids (one workgroup, ragged, large);
        # every unroll depth; plain and non-temporal accesses
        for wgs, unroll, nt in ((0, 1, 0), (0, 8, 1), (1, 8, 0), (333, 1, 1), (333, 2, 0), (2048, 4, 1)):
            ms, mv = ctypes.c_float(), ctypes.c_double()
            assert g(kind, nbytes, wgs, unroll, nt, 3, ctypes.byref(ms), ctypes.byref(mv)) == 0
            assert mv.value == moved
            assert ms.value > 0 and mv.value / (ms.value * 1e-3) < 50e12
