"""The C ABI on a GPU: a HIP error that an earlier call of the caller left
pending on the thread is not reported as a failure of a libmx launch."""
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
