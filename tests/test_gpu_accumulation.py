"""GPU accumulation bound on operands built to make every partial sum of a
long K chain round the same way (chain_operands.py, pinned on the CPU by
test_chain_operands.py): the fp32 output stays within
2^-18 * sum_k |a_k b_k| of the oracle's exact sum at K = 12288 (MXFP4, the
256 x 256-tile kernel), K = 12416 (MXFP4, the 128 x 128-tile kernel) and
K = 3072 (MXFP8 and NVFP4 on the 16-bit path), where a plain fp32 chain over
the kernels' K groups is 1.5 - 3x outside it."""
import numpy as np
import pytest
import torch

import chain_operands as co
import microscaling_precision_quantization_amd as mx
import oracle as orc
from gpu_helpers import check_gemm, dev_u8, host, require_gpu

pytestmark = pytest.mark.gpu

ROWS = 96  # rows of A and of B: all identical, so every output is the same sum


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _case(name):
    if name == "mxfp4_tile256":
        K = 12288
        c, s, _ = co.mxfp4(K, "tile256")
        return "mxfp4", orc.FMT_MXFP4, mx.MX_FMT_MXFP4, K, c, s
    if name == "mxfp4_tile128":
        K = 12288 + 128
        c, s, _ = co.mxfp4(K, "tile128")
        return "mxfp4", orc.FMT_MXFP4, mx.MX_FMT_MXFP4, K, c, s
    if name == "mxfp8":
        K = 3072
        c, s = co.mxfp8(K)
        return "mxfp8", orc.FMT_MXFP8, mx.MX_FMT_MXFP8, K, c, s
    K = 3072
    c, s = co.nvfp4(K)
    return "nvfp4", orc.FMT_NVFP4, mx.MX_FMT_NVFP4, K, c, s


@pytest.mark.parametrize("name", ["mxfp4_tile256", "mxfp4_tile128", "mxfp8", "nvfp4"])
def test_one_direction_chain_f32(name):
    fmt, ofmt, mfmt, K, codes, scales = _case(name)
    print(f"accumulation case {name}: K={K}", flush=True)
    A = co.tile(codes, ROWS)
    S_ = co.tile(scales, ROWS)
    ts = torch.ones(1, dtype=torch.float32, device="cuda") if fmt == "nvfp4" else None
    q = mx.QTensor(mfmt, ROWS, K, dev_u8(A), dev_u8(S_), ts)
    got = host(mx.gemm(q, q, torch.float32))
    C, S = orc.gemm(ofmt, ofmt, ROWS, ROWS, K, A, S_, 1.0, A, S_, 1.0)
    rel = check_gemm(got, C, S, "f32", f"{name} one-direction chain")
    print(f"{name}: max |err| / sum|ab| = {rel:.3g} (bound {2.0**-18:.3g})")
