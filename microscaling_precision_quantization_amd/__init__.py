"""Python binding for libmx: microscaling (MX / NVFP4) quantization and the
block-scaled GEMM on AMD Instinct MI355X (gfx950).

Two layers:
  * mx_quantize, mx_dequantize, mx_gemm, ... : the C ABI (include/mx.h) under
    the same names, taking integers and raw device pointers;
  * quantize, dequantize, gemm : torch conveniences that allocate outputs on
    the input's device and pass data_ptr() plus the current HIP stream.

Every step of the computation runs in libmx's HIP kernels. If libmx.so is not
built, loading fails with an error; there is no fallback path.
"""
import ctypes
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmx.so")

MX_FMT_BF16, MX_FMT_MXFP4, MX_FMT_MXFP8, MX_FMT_NVFP4 = 0, 1, 2, 3
MX_FMT_MXFP8_E5M2, MX_FMT_MXFP6_E3M2, MX_FMT_MXFP4_MBS, MX_FMT_MXFP4_MBS16 = 4, 5, 6, 7
MX_ROUND_RNE = 0
MX_SCALE_CEIL, MX_SCALE_OAS = 0, 1
MX_ROTATE_NONE, MX_ROTATE_WHT32 = 0, 1
MX_OUT_F32, MX_OUT_BF16 = 0, 1
MX_OK, MX_ERR_INVALID_ARG, MX_ERR_UNSUPPORTED, MX_ERR_HIP = 0, 1, 2, 3
MX_LAYOUT_ROWS, MX_LAYOUT_KPANEL = 0, 1

FORMATS = {"mxfp4": MX_FMT_MXFP4, "mxfp8": MX_FMT_MXFP8, "nvfp4": MX_FMT_NVFP4, "bf16": MX_FMT_BF16,
           "mxfp8_e5m2": MX_FMT_MXFP8_E5M2, "mxfp6_e3m2": MX_FMT_MXFP6_E3M2,
           "mxfp4_mbs": MX_FMT_MXFP4_MBS, "mxfp4_mbs16": MX_FMT_MXFP4_MBS16}
BLOCK = {MX_FMT_MXFP4: 32, MX_FMT_MXFP8: 32, MX_FMT_NVFP4: 16, MX_FMT_BF16: 32,
         MX_FMT_MXFP8_E5M2: 32, MX_FMT_MXFP6_E3M2: 32, MX_FMT_MXFP4_MBS: 32,
         MX_FMT_MXFP4_MBS16: 16}
MBS_FORMATS = (MX_FMT_MXFP4_MBS, MX_FMT_MXFP4_MBS16)


def code_cols(fmt, cols):
    """Bytes of codes per row of `cols` elements."""
    if fmt in (MX_FMT_MXFP8, MX_FMT_MXFP8_E5M2):
        return cols
    if fmt == MX_FMT_MXFP6_E3M2:
        return cols * 3 // 4
    return cols // 2

def scale_shape(fmt, rows, cols):
    """Shape of the scales tensor: [rows][cols/block]; for MXFP4-MBS (block 32)
    and MXFP4-MBS16 (block 16) one flat buffer, the E8M0 plane
    [rows][cols/block] followed by the macro mantissa plane [rows][cols/128]."""
    if fmt in MBS_FORMATS:
        return (rows * (cols // BLOCK[fmt]) + rows * (cols // 128),)
    return (rows, cols // BLOCK[fmt])


def mbs_planes(scales, rows, cols, block=32):
    """Views of an MXFP4-MBS (block 32) or MBS16 (block 16) scales buffer:
    (E8M0 [rows][cols/block], macro mantissas [rows][cols/128])."""
    n = rows * (cols // block)
    return scales[:n].view(rows, cols // block), scales[n:].view(rows, cols // 128)


# Symbols declared in include/mx.h.
EXPORTS = ("mx_quantize", "mx_quantize_workspace_bytes", "mx_quantize_ex", "mx_quantize_layout",
           "mx_dequantize",
           "mx_gemm", "mx_gemm_workspace_bytes", "mx_last_hip_error", "mx_status_string",
           "mx_pack", "mx_gemm_ex", "mx_gemm_noalloc")

_lib = None


class MXError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        msg = f"{what}: {status_string(status)}"
        if status == MX_ERR_HIP:
            msg += f" (hipError_t {mx_last_hip_error()})"
        super().__init__(msg)


def lib():
    """Load libmx.so (built by build.py). Raises if it is missing.
    MX_LIBRARY, if set, names another build of the same sources to load
    instead (the host-sanitizer build, in that CPU test's child process)."""
    global _lib
    if _lib is None:
        path = os.environ.get("MX_LIBRARY") or LIB_PATH
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run "
                               "microscaling_precision_quantization_amd.build.build()")
        L = ctypes.CDLL(path)
        P, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        L.mx_quantize.restype = i32
        L.mx_quantize.argtypes = [i32, i32, i32, i64, i64, P, P, P, P, P, sz, P]
        L.mx_quantize_ex.restype = i32
        L.mx_quantize_ex.argtypes = [i32, i32, i32, i32, i32, i64, i64, P, P, P, P, i32]
        L.mx_quantize_layout.restype = i32
        L.mx_quantize_layout.argtypes = [i32, i32, i32, i64, i64, P, P, P, P, P, sz, P, i32]
        L.mx_quantize_workspace_bytes.restype = sz
        L.mx_quantize_workspace_bytes.argtypes = [i32, i64, i64]
        L.mx_dequantize.restype = i32
        L.mx_dequantize.argtypes = [i32, i32, i32, i64, i64, P, P, P, i32, P, P]
        L.mx_gemm.restype = i32
        L.mx_gemm.argtypes = [i32, i32, i32, i32, i64, i64, i64, P, P, P, P, P, P, i32, P, i64,
                              P, sz, P]
        L.mx_gemm_ex.restype = i32
        L.mx_gemm_ex.argtypes = [i32, i32, i32, i32, i64, i64, i64, P, P, P, P, P, P, i32, P, i64,
                                 P, sz, P, i32, i32]
        L.mx_gemm_noalloc.restype = i32
        L.mx_gemm_noalloc.argtypes = [i32, i32, i32, i32, i64, i64, i64, P, P, P, P, P, P, i32, P,
                                      i64, P]
        L.mx_pack.restype = i32
        L.mx_pack.argtypes = [i32, i32, i64, i64, P, P, P, P, P]
        L.mx_gemm_workspace_bytes.restype = sz
        L.mx_gemm_workspace_bytes.argtypes = [i32, i32, i64, i64, i64]
        L.mx_last_hip_error.restype = i32
        L.mx_last_hip_error.argtypes = []
        L.mx_status_string.restype = ctypes.c_char_p
        L.mx_status_string.argtypes = [i32]
        _lib = L
    return _lib


# ---- the C ABI, same names ---------------------------------------------------
def mx_quantize(fmt, block, rnd, rows, cols, x, codes, scales, tensor_scale, workspace,
                workspace_bytes, stream):
    return lib().mx_quantize(fmt, block, rnd, rows, cols, x, codes, scales, tensor_scale,
                             workspace, workspace_bytes, stream)


def mx_quantize_ex(fmt, block, rnd, rule, rot, rows, cols, x, codes, scales, stream, layout):
    return lib().mx_quantize_ex(fmt, block, rnd, rule, rot, rows, cols, x, codes, scales, stream,
                                layout)


def mx_quantize_layout(fmt, block, rnd, rows, cols, x, codes, scales, tensor_scale, workspace,
                       workspace_bytes, stream, layout):
    return lib().mx_quantize_layout(fmt, block, rnd, rows, cols, x, codes, scales, tensor_scale,
                                    workspace, workspace_bytes, stream, layout)


def mx_quantize_workspace_bytes(fmt, rows, cols):
    return lib().mx_quantize_workspace_bytes(fmt, rows, cols)


def mx_dequantize(fmt, block, rnd, rows, cols, codes, scales, tensor_scale, out_dtype, y, stream):
    return lib().mx_dequantize(fmt, block, rnd, rows, cols, codes, scales, tensor_scale,
                               out_dtype, y, stream)


def mx_gemm(fmt_a, fmt_b, block, rnd, M, N, K, a, a_scales, a_ts, b, b_scales, b_ts, out_dtype,
            c, ldc, workspace, workspace_bytes, stream):
    return lib().mx_gemm(fmt_a, fmt_b, block, rnd, M, N, K, a, a_scales, a_ts, b, b_scales, b_ts,
                         out_dtype, c, ldc, workspace, workspace_bytes, stream)


def mx_gemm_ex(fmt_a, fmt_b, block, rnd, M, N, K, a, a_scales, a_ts, b, b_scales, b_ts, out_dtype,
               c, ldc, workspace, workspace_bytes, stream, a_layout, b_layout):
    return lib().mx_gemm_ex(fmt_a, fmt_b, block, rnd, M, N, K, a, a_scales, a_ts, b, b_scales,
                            b_ts, out_dtype, c, ldc, workspace, workspace_bytes, stream, a_layout,
                            b_layout)


def mx_gemm_noalloc(fmt_a, fmt_b, block, rnd, M, N, K, a, a_scales, a_ts, b, b_scales, b_ts,
                    out_dtype, c, ldc, stream):
    return lib().mx_gemm_noalloc(fmt_a, fmt_b, block, rnd, M, N, K, a, a_scales, a_ts, b, b_scales,
                                 b_ts, out_dtype, c, ldc, stream)


def mx_pack(fmt, block, rows, cols, codes, scales, packed_codes, packed_scales, stream):
    return lib().mx_pack(fmt, block, rows, cols, codes, scales, packed_codes, packed_scales, stream)


def mx_gemm_workspace_bytes(fmt_a, fmt_b, M, N, K):
    return lib().mx_gemm_workspace_bytes(fmt_a, fmt_b, M, N, K)


def mx_last_hip_error():
    return lib().mx_last_hip_error()


def mx_status_string(status):
    return lib().mx_status_string(status).decode()


def status_string(status):
    return mx_status_string(status)


# ---- torch conveniences --------------------------------------------------------
@dataclass
class QTensor:
    """A block-quantized [rows][cols] tensor: codes, scales and (NVFP4) the
    fp32 tensor scale, all device tensors; layout MX_LAYOUT_KPANEL after pack()."""
    fmt: int
    rows: int
    cols: int
    codes: "object"
    scales: "object"
    tensor_scale: "object" = None
    layout: int = MX_LAYOUT_ROWS

    @property
    def block(self):
        return BLOCK[self.fmt]


def _check_qtensor(q, what):
    """The kernels read exactly the bytes a QTensor's shape implies: refuse
    buffers of another size, type or layout in memory."""
    import torch
    if q.fmt not in BLOCK or q.fmt == MX_FMT_BF16 or q.cols % BLOCK[q.fmt] != 0:
        raise ValueError(f"{what}: not a quantized tensor of a supported format")
    need_c = q.rows * code_cols(q.fmt, q.cols)
    need_s = 1
    for d in scale_shape(q.fmt, q.rows, q.cols):
        need_s *= d
    for t, n, name in ((q.codes, need_c, "codes"), (q.scales, need_s, "scales")):
        if t.dtype != torch.uint8 or not t.is_contiguous() or t.numel() != n:
            raise ValueError(f"{what}: {name} must be a contiguous uint8 tensor of {n} bytes")
    if q.fmt == MX_FMT_NVFP4:
        ts = q.tensor_scale
        if ts is None or ts.dtype != torch.float32 or ts.numel() < 1:
            raise ValueError(f"{what}: NVFP4 needs a float32 tensor scale")


def _fmt_id(fmt):
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def _stream(torch, device, *tensors):
    """The current stream of `device`, after checking that the device is a GPU
    and that every tensor handed to the kernels lives on it (a host or
    foreign-device pointer must never reach a kernel)."""
    if device.type != "cuda":
        raise ValueError(f"libmx runs on GPU tensors; got a tensor on {device}")
    for t in tensors:
        if t is not None and t.device != device:
            raise ValueError(f"all tensors must be on {device}; got one on {t.device}")
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(status, what):
    if status != MX_OK:
        raise MXError(status, what)


SCALE_RULES = {"ceil": MX_SCALE_CEIL, "oas": MX_SCALE_OAS}
ROTATIONS = {None: MX_ROTATE_NONE, "none": MX_ROTATE_NONE, "wht32": MX_ROTATE_WHT32}


LAYOUTS = {"rows": MX_LAYOUT_ROWS, "kpanel": MX_LAYOUT_KPANEL}


def quantize(x, fmt, scale_rule="ceil", rotation=None, layout="rows"):
    """Quantize a contiguous bf16 [rows][cols] device tensor. scale_rule "oas"
    (MXFP4) and rotation "wht32" (MXFP4, MXFP8) select mx_quantize_ex, with
    the layout given; otherwise layout "kpanel" (MXFP4, MXFP8, E5M2, E3M2,
    NVFP4) selects mx_quantize_layout."""
    import torch
    f = _fmt_id(fmt)
    lay = LAYOUTS[layout]
    if scale_rule != "ceil" or rotation not in (None, "none"):
        if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous():
            raise ValueError("quantize expects a contiguous 2-D bfloat16 tensor")
        rows, cols = x.shape
        codes = torch.empty((rows, code_cols(f, cols)), dtype=torch.uint8, device=x.device)
        scales = torch.empty(scale_shape(f, rows, cols), dtype=torch.uint8, device=x.device)
        _check(mx_quantize_ex(f, BLOCK[f], MX_ROUND_RNE, SCALE_RULES[scale_rule], ROTATIONS[rotation], rows,
                              cols, _ptr(x), _ptr(codes), _ptr(scales), _stream(torch, x.device, x), lay),
               "mx_quantize_ex")
        return QTensor(f, rows, cols, codes, scales, None, lay)
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("quantize expects a contiguous 2-D bfloat16 tensor")
    rows, cols = x.shape
    dev = x.device
    codes = torch.empty((rows, code_cols(f, cols)), dtype=torch.uint8, device=dev)
    scales = torch.empty(scale_shape(f, rows, cols), dtype=torch.uint8, device=dev)
    ts = ws = None
    wsb = 0
    if f == MX_FMT_NVFP4:
        ts = torch.empty(1, dtype=torch.float32, device=dev)
        wsb = mx_quantize_workspace_bytes(f, rows, cols)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    if lay == MX_LAYOUT_ROWS:
        _check(mx_quantize(f, BLOCK[f], MX_ROUND_RNE, rows, cols, _ptr(x), _ptr(codes), _ptr(scales),
                           _ptr(ts), _ptr(ws), wsb, _stream(torch, dev, x)), "mx_quantize")
    else:
        _check(mx_quantize_layout(f, BLOCK[f], MX_ROUND_RNE, rows, cols, _ptr(x), _ptr(codes),
                                  _ptr(scales), _ptr(ts), _ptr(ws), wsb, _stream(torch, dev, x), lay),
               "mx_quantize_layout")
    return QTensor(f, rows, cols, codes, scales, ts, lay)


def dequantize(q, out_dtype=None):
    """Expand a QTensor (row layout) to float32 (default) or bfloat16."""
    import torch
    _check_qtensor(q, "dequantize")
    if q.layout != MX_LAYOUT_ROWS:
        raise ValueError("dequantize takes a tensor in the row layout")
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be torch.float32 or torch.bfloat16")
    od = MX_OUT_F32 if out_dtype == torch.float32 else MX_OUT_BF16
    y = torch.empty((q.rows, q.cols), dtype=out_dtype, device=q.codes.device)
    _check(mx_dequantize(q.fmt, q.block, MX_ROUND_RNE, q.rows, q.cols, _ptr(q.codes),
                         _ptr(q.scales), _ptr(q.tensor_scale), od, _ptr(y),
                         _stream(torch, q.codes.device, q.codes, q.scales, q.tensor_scale)), "mx_dequantize")
    return y


def pack(q):
    """A QTensor (MXFP4, MXFP8, E5M2, E3M2 or NVFP4) re-laid into the K-panel
    layout (mx_pack), for use as a gemm() operand."""
    import torch
    if q.layout != MX_LAYOUT_ROWS:
        raise ValueError("pack() takes a tensor in the row layout")
    _check_qtensor(q, "pack")
    codes = torch.empty_like(q.codes)
    scales = torch.empty_like(q.scales)
    _check(mx_pack(q.fmt, q.block, q.rows, q.cols, _ptr(q.codes), _ptr(q.scales), _ptr(codes),
                   _ptr(scales), _stream(torch, q.codes.device, q.codes, q.scales)), "mx_pack")
    return QTensor(q.fmt, q.rows, q.cols, codes, scales, q.tensor_scale, MX_LAYOUT_KPANEL)


def gemm(a, b, out_dtype=None, out=None, workspace=None):
    """C = A * B^T. a: QTensor (any quantized format, M x K; b of the same format) or a bf16 [M][K]
    tensor (with an MXFP4 b: W4A16); b: QTensor stored N x K (MXFP4: row or
    K-panel layout)."""
    import torch
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be torch.float32 or torch.bfloat16")
    od = MX_OUT_F32 if out_dtype == torch.float32 else MX_OUT_BF16
    _check_qtensor(b, "gemm operand b")
    if isinstance(a, QTensor):
        _check_qtensor(a, "gemm operand a")
        fa, M, K = a.fmt, a.rows, a.cols
        pa, psa, pta = _ptr(a.codes), _ptr(a.scales), _ptr(a.tensor_scale)
        dev = a.codes.device
    else:
        if a.dtype != torch.bfloat16 or a.dim() != 2 or not a.is_contiguous():
            raise ValueError("bf16 activations must be a contiguous 2-D bfloat16 tensor")
        fa, (M, K) = MX_FMT_BF16, a.shape
        pa, psa, pta = _ptr(a), None, None
        dev = a.device
    N = b.rows
    if b.cols != K:
        raise ValueError(f"K mismatch: A has {K}, B has {b.cols}")
    if out is not None:
        if (out.dtype != out_dtype or out.dim() != 2 or tuple(out.shape) != (M, N)
                or out.stride(1) != 1):
            raise ValueError(f"out must be a [{M}][{N}] {out_dtype} tensor with unit column stride")
    c = out if out is not None else torch.empty((M, N), dtype=out_dtype, device=dev)
    wsb = mx_gemm_workspace_bytes(fa, b.fmt, M, N, K)
    if wsb and workspace is None:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    if workspace is not None:
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        wsb = workspace.numel() * workspace.element_size()  # the C call checks it is enough
    la = a.layout if isinstance(a, QTensor) else MX_LAYOUT_ROWS
    a_parts = (a.codes, a.scales, a.tensor_scale) if isinstance(a, QTensor) else (a,)
    stream = _stream(torch, dev, *a_parts, b.codes, b.scales, b.tensor_scale, c, workspace)
    if la != MX_LAYOUT_ROWS or b.layout != MX_LAYOUT_ROWS:
        _check(mx_gemm_ex(fa, b.fmt, b.block, MX_ROUND_RNE, M, N, K, pa, psa, pta, _ptr(b.codes),
                          _ptr(b.scales), _ptr(b.tensor_scale), od, _ptr(c), c.stride(0),
                          _ptr(workspace), wsb, stream, la, b.layout), "mx_gemm_ex")
        return c
    _check(mx_gemm(fa, b.fmt, b.block, MX_ROUND_RNE, M, N, K, pa, psa, pta, _ptr(b.codes),
                   _ptr(b.scales), _ptr(b.tensor_scale), od, _ptr(c), c.stride(0),
                   _ptr(workspace), wsb, stream), "mx_gemm")
    return c
