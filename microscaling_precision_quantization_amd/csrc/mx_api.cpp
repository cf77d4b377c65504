// C ABI of libmx: argument checks, dispatch to the gfx950 kernels, and error
// mapping. Every check runs before anything is enqueued; nothing here
// allocates, synchronizes or prints.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "../../include/mx.h"
#include "mx_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

bool is_quant_fmt(int f) {
  return f == MX_FMT_MXFP4 || f == MX_FMT_MXFP8 || f == MX_FMT_NVFP4 || f == MX_FMT_MXFP8_E5M2 ||
         f == MX_FMT_MXFP6_E3M2 || f == MX_FMT_MXFP4_MBS || f == MX_FMT_MXFP4_MBS16;
}
bool is_mbs(int f) { return f == MX_FMT_MXFP4_MBS || f == MX_FMT_MXFP4_MBS16; }
int block_of(int f) { return (f == MX_FMT_NVFP4 || f == MX_FMT_MXFP4_MBS16) ? 16 : 32; }
// cols (and K) must be a multiple of this: the block, or the 128-element macro
// block of MXFP4-MBS and MXFP4-MBS16.
int granule_of(int f) { return is_mbs(f) ? 128 : block_of(f); }

// Elements per tensor stay below 2^40 and every GEMM extent below 2^30 so that
// the kernels' index arithmetic (int64 offsets, int extents) cannot overflow.
constexpr int64_t kMaxElems = (int64_t)1 << 40;
constexpr int64_t kMaxExtent = (int64_t)1 << 30;
constexpr int64_t kW4A16MaxK = 65536;

mx_status hip_status(hipError_t e) {
  if (e == hipSuccess) return MX_OK;
  g_last_hip_error = (int)e;
  return MX_ERR_HIP;
}

// Elements per K panel of a K-panel tensor: 256 for MXFP4 (one step of its
// GEMM), 64 for MXFP8, E5M2, E3M2 and NVFP4 (one stage of theirs).
int panel_width(int fmt) { return fmt == MX_FMT_MXFP4 ? 256 : 64; }

// Code bytes of a row of cols elements.
int64_t code_bytes(int fmt, int64_t cols) {
  if (fmt == MX_FMT_MXFP8 || fmt == MX_FMT_MXFP8_E5M2) return cols;
  if (fmt == MX_FMT_MXFP6_E3M2) return cols * 3 / 4;
  return cols / 2;
}

// Formats with a K-panel layout.
bool has_panel(int fmt) {
  return fmt == MX_FMT_MXFP4 || fmt == MX_FMT_MXFP8 || fmt == MX_FMT_MXFP8_E5M2 ||
         fmt == MX_FMT_MXFP6_E3M2 || fmt == MX_FMT_NVFP4;
}

// A K-panel tensor: whole panels, at most 65535 of them (a grid dimension of
// the panel quantizer), and 32-bit byte offsets.
bool panel_shape_ok(int fmt, int64_t rows, int64_t cols) {
  const int w = panel_width(fmt);
  return cols % w == 0 && cols / w <= 65535 && rows < ((int64_t)1 << 31) / code_bytes(fmt, cols);
}

// Common checks for a [rows][cols] quantized tensor.
mx_status check_tensor(int fmt, int block, int rnd, int64_t rows, int64_t cols) {
  if (!is_quant_fmt(fmt) || block != block_of(fmt)) return MX_ERR_UNSUPPORTED;
  if (rnd != MX_ROUND_RNE) return MX_ERR_UNSUPPORTED;
  if (rows <= 0 || cols <= 0 || cols % granule_of(fmt) != 0) return MX_ERR_INVALID_ARG;
  if (rows > kMaxElems / cols) return MX_ERR_INVALID_ARG;
  return MX_OK;
}

}  // namespace

extern "C" {

size_t mx_quantize_workspace_bytes(mx_format fmt, int64_t rows, int64_t cols) {
  if (fmt != MX_FMT_NVFP4 || rows <= 0 || cols <= 0) return 0;
  return mx::quant_nvfp4_workspace(rows, cols);
}

mx_status mx_quantize_layout(mx_format fmt, int block, mx_round rnd, int64_t rows, int64_t cols,
                             const void* x, void* codes, void* scales, float* tensor_scale,
                             void* workspace, size_t workspace_bytes, void* stream,
                             mx_layout layout) {
  mx_status st = check_tensor(fmt, block, rnd, rows, cols);
  if (st != MX_OK) return st;
  if (layout != MX_LAYOUT_ROWS && layout != MX_LAYOUT_KPANEL) return MX_ERR_UNSUPPORTED;
  const bool panel = layout == MX_LAYOUT_KPANEL;
  if (panel && !has_panel(fmt)) return MX_ERR_UNSUPPORTED;
  if (panel && !panel_shape_ok(fmt, rows, cols)) return MX_ERR_INVALID_ARG;
  if (!x || !codes || !scales) return MX_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return MX_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (fmt == MX_FMT_NVFP4) {
    if (!tensor_scale || !aligned4(tensor_scale)) return MX_ERR_INVALID_ARG;
    if (!workspace || !aligned16(workspace)) return MX_ERR_INVALID_ARG;
    if (workspace_bytes < mx::quant_nvfp4_workspace(rows, cols)) return MX_ERR_INVALID_ARG;
    return hip_status(mx::quant_nvfp4(rows, cols, x, codes, scales, tensor_scale, workspace, s, panel));
  }
  if (tensor_scale) return MX_ERR_INVALID_ARG;
  if (is_mbs(fmt)) return hip_status(mx::quant_mbs(rows, cols, x, codes, scales, s, block));
  return hip_status(mx::quant_mx(fmt, rows, cols, x, codes, scales, s, false, false, panel));
}

mx_status mx_quantize(mx_format fmt, int block, mx_round rnd, int64_t rows, int64_t cols,
                      const void* x, void* codes, void* scales, float* tensor_scale,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return mx_quantize_layout(fmt, block, rnd, rows, cols, x, codes, scales, tensor_scale, workspace,
                            workspace_bytes, stream, MX_LAYOUT_ROWS);
}

mx_status mx_quantize_ex(mx_format fmt, int block, mx_round rnd, mx_scale_rule rule,
                         mx_rotation rot, int64_t rows, int64_t cols, const void* x,
                         void* codes, void* scales, void* stream, mx_layout layout) {
  mx_status st = check_tensor(fmt, block, rnd, rows, cols);
  if (st != MX_OK) return st;
  if (layout != MX_LAYOUT_ROWS && layout != MX_LAYOUT_KPANEL) return MX_ERR_UNSUPPORTED;
  const bool panel = layout == MX_LAYOUT_KPANEL;
  if (fmt != MX_FMT_MXFP4 && fmt != MX_FMT_MXFP8) return MX_ERR_UNSUPPORTED;
  if (panel && !panel_shape_ok(fmt, rows, cols)) return MX_ERR_INVALID_ARG;
  if (rule != MX_SCALE_CEIL && !(rule == MX_SCALE_OAS && fmt == MX_FMT_MXFP4))
    return MX_ERR_UNSUPPORTED;
  if (rot != MX_ROTATE_NONE && rot != MX_ROTATE_WHT32) return MX_ERR_UNSUPPORTED;
  if (!x || !codes || !scales) return MX_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return MX_ERR_INVALID_ARG;
  return hip_status(mx::quant_mx(fmt, rows, cols, x, codes, scales, (hipStream_t)stream,
                                 rule == MX_SCALE_OAS, rot == MX_ROTATE_WHT32, panel));
}

mx_status mx_dequantize(mx_format fmt, int block, mx_round rnd, int64_t rows, int64_t cols,
                        const void* codes, const void* scales, const float* tensor_scale,
                        mx_dtype out_dtype, void* y, void* stream) {
  mx_status st = check_tensor(fmt, block, rnd, rows, cols);
  if (st != MX_OK) return st;
  if (out_dtype != MX_OUT_F32 && out_dtype != MX_OUT_BF16) return MX_ERR_UNSUPPORTED;
  if (!codes || !scales || !y) return MX_ERR_INVALID_ARG;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(y)) return MX_ERR_INVALID_ARG;
  if (fmt == MX_FMT_NVFP4) {
    if (!tensor_scale || !aligned4(tensor_scale)) return MX_ERR_INVALID_ARG;
  } else if (tensor_scale) {
    return MX_ERR_INVALID_ARG;
  }
  return hip_status(mx::dequant(fmt, rows, cols, codes, scales, tensor_scale, out_dtype, y,
                                (hipStream_t)stream));
}

size_t mx_gemm_workspace_bytes(mx_format fmt_a, mx_format fmt_b, int64_t M, int64_t N, int64_t K) {
  if (fmt_a == MX_FMT_BF16 && fmt_b == MX_FMT_MXFP4 && M > 0 && N > 0 && K > 0 && K % 32 == 0 &&
      M <= kMaxExtent && N <= kMaxExtent && K <= kW4A16MaxK)
    return mx::gemm_w4a16_workspace(M, N, K);
  return 0;
}

}  // extern "C"

namespace {

// mx_gemm and mx_gemm_ex; panel_a / panel_b: that operand in the K-panel layout.
mx_status gemm_impl(mx_format fmt_a, mx_format fmt_b, int block, mx_round rnd, int64_t M, int64_t N,
                    int64_t K, const void* a, const void* a_scales, const float* a_ts,
                    const void* b, const void* b_scales, const float* b_ts, mx_dtype out_dtype,
                    void* c, int64_t ldc, void* workspace, size_t workspace_bytes, void* stream,
                    bool panel_a, bool panel_b) {
  const bool w4a4 = fmt_a == MX_FMT_MXFP4 && fmt_b == MX_FMT_MXFP4 && block == 32;
  const bool w8a8 = fmt_a == MX_FMT_MXFP8 && fmt_b == MX_FMT_MXFP8 && block == 32;
  const bool nv = fmt_a == MX_FMT_NVFP4 && fmt_b == MX_FMT_NVFP4 && block == 16;
  const bool w4a16 = fmt_a == MX_FMT_BF16 && fmt_b == MX_FMT_MXFP4 && block == 32;
  const bool alt = fmt_a == fmt_b && block == 32 &&
                   (fmt_a == MX_FMT_MXFP8_E5M2 || fmt_a == MX_FMT_MXFP6_E3M2);
  const bool mbs = (fmt_a == MX_FMT_MXFP4_MBS && fmt_b == MX_FMT_MXFP4_MBS && block == 32) ||
                   (fmt_a == MX_FMT_MXFP4_MBS16 && fmt_b == MX_FMT_MXFP4_MBS16 && block == 16);
  if (!(w4a4 || w8a8 || nv || w4a16 || alt || mbs)) return MX_ERR_UNSUPPORTED;
  // K-panel operands: the MXFP4 pair (either operand or both), or both
  // operands of the pairs on the 16-bit MFMAs.
  if ((panel_a || panel_b) && !w4a4 && !((w8a8 || nv || alt) && panel_a && panel_b))
    return MX_ERR_UNSUPPORTED;
  if (rnd != MX_ROUND_RNE) return MX_ERR_UNSUPPORTED;
  if (out_dtype != MX_OUT_F32 && out_dtype != MX_OUT_BF16) return MX_ERR_UNSUPPORTED;
  if (M <= 0 || N <= 0 || K <= 0 || M > kMaxExtent || N > kMaxExtent || K > kMaxExtent)
    return MX_ERR_INVALID_ARG;
  // K is a whole number of 32-element groups for every path (NVFP4 included:
  // its 16-blocks are staged in pairs).
  if (K % 32 != 0 || (mbs && K % 128 != 0)) return MX_ERR_INVALID_ARG;
  if (ldc < N) return MX_ERR_INVALID_ARG;
  // Row tiles run along gridDim.y (at most 65535): 128 rows per tile for the
  // W4A4/W8A8 kernels, 16 for W4A16.
  if (M > (w4a16 ? 16 : 128) * (int64_t)65535) return MX_ERR_INVALID_ARG;
  // W4A16: at most 32 K-splits of 2048, so that each output's fp32 chain (33
  // roundings in a split, then the fixed-order sum of the splits) stays within
  // 64 steps, the accumulation bound of mx.h.
  if (w4a16 && K > kW4A16MaxK) return MX_ERR_INVALID_ARG;
  if (!a || !b || !b_scales || !c) return MX_ERR_INVALID_ARG;
  if (!aligned16(a) || !aligned16(b) || !aligned16(b_scales) || !aligned16(c))
    return MX_ERR_INVALID_ARG;
  if (w4a16) {
    if (a_scales || a_ts || b_ts) return MX_ERR_INVALID_ARG;
  } else {
    if (!a_scales || !aligned16(a_scales)) return MX_ERR_INVALID_ARG;
  }
  if (nv) {
    if (!a_ts || !b_ts || !aligned4(a_ts) || !aligned4(b_ts)) return MX_ERR_INVALID_ARG;
  } else if (a_ts || b_ts) {
    return MX_ERR_INVALID_ARG;
  }
  const size_t need = mx_gemm_workspace_bytes(fmt_a, fmt_b, M, N, K);
  if (need > 0 && (!workspace || !aligned16(workspace) || workspace_bytes < need))
    return MX_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (panel_a || panel_b) {
    if ((panel_a && !panel_shape_ok(fmt_a, M, K)) || (panel_b && !panel_shape_ok(fmt_b, N, K)))
      return MX_ERR_INVALID_ARG;
    if (!w4a4) {
      // The large-tile kernel of the 16-bit MFMAs reads K-panel operands.
      if (!mx::gemm_bf16x_large_fits(fmt_a, M, N, K)) return MX_ERR_INVALID_ARG;
      return hip_status(mx::gemm_bf16x_large(fmt_a, M, N, K, a, a_scales, a_ts, b, b_scales, b_ts,
                                             out_dtype, c, ldc, s, true));
    }
    // Only the 256 x 256-tile kernel reads K-panel MXFP4 operands.
    if (!mx::gemm_mxfp4_fits(M, N, K)) return MX_ERR_INVALID_ARG;
    return hip_status(mx::gemm_mxfp4(M, N, K, a, a_scales, b, b_scales, out_dtype, c, ldc, s,
                                     panel_a, panel_b));
  }
  if (w4a4)
    return hip_status(mx::gemm_mx(M, N, K, a, a_scales, b, b_scales, out_dtype, c, ldc, s));
  if (mbs)
    return hip_status(mx::gemm_mbs(M, N, K, a, a_scales, b, b_scales, out_dtype, c, ldc, s, block));
  if (w8a8 || nv)
    return hip_status(mx::gemm_bf16x(fmt_a, M, N, K, a, a_scales, a_ts, b, b_scales, b_ts,
                                     out_dtype, c, ldc, s));
  if (alt) {
    if (!mx::gemm_bf16x_large_fits(fmt_a, M, N, K)) return MX_ERR_INVALID_ARG;
    return hip_status(mx::gemm_bf16x_large(fmt_a, M, N, K, a, a_scales, nullptr, b, b_scales,
                                           nullptr, out_dtype, c, ldc, s));
  }
  return hip_status(mx::gemm_w4a16(M, N, K, a, b, b_scales, out_dtype, c, ldc, workspace, s));
}

// [p, p + n) and [q, q + m) share a byte.
bool overlap(const void* p, size_t n, const void* q, size_t m) {
  const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
  return a < b + m && b < a + n;
}

}  // namespace

extern "C" {

mx_status mx_gemm(mx_format fmt_a, mx_format fmt_b, int block, mx_round rnd, int64_t M, int64_t N,
                  int64_t K, const void* a, const void* a_scales, const float* a_ts,
                  const void* b, const void* b_scales, const float* b_ts, mx_dtype out_dtype,
                  void* c, int64_t ldc, void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_impl(fmt_a, fmt_b, block, rnd, M, N, K, a, a_scales, a_ts, b, b_scales, b_ts,
                   out_dtype, c, ldc, workspace, workspace_bytes, stream, false, false);
}

mx_status mx_gemm_ex(mx_format fmt_a, mx_format fmt_b, int block, mx_round rnd, int64_t M,
                     int64_t N, int64_t K, const void* a, const void* a_scales, const float* a_ts,
                     const void* b, const void* b_scales, const float* b_ts, mx_dtype out_dtype,
                     void* c, int64_t ldc, void* workspace, size_t workspace_bytes, void* stream,
                     mx_layout a_layout, mx_layout b_layout) {
  if (a_layout != MX_LAYOUT_ROWS && a_layout != MX_LAYOUT_KPANEL) return MX_ERR_UNSUPPORTED;
  if (b_layout != MX_LAYOUT_ROWS && b_layout != MX_LAYOUT_KPANEL) return MX_ERR_UNSUPPORTED;
  return gemm_impl(fmt_a, fmt_b, block, rnd, M, N, K, a, a_scales, a_ts, b, b_scales, b_ts,
                   out_dtype, c, ldc, workspace, workspace_bytes, stream,
                   a_layout == MX_LAYOUT_KPANEL, b_layout == MX_LAYOUT_KPANEL);
}

mx_status mx_gemm_noalloc(mx_format fmt_a, mx_format fmt_b, int block, mx_round rnd, int64_t M,
                          int64_t N, int64_t K, const void* a, const void* a_scales,
                          const float* a_ts, const void* b, const void* b_scales,
                          const float* b_ts, mx_dtype out_dtype, void* c, int64_t ldc,
                          void* stream) {
  const size_t need = mx_gemm_workspace_bytes(fmt_a, fmt_b, M, N, K);
  void* ws = nullptr;
  if (need > 0) {
    if (need > mx::kNoAllocScratchBytes) return MX_ERR_INVALID_ARG;
    const hipError_t e = mx::noalloc_scratch(&ws);
    if (e != hipSuccess) return hip_status(e);
  }
  return gemm_impl(fmt_a, fmt_b, block, rnd, M, N, K, a, a_scales, a_ts, b, b_scales, b_ts,
                   out_dtype, c, ldc, ws, need, stream, false, false);
}

mx_status mx_pack(mx_format fmt, int block, int64_t rows, int64_t cols, const void* codes,
                  const void* scales, void* packed_codes, void* packed_scales, void* stream) {
  if (!has_panel(fmt) || block != block_of(fmt)) return MX_ERR_UNSUPPORTED;
  if (rows <= 0 || cols <= 0 || !panel_shape_ok(fmt, rows, cols)) return MX_ERR_INVALID_ARG;
  if (!codes || !scales || !packed_codes || !packed_scales) return MX_ERR_INVALID_ARG;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(packed_codes) || !aligned16(packed_scales))
    return MX_ERR_INVALID_ARG;
  const size_t cb = (size_t)rows * (size_t)code_bytes(fmt, cols),
               sb = (size_t)rows * (size_t)(cols / block);
  if (overlap(codes, cb, packed_codes, cb) || overlap(codes, cb, packed_scales, sb) ||
      overlap(scales, sb, packed_codes, cb) || overlap(scales, sb, packed_scales, sb))
    return MX_ERR_INVALID_ARG;
  const int w = panel_width(fmt);
  return hip_status(mx::pack_kpanel(rows, cols / w, (int)code_bytes(fmt, w), w / block, codes, scales,
                                    packed_codes, packed_scales, (hipStream_t)stream));
}

int mx_last_hip_error(void) { return g_last_hip_error; }

const char* mx_status_string(mx_status s) {
  switch (s) {
    case MX_OK: return "MX_OK";
    case MX_ERR_INVALID_ARG: return "MX_ERR_INVALID_ARG";
    case MX_ERR_UNSUPPORTED: return "MX_ERR_UNSUPPORTED";
    case MX_ERR_HIP: return "MX_ERR_HIP";
  }
  return "MX_ERR_UNKNOWN";
}

}  // extern "C"
