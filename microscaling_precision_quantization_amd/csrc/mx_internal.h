// Internal launch interface of libmx (not part of the public ABI).
#pragma once
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace mx {

// Format ids, kept equal to the public mx_format values.
enum : int { kBF16 = 0, kMXFP4 = 1, kMXFP8 = 2, kNVFP4 = 3, kMXFP8E5M2 = 4, kMXFP6 = 5, kMXFP4MBS = 6 };
enum : int { kOutF32 = 0, kOutBF16 = 1 };

// ---- quantize.hip
// oas: MXFP4's overflow-aware scale rule; rot: 32-point Walsh-Hadamard rotation first.
// panel: MXFP4 codes and scales in the K-panel layout (cols % 256 = 0).
hipError_t quant_mx(int fmt, int64_t rows, int64_t cols, const void* x, void* codes,
                    void* scales, hipStream_t s, bool oas = false,
                    bool rot = false, bool panel = false);
// MXFP4 with static macro-block scaling: scales holds the E8M0 plane
// [rows][cols/32] followed by the macro mantissa plane [rows][cols/128].
hipError_t quant_mbs(int64_t rows, int64_t cols, const void* x, void* codes, void* scales,
                     hipStream_t s);
size_t quant_nvfp4_workspace(int64_t rows, int64_t cols);
hipError_t quant_nvfp4(int64_t rows, int64_t cols, const void* x, void* codes, void* scales,
                       float* tensor_scale, void* workspace, hipStream_t s);

// ---- dequantize.hip
hipError_t dequant(int fmt, int64_t rows, int64_t cols, const void* codes, const void* scales,
                   const float* tensor_scale, int out_dtype, void* y, hipStream_t s);

// ---- gemm_mx.hip (MXFP4 x MXFP4 on the FP4 scaled MFMA)
hipError_t gemm_mx(int fmt, int64_t M, int64_t N, int64_t K, const void* a, const void* sa,
                   const void* b, const void* sb, int out_dtype, void* c, int64_t ldc,
                   hipStream_t s);

// ---- gemm_mx.hip, MXFP4-MBS x MXFP4-MBS (128 x 128 tiles, any K % 128 = 0);
// sa / sb are the two-plane scale buffers.
hipError_t gemm_mbs_small(int64_t M, int64_t N, int64_t K, const void* a, const void* sa,
                          const void* b, const void* sb, int out_dtype, void* c, int64_t ldc,
                          hipStream_t s);

// ---- gemm_mbs.hip (MXFP4-MBS x MXFP4-MBS; 256 x 128 tiles when they fit,
// else gemm_mbs_small)
bool gemm_mbs_fits(int64_t M, int64_t N, int64_t K);
hipError_t gemm_mbs(int64_t M, int64_t N, int64_t K, const void* a, const void* sa,
                    const void* b, const void* sb, int out_dtype, void* c, int64_t ldc,
                    hipStream_t s);

// ---- gemm_mxfp4.hip (MXFP4 x MXFP4, 256 x 256 tiles, register-staged
// pipeline); panel_a / panel_b: that operand in the K-panel layout (its
// rows * K / 2 below 2^31)
bool gemm_mxfp4_fits(int64_t M, int64_t N, int64_t K);
hipError_t gemm_mxfp4(int64_t M, int64_t N, int64_t K, const void* a, const void* sa,
                      const void* b, const void* sb, int out_dtype, void* c, int64_t ldc,
                      hipStream_t s, bool panel_a, bool panel_b);

// ---- pack.hip (MXFP4 codes and scales into the K-panel layout)
hipError_t pack_mxfp4(int64_t rows, int64_t cols, const void* codes, const void* scales,
                      void* packed_codes, void* packed_scales, hipStream_t s);

// ---- gemm_bf16x.hip (MXFP8 x MXFP8 and NVFP4 x NVFP4, expanded exactly to bf16)
hipError_t gemm_bf16x(int fmt, int64_t M, int64_t N, int64_t K, const void* a, const void* sa,
                      const float* ta, const void* b, const void* sb, const float* tb,
                      int out_dtype, void* c, int64_t ldc, hipStream_t s);

// ---- gemm_bf16x_large.hip (256 x 256 tiles; MXFP8 / NVFP4 on the bf16 MFMA)
bool gemm_bf16x_large_fits(int fmt, int64_t M, int64_t N, int64_t K);
hipError_t gemm_bf16x_large(int fmt, int64_t M, int64_t N, int64_t K, const void* a, const void* sa,
                            const float* ta, const void* b, const void* sb, const float* tb,
                            int out_dtype, void* c, int64_t ldc, hipStream_t s);

// ---- gemm_w4a16.hip (bf16 activations x MXFP4 weights)
size_t gemm_w4a16_workspace(int64_t M, int64_t N, int64_t K);
hipError_t gemm_w4a16(int64_t M, int64_t N, int64_t K, const void* a, const void* b,
                      const void* sb, int out_dtype, void* c, int64_t ldc, void* workspace,
                      hipStream_t s);

}  // namespace mx
