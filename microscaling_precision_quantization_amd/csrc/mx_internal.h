// Internal launch interface of libmx (not part of the public ABI).
#pragma once
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <tuple>
#include <utility>

namespace mx {

// Launches kernel<<<grid, block, shmem, stream>>>(args...) through
// hipLaunchKernel and returns the status of that launch itself. (A status
// read back with hipGetLastError afterwards could instead be an error that
// an earlier HIP call of the caller left pending on this thread, and reading
// it would also clear the caller's error.) Arguments are converted to the
// kernel's parameter types first.
template <typename... P, typename... A, size_t... I>
inline hipError_t launch_impl(void (*kernel)(P...), dim3 grid, dim3 block, size_t shmem,
                              hipStream_t stream, std::index_sequence<I...>, A&&... args) {
  std::tuple<P...> params(static_cast<P>(std::forward<A>(args))...);
  void* argv[] = {(void*)&std::get<I>(params)...};
  return hipLaunchKernel((const void*)kernel, grid, block, argv, shmem, stream);
}

template <typename... P, typename... A>
inline hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, size_t shmem,
                                hipStream_t stream, A&&... args) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  return launch_impl(kernel, grid, block, shmem, stream, std::index_sequence_for<P...>{},
                     std::forward<A>(args)...);
}

// Returns from the enclosing launcher with the first failed launch's status.
#define MX_TRY(launch)                     \
  do {                                     \
    const hipError_t mx_e_ = (launch);     \
    if (mx_e_ != hipSuccess) return mx_e_; \
  } while (0)

// Format ids, kept equal to the public mx_format values.
enum : int { kBF16 = 0, kMXFP4 = 1, kMXFP8 = 2, kNVFP4 = 3, kMXFP8E5M2 = 4, kMXFP6 = 5, kMXFP4MBS = 6,
             kMXFP4MBS16 = 7 };
enum : int { kOutF32 = 0, kOutBF16 = 1 };

// ---- quantize.hip
// oas: MXFP4's overflow-aware scale rule; rot: 32-point Walsh-Hadamard rotation first.
// panel: codes and scales in the K-panel layout (panels of 256 elements for
// MXFP4, of 64 for MXFP8, E5M2 and E3M2; cols a multiple of that).
hipError_t quant_mx(int fmt, int64_t rows, int64_t cols, const void* x, void* codes,
                    void* scales, hipStream_t s, bool oas = false,
                    bool rot = false, bool panel = false);
// MXFP4 with static macro-block scaling over base blocks of `base` (16 or
// 32) elements: scales holds the E8M0 plane [rows][cols/base] followed by the
// macro mantissa plane [rows][cols/128].
hipError_t quant_mbs(int64_t rows, int64_t cols, const void* x, void* codes, void* scales,
                     hipStream_t s, int base);
size_t quant_nvfp4_workspace(int64_t rows, int64_t cols);
// panel: codes and scales in the K-panel layout with 64-element panels.
hipError_t quant_nvfp4(int64_t rows, int64_t cols, const void* x, void* codes, void* scales,
                       float* tensor_scale, void* workspace, hipStream_t s, bool panel = false);

// ---- dequantize.hip
hipError_t dequant(int fmt, int64_t rows, int64_t cols, const void* codes, const void* scales,
                   const float* tensor_scale, int out_dtype, void* y, hipStream_t s);

// ---- gemm_mx.hip (MXFP4 x MXFP4 on the FP4 scaled MFMA: the 256 x 256-tile
// kernel when it fits, else 128 x 128 tiles)
hipError_t gemm_mx(int64_t M, int64_t N, int64_t K, const void* a, const void* sa, const void* b,
                   const void* sb, int out_dtype, void* c, int64_t ldc, hipStream_t s);

// ---- gemm_mx.hip, MXFP4-MBS x MXFP4-MBS (128 x 128 tiles, any K % 128 = 0);
// sa / sb are the two-plane scale buffers.
hipError_t gemm_mbs_small(int64_t M, int64_t N, int64_t K, const void* a, const void* sa,
                          const void* b, const void* sb, int out_dtype, void* c, int64_t ldc,
                          hipStream_t s, int base);

// ---- gemm_mbs.hip (MXFP4-MBS x MXFP4-MBS over base blocks of `base` = 32 or
// 16 elements; 256 x 256 tiles when they fit, else gemm_mbs_small)
bool gemm_mbs_fits(int64_t M, int64_t N, int64_t K);
hipError_t gemm_mbs(int64_t M, int64_t N, int64_t K, const void* a, const void* sa,
                    const void* b, const void* sb, int out_dtype, void* c, int64_t ldc,
                    hipStream_t s, int base);

// ---- gemm_mxfp4.hip (MXFP4 x MXFP4, 256 x 256 tiles, register-staged
// pipeline); panel_a / panel_b: that operand in the K-panel layout (its
// rows * K / 2 below 2^31)
bool gemm_mxfp4_fits(int64_t M, int64_t N, int64_t K);
hipError_t gemm_mxfp4(int64_t M, int64_t N, int64_t K, const void* a, const void* sa,
                      const void* b, const void* sb, int out_dtype, void* c, int64_t ldc,
                      hipStream_t s, bool panel_a, bool panel_b);

// ---- pack.hip (codes and scales into the K-panel layout): `panels` panels,
// wb code bytes (a multiple of 16) and sb scale bytes (8, 4 or 2) per row
// and panel.
hipError_t pack_kpanel(int64_t rows, int64_t panels, int wb, int sb, const void* codes,
                       const void* scales, void* packed_codes, void* packed_scales, hipStream_t s);

// ---- gemm_bf16x.hip (MXFP8 x MXFP8 and NVFP4 x NVFP4, expanded exactly to bf16)
hipError_t gemm_bf16x(int fmt, int64_t M, int64_t N, int64_t K, const void* a, const void* sa,
                      const float* ta, const void* b, const void* sb, const float* tb,
                      int out_dtype, void* c, int64_t ldc, hipStream_t s);

// ---- gemm_bf16x_large.hip (256 x 256 or 224 x 256 tiles; MXFP8 / NVFP4 on the bf16 MFMA)
bool gemm_bf16x_large_fits(int fmt, int64_t M, int64_t N, int64_t K);
// panel: both operands in the K-panel layout (64-element panels).
hipError_t gemm_bf16x_large(int fmt, int64_t M, int64_t N, int64_t K, const void* a, const void* sa,
                            const float* ta, const void* b, const void* sb, const float* tb,
                            int out_dtype, void* c, int64_t ldc, hipStream_t s, bool panel = false);

// ---- gemm_w4a16.hip: the library's own scratch for mx_gemm_noalloc (the
// W4A16 split-K partials), a file-scope device array of this many bytes per
// GPU; noalloc_scratch returns its address on the current device (looked up
// once per device).
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
constexpr int kMaxDevices = 64;
hipError_t noalloc_scratch(void** ptr);

// ---- gemm_w4a16.hip (bf16 activations x MXFP4 weights)
size_t gemm_w4a16_workspace(int64_t M, int64_t N, int64_t K);
hipError_t gemm_w4a16(int64_t M, int64_t N, int64_t K, const void* a, const void* b,
                      const void* sb, int out_dtype, void* c, int64_t ldc, void* workspace,
                      hipStream_t s);

}  // namespace mx
